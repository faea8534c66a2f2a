// Split planner, LSE-weighted combine and the paged-gather test kernel.
#include "device_common.h"
#include "launch.h"
#include "paged.h"

namespace attn {

namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// Split plan [MATE get_scheduler_metadata / get_mla_metadata; CANN
// flash_attn_metadata: a metadata pass that fixes the work split before the
// main call]. The rule is this library's own, integer only:
//   nblk_b = ceil(len_b / page) (0 if len_b <= 0)
//   bps    = max(min_blocks, ceil(sum nblk_b * upb / (num_cu * waves)))
//   ns_b   = min(max_splits, max(1, ceil(nblk_b / bps)))
//   pps_b  = ceil(nblk_b / ns_b), ns_b = ceil(nblk_b / pps_b)
// One workgroup; each thread owns a contiguous run of sequences.
__global__ void __launch_bounds__(kPlanThreads)
k_plan(const int32_t* __restrict__ lens, int batch, int page, int upb, int num_cu, int waves,
       int max_splits, int min_blocks, int32_t* __restrict__ plan) {
  __shared__ long red[kPlanThreads];
  __shared__ int scan[kPlanThreads];
  const int tid = threadIdx.x;
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(batch, tid * per), b1 = min(batch, b0 + per);
  long blocks = 0;
  for (int b = b0; b < b1; ++b) blocks += lens[b] > 0 ? cdiv(lens[b], page) : 0;
  red[tid] = blocks;
  __syncthreads();
  for (int w = kPlanThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const long total_units = red[0] * upb;
  const int bps = max(min_blocks, cdiv(total_units, (long)num_cu * waves));
  int mine = 0;
  for (int b = b0; b < b1; ++b) {
    const int nb = lens[b] > 0 ? cdiv(lens[b], page) : 0;
    if (nb) {
      int ns = min(max_splits, max(1, cdiv(nb, bps)));
      ns = cdiv(nb, cdiv(nb, ns));
      mine += ns;
    }
  }
  scan[tid] = mine;
  __syncthreads();
  // inclusive Hillis-Steele scan over the per-thread split counts
  for (int w = 1; w < kPlanThreads; w <<= 1) {
    const int v = tid >= w ? scan[tid - w] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int ptr = scan[tid] - mine;
  int32_t* split_ptr = plan + 2;
  int32_t* tri = plan + 3 + batch;
  for (int b = b0; b < b1; ++b) {
    split_ptr[b] = ptr;
    const int len = lens[b];
    const int nb = len > 0 ? cdiv(len, page) : 0;
    if (nb) {
      int ns = min(max_splits, max(1, cdiv(nb, bps)));
      const int pps = cdiv(nb, ns);
      ns = cdiv(nb, pps);
      for (int s = 0; s < ns; ++s) {
        tri[3 * (ptr + s)] = b;
        tri[3 * (ptr + s) + 1] = s * pps * page;
        tri[3 * (ptr + s) + 2] = min((s + 1) * pps * page, len);
      }
      ptr += ns;
    }
  }
  if (tid == kPlanThreads - 1) {
    split_ptr[batch] = scan[tid];
    plan[0] = scan[tid];
    plan[1] = bps;
  }
}

// LSE-weighted combine [MATE flash_attn_combine; CANN softmax_lse]. Each
// thread owns four output columns of one row; rows are (b, t, h) with the
// partial layout slot = b*max_splits + s, row t*hq + h. All of a row's split
// LSEs and partial outputs are loaded before any is used (unrolled over
// kMaxSplits >= max_splits, the instance chosen at launch; extra splits
// re-read the last one with weight 0), so a thread waits for one round trip
// to memory instead of one per split.
constexpr int kCombineThreads = 256;

template <int kMaxSplits>
__global__ void __launch_bounds__(kCombineThreads)
k_combine(CombineArgs a) {
  const int per_row = a.dv / 4;
  const int rows_per_block = kCombineThreads / per_row;
  const int lrow = threadIdx.x / per_row;
  const int col = (threadIdx.x % per_row) * 4;
  const long row = (long)blockIdx.x * rows_per_block + lrow;
  const int rows_per_b = a.sq * a.hq;
  if (lrow >= rows_per_block || row >= (long)a.batch * rows_per_b) return;
  const int b = (int)(row / rows_per_b);
  const int rr = (int)(row % rows_per_b);
  const int t = rr / a.hq, h = rr % a.hq;
  const int ns = a.plan[2 + b + 1] - a.plan[2 + b];
  const size_t slot0 = (size_t)b * a.max_splits;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = kNegInf;
  if (ns > 0) {
    float ls[kMaxSplits];
    f32x4 o[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      const size_t r = (slot0 + min(s, ns - 1)) * rows_per_b + rr;
      ls[s] = a.lse_part[r];
      o[s] = *reinterpret_cast<const f32x4*>(a.o_part + r * a.dv + col);
    }
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) mx = fmaxf(mx, ls[s]);
    if (mx != kNegInf) {
      float ref = mx;
      float extra = 0.f;
      if (a.sinks) {
        const float sg = a.sinks[h];
        ref = fmaxf(mx, sg);
        extra = __expf(sg - ref);
      }
      float wsum = 0.f, wsum_ref = 0.f;
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) {
        const float w = s < ns ? __expf(ls[s] - ref) : 0.f;
        wsum += w;
        wsum_ref += s < ns ? __expf(ls[s] - mx) : 0.f;
        acc += w * o[s];
      }
      acc *= 1.f / (wsum + extra);
      lse = mx + __logf(wsum_ref);
    }
  }
  const size_t orow = ((size_t)b * a.sq + t) * a.hq + h;
  if (a.out_bf16) {
    const u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16_t*>(a.out) + orow * a.dv + col) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow * a.dv + col) = acc;
  }
  if (a.lse && col == 0) a.lse[((size_t)b * a.hq + h) * a.sq + t] = lse;
}

// Copies logical rows [0, min(len_b, max_rows)) of sequence b out of a paged
// cache through paged_row_offset(), 16 bytes per thread.
__global__ void k_gather(const bf16_t* __restrict__ cache, const int32_t* __restrict__ bt,
                         int max_pages, const int32_t* __restrict__ lens, int b, int page,
                         int row_elems, int max_rows, bf16_t* __restrict__ dst) {
  const int n = min(lens[b], max_rows);
  const int chunks = row_elems / 8;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)n * chunks) return;
  const int j = (int)(i / chunks), c = (int)(i % chunks);
  const bf16_t* src = cache + paged_row_offset(bt, max_pages, b, j, page, 1, 0, row_elems);
  *reinterpret_cast<u32x4*>(dst + (size_t)j * row_elems + c * 8) =
      *reinterpret_cast<const u32x4*>(src + c * 8);
}

}  // namespace

hipError_t launch_plan(const int32_t* lens, int batch, int page, int upb, int num_cu, int waves,
                       int max_splits, int min_blocks, int32_t* plan, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, s, lens, batch, page, upb, num_cu,
                     waves, max_splits, min_blocks, plan);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int rows_per_block = kCombineThreads / (a.dv / 4);
  const long rows = (long)a.batch * a.sq * a.hq;
  const long grid = (rows + rows_per_block - 1) / rows_per_block;
  // the smallest unrolled split count that covers the plan's maximum
  if (a.max_splits <= 4)
    hipLaunchKernelGGL(k_combine<4>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  else if (a.max_splits <= 8)
    hipLaunchKernelGGL(k_combine<8>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_combine<16>, dim3((unsigned)grid), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const void* cache, const int32_t* block_table, int max_pages,
                         const int32_t* lens, int b, int page, int row_elems, int max_rows,
                         void* dst, hipStream_t s) {
  const long total = (long)max_rows * (row_elems / 8);
  const long grid = (total + 255) / 256;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const bf16_t*>(cache), block_table, max_pages, lens, b, page,
                     row_elems, max_rows, static_cast<bf16_t*>(dst));
  return hipGetLastError();
}

}  // namespace attn
