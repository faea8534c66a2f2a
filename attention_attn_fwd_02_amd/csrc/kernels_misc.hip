// Split planner and LSE-weighted combine.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
// plans of at most this many splits get a longest-first work order
constexpr int kPlanSortMax = 4096;

// ceil(a / b) for a >= 0, b > 0, with no overflow near the type's maximum
__device__ __forceinline__ int cdiv(int a, int b) { return a / b + (a % b != 0); }
__device__ __forceinline__ long cdiv(long a, long b) { return a / b + (a % b != 0); }

// Number of splits of a sequence of nb > 0 blocks; pps = blocks per split.
__device__ __forceinline__ int plan_splits_of(int nb, int bps, int max_splits, int& pps) {
  const int ns = min(max_splits, max(1, cdiv(nb, bps)));
  pps = cdiv(nb, ns);
  return cdiv(nb, pps);
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ long wave_prefix_sum(long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long u = __shfl_up(v, (unsigned)d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Work-order key of a split: longer first, then lower split index.
__device__ __forceinline__ unsigned long long order_key(int length, int index) {
  return ((unsigned long long)(0x7FFFFFFF - length) << 32) | (unsigned)index;
}

// Split plan [MATE get_scheduler_metadata / get_mla_metadata; CANN
// flash_attn_metadata: a metadata pass that fixes the work split before the
// main call]. The rule is this library's own, integer only:
//   nblk_b = ceil(len_b / page) (0 if len_b <= 0)
//   bps    = max(min_blocks, ceil(sum nblk_b * upb / (num_cu * waves)))
//   ns_b   = min(max_splits, max(1, ceil(nblk_b / bps)))
//   pps_b  = ceil(nblk_b / ns_b), ns_b = ceil(nblk_b / pps_b)
// One workgroup; each thread owns a contiguous run of sequences, and the
// sums over sequences are wave prefix sums joined through LDS. The work
// order after the triples lists the splits longest first (ties in split
// order): the decode workgroups take splits in that order, the
// longest-processing-time rule of list scheduling. The keys ((2^31 - 1 -
// length) << 32 | index) are unique, so the result does not depend on how
// they are sorted. All splits of a sequence but its last have one length and
// consecutive indices, so they form a group that no other key falls inside:
// a group's place in the order is the total size of the groups whose first
// key is smaller, and the sort reduces to ranking at most two groups per
// sequence (one group per thread, up to kPlanThreads groups). Beyond that, a
// bitonic network in LDS sorts the split keys themselves, up to kPlanSortMax.
__global__ void __launch_bounds__(kPlanThreads)
k_plan(const int32_t* __restrict__ lens, int batch, int page, int upb, int num_cu, int waves,
       int max_splits, int min_blocks, int32_t* __restrict__ plan) {
  __shared__ long wsum[2][kPlanWaves];
  __shared__ __attribute__((aligned(16))) unsigned long long skey[kPlanSortMax];
  __shared__ __attribute__((aligned(16))) int gsize[kPlanThreads];

  const int tid = threadIdx.x, wave = tid >> 6;
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(batch, tid * per), b1 = min(batch, b0 + per);
  long blocks = 0;
  for (int b = b0; b < b1; ++b) blocks += lens[b] > 0 ? cdiv(lens[b], page) : 0;
  blocks = wave_prefix_sum(blocks);
  if ((tid & 63) == 63) wsum[0][wave] = blocks;
  __syncthreads();
  long total_blocks = 0;
  for (int w = 0; w < kPlanWaves; ++w) total_blocks += wsum[0][w];
  const long total_units = total_blocks * upb;
  const int bps = (int)max((long)min_blocks, cdiv(total_units, (long)num_cu * waves));

  // splits (high word) and groups (low word) of this thread's sequences
  long mine = 0;
  for (int b = b0; b < b1; ++b) {
    const int nb = lens[b] > 0 ? cdiv(lens[b], page) : 0;
    if (nb) {
      int pps;
      const int ns = plan_splits_of(nb, bps, max_splits, pps);
      mine += ((long)ns << 32) + (ns > 1 ? 2 : 1);
    }
  }
  const long incl = wave_prefix_sum(mine);
  if ((tid & 63) == 63) wsum[1][wave] = incl;
  __syncthreads();
  long before = 0, all = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    const long v = wsum[1][w];
    before += w < wave ? v : 0;
    all += v;
  }
  const long first = before + incl - mine;
  int ptr = (int)(first >> 32), gptr = (int)(first & 0xFFFFFFFFl);
  const int total = (int)(all >> 32), ngroups = (int)(all & 0xFFFFFFFFl);
  const bool sort = total <= kPlanSortMax;
  const bool by_group = sort && ngroups <= kPlanThreads;

  int32_t* split_ptr = plan + 2;
  int32_t* tri = plan + 3 + batch;
  for (int b = b0; b < b1; ++b) {
    split_ptr[b] = ptr;
    const int len = lens[b];
    const int nb = len > 0 ? cdiv(len, page) : 0;
    if (nb) {
      int pps;
      const int ns = plan_splits_of(nb, bps, max_splits, pps);
      const long span = (long)pps * page;
      for (int s = 0; s < ns; ++s) {
        const int kv0 = (int)(s * span), kv1 = (int)min((s + 1) * span, (long)len);
        tri[3 * (ptr + s)] = b;
        tri[3 * (ptr + s) + 1] = kv0;
        tri[3 * (ptr + s) + 2] = kv1;
        if (sort && !by_group) skey[ptr + s] = order_key(kv1 - kv0, ptr + s);
      }
      if (by_group) {
        if (ns > 1) {
          skey[gptr] = order_key((int)span, ptr);
          gsize[gptr++] = ns - 1;
        }
        skey[gptr] = order_key(len - (int)((ns - 1) * span), ptr + ns - 1);
        gsize[gptr++] = 1;
      }
      ptr += ns;
    }
  }
  if (tid == kPlanThreads - 1) {
    split_ptr[batch] = total;
    plan[0] = total;
    plan[1] = bps;
  }
  int32_t* order = plan + 3 + batch + 3 * batch * max_splits;
  if (by_group) {
    // Keys and sizes are read 8 at a time (the pad up to a multiple of 8 has
    // keys above any group's and size 0) into independent sums, so that the
    // reads of one iteration overlap.
    const int n8 = (ngroups + 7) & ~7;
    if (tid >= ngroups && tid < n8) {
      skey[tid] = ~0ull;
      gsize[tid] = 0;
    }
    __syncthreads();
    if (tid < ngroups) {
      typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      const unsigned long long key = skey[tid];
      const u64x2* kv = reinterpret_cast<const u64x2*>(skey);
      const i32x4* sz = reinterpret_cast<const i32x4*>(gsize);
      int r[4] = {0, 0, 0, 0};
      for (int i = 0; i < n8; i += 8) {
        u64x2 k[4];
        i32x4 z[2];
#pragma unroll
        for (int u = 0; u < 4; ++u) k[u] = kv[i / 2 + u];
        z[0] = sz[i / 4];
        z[1] = sz[i / 4 + 1];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          r[u] += (k[u][0] < key ? z[u / 2][2 * (u % 2)] : 0) +
                  (k[u][1] < key ? z[u / 2][2 * (u % 2) + 1] : 0);
      }
      const int pos = (r[0] + r[1]) + (r[2] + r[3]);
      const int idx = (int)(unsigned)key;
      for (int i = 0; i < gsize[tid]; ++i) order[pos + i] = idx + i;
    }
  } else if (sort) {
    int n2 = 1;
    while (n2 < total) n2 <<= 1;
    for (int i = total + tid; i < n2; i += kPlanThreads) skey[i] = ~0ull;
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kPlanThreads) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long x = skey[i], y = skey[l];
            if ((x > y) == ((i & k) == 0)) {
              skey[i] = y;
              skey[l] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < total; i += kPlanThreads) order[i] = (int32_t)(unsigned)skey[i];
  } else {
    for (int i = tid; i < total; i += kPlanThreads) order[i] = i;
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

}  // namespace attn
