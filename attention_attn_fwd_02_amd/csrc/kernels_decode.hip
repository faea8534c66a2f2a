// Split-KV decode against a paged cache (GQA and MLA-absorbed shapes) and
// top-k sparse MLA with sinks, for gfx950.
// [MATE "Attention" page: flash_attn_with_kvcache, flash_mla_with_kvcache,
//  flash_mla_sparse_fwd; MindSpore sparse_flash_attention: sparse_indices,
//  sparse_mode, MLA-absorb concat; CANN flash_attn: paged attention via
//  block_table, shared KV, sink formulas]
#include "attn_core.h"
#include "launch.h"
#include "paged.h"

namespace attn {

namespace {

// Maps a workgroup id to a logical id such that the `grp` workgroups
// [g*grp, (g+1)*grp) that read the same keys are dispatched 8 ids apart and
// therefore land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_group(int p, int grp) {
  const int rest = (p / (8 * grp)) * 8 + (p & 7);
  return rest * grp + ((p >> 3) % grp);
}

inline int round_grid(long total, int grp) {
  const long unit = 8L * grp;
  return (int)(((total + unit - 1) / unit) * unit);
}

// One workgroup = (sequence b, split s, KV head kvh, row tile mt). Rows of a
// KV head are (query token t, query head of the group): row r -> t = r / G,
// head kvh*G + r % G. Keys are the split's range [kv0, kv1) of the sequence.
template <class C>
__global__ void __launch_bounds__(C::THREADS)
k_decode(DecodeArgs a) {
  using Core = TileCore<C>;
  using M = typename Core::M;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_BYTES / 2];
  const int grp = a.hq / a.hkv;
  const int nrows = a.sq * grp;
  const int mtiles = (nrows + C::ROWS - 1) / C::ROWS;
  const int logical = xcd_group(blockIdx.x, mtiles);
  if (logical >= a.batch * a.max_splits * a.hkv * mtiles) return;
  const int mt = logical % mtiles;
  int t = logical / mtiles;
  const int kvh = t % a.hkv;
  t /= a.hkv;
  const int s = t % a.max_splits;
  const int b = t / a.max_splits;
  const int* split_ptr = a.plan + 2;
  const int sp = split_ptr[b];
  if (s >= split_ptr[b + 1] - sp) return;
  const int* tri = a.plan + 3 + a.batch + 3 * (sp + s);
  const int kv0 = tri[1], kv1 = tri[2];
  const int lk = a.lens[b];
  const int delta = lk - a.sq;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = mt * C::ROWS + wave * C::R + M::row(lane);
  const bool row_ok = r < nrows;
  const int tq = row_ok ? r / grp : 0;
  const int h = kvh * grp + (row_ok ? r % grp : 0);
  const bf16_t* q = static_cast<const bf16_t*>(a.q);
  Core core;
  core.init();
  core.load_q(row_ok ? q + (((size_t)b * a.sq + tq) * a.hq + h) * C::D : nullptr, lane);

  const bf16_t* kc = static_cast<const bf16_t*>(a.kc);
  const bf16_t* vc = static_cast<const bf16_t*>(a.vc);
  auto kptr = [&](int j) -> const bf16_t* {
    return j < kv1 ? kc + paged_row_offset(a.block_table, a.max_pages, b, j, a.page, a.hkv, kvh,
                                           C::D)
                   : nullptr;
  };
  auto vptr = [&](int j) -> const bf16_t* {
    return j < kv1 ? vc + paged_row_offset(a.block_table, a.max_pages, b, j, a.page, a.hkv, kvh,
                                           C::DV)
                   : nullptr;
  };
  const int first_t = (mt * C::ROWS) / grp;
  auto vis = [&](int j) { return j < kv1 && (!a.causal || j <= tq + delta); };
  auto need = [&](int j0) {
    return j0 + C::BN > kv1 || (a.causal && j0 + C::BN - 1 > first_t + delta);
  };
  run_keys(core, lds, kv0, kv1, a.scale_log2, kptr, vptr, need, vis);

  float lse;
  const float inv = core.finish(false, 0.f, lse);
  if (row_ok) {
    const size_t slot = (size_t)b * a.max_splits + s;
    const size_t row = slot * nrows * a.hkv + (size_t)tq * a.hq + h;
    core.store(a.o_part + row * C::DV, inv, lane);
    if (M::grp(lane) == 0) a.lse_part[row] = lse;
  }
}

// One workgroup = (sequence b, query token t, head tile mt); all heads of a
// token share its index list, so the gathered key rows are staged once.
template <class C>
__global__ void __launch_bounds__(C::THREADS)
k_sparse(SparseArgs a) {
  using Core = TileCore<C>;
  using M = typename Core::M;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_BYTES / 2];
  const int mtiles = (a.hq + C::ROWS - 1) / C::ROWS;
  const int p = blockIdx.x;
  const int mt = p % mtiles;
  const int t = (p / mtiles) % a.sq;
  const int b = p / (mtiles * a.sq);
  if (b >= a.batch) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = mt * C::ROWS + wave * C::R + M::row(lane);
  const bool row_ok = h < a.hq;
  const bf16_t* q = static_cast<const bf16_t*>(a.q);
  Core core;
  core.init();
  core.load_q(row_ok ? q + (((size_t)b * a.sq + t) * a.hq + h) * C::D : nullptr, lane);

  const int32_t* ix = a.idx + ((size_t)b * a.sq + t) * a.topk;
  const int limit = a.mode == 3 ? min(a.sk - 1, t + a.sk - a.sq) : a.sk - 1;
  const bf16_t* kvb = static_cast<const bf16_t*>(a.kv) + (size_t)b * a.sk * C::D;
  auto kptr = [&](int j) -> const bf16_t* {
    if (j >= a.topk) return nullptr;
    const int id = ix[j];
    return (id >= 0 && id <= limit) ? kvb + (size_t)id * C::D : nullptr;
  };
  auto vis = [](int) { return true; };
  auto need = [](int) { return true; };
  run_keys(core, lds, 0, a.topk, a.scale_log2, kptr, kptr, need, vis);

  float lse;
  const float sink2 = (a.sinks && row_ok) ? a.sinks[h] * kLog2e : 0.f;
  const float inv = core.finish(a.sinks != nullptr, sink2, lse);
  if (row_ok) {
    core.store(static_cast<bf16_t*>(a.out) + (((size_t)b * a.sq + t) * a.hq + h) * C::DV, inv,
               lane);
    if (a.lse && M::grp(lane) == 0) a.lse[((size_t)b * a.hq + h) * a.sq + t] = lse;
  }
}

using CfgDecodeGqa = TileCfg<16, 128, 128, 1, 32, false>;
using CfgDecodeMla = TileCfg<16, 576, 512, 4, 32, true>;
using CfgSparseMla = TileCfg<16, 576, 512, 4, 32, true, true>;

}  // namespace

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t s) {
  using C = CfgDecodeGqa;
  const int nrows = a.sq * (a.hq / a.hkv);
  const int mt = (nrows + C::ROWS - 1) / C::ROWS;
  const int grid = round_grid((long)a.batch * a.max_splits * a.hkv * mt, mt);
  hipLaunchKernelGGL(k_decode<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s) {
  using C = CfgDecodeMla;
  const int nrows = a.sq * a.hq;
  const int mt = (nrows + C::ROWS - 1) / C::ROWS;
  const int grid = round_grid((long)a.batch * a.max_splits * mt, mt);
  hipLaunchKernelGGL(k_decode<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t s) {
  using C = CfgSparseMla;
  const int mt = (a.hq + C::ROWS - 1) / C::ROWS;
  const long grid = (long)a.batch * a.sq * mt;
  hipLaunchKernelGGL(k_sparse<C>, dim3((unsigned)grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
