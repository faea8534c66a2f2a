// Split-KV decode against a paged cache (GQA and MLA-absorbed shapes) and
// top-k sparse MLA with sinks, for gfx950.
// [MATE "Attention" page: flash_attn_with_kvcache, flash_mla_with_kvcache,
//  flash_mla_sparse_fwd; MindSpore sparse_flash_attention: sparse_indices,
//  sparse_mode, MLA-absorb concat; CANN flash_attn: paged attention via
//  block_table, shared KV, sink formulas]
#include "attn_core.h"
#include "attn_wide.h"
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
// Each 16-row block of a tile lies on one cache page (page sizes are
// multiples of 16 and splits start on page boundaries); the blocks' physical
// page numbers are wave-uniform and come from scalar loads of the block table.
template <class C>
__global__ void __launch_bounds__(C::THREADS)
k_decode(DecodeArgs a) {
  using T = StreamTile<C>;
  using M = Mfma<16>;
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char xchg[C::XCHG_BYTES > 0 ? C::XCHG_BYTES : 16];
  const int grp = a.hq / a.hkv;
  const int nrows = a.sq * grp;
  const int mtiles = (nrows + C::ROWS - 1) / C::ROWS;
  // Work items follow the plan's split list (batch-major, total = plan[0]):
  // item = (split, kv head, row tile). Real items come first, so they spread
  // over all XCDs; the row tiles of one (split, kv head) read the same keys
  // and are placed on one XCD.
  const int logical = xcd_group(blockIdx.x, mtiles);
  const int total = a.plan[0];
  if (logical >= total * a.hkv * mtiles) return;
  const int mt = logical % mtiles;
  const int kvh = (logical / mtiles) % a.hkv;
  const int split = logical / (mtiles * a.hkv);
  const int* tri = a.plan + 3 + a.batch + 3 * split;
  const int b = tri[0], kv0 = tri[1], kv1 = tri[2];
  const int s = split - a.plan[2 + b];
  const int lk = a.lens[b];
  const int delta = lk - a.sq;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = mt * C::ROWS + (wave / C::DSPLIT) * C::R + (lane & 15);
  const bool row_ok = r < nrows;
  const int tq = row_ok ? r / grp : 0;
  const int h = kvh * grp + (row_ok ? r % grp : 0);
  T tile;
  tile.init(wave);
  const size_t qoff = (((size_t)b * a.sq + tq) * a.hq + h) * C::D;
  if constexpr (C::QV == 2) {
    // only the qv path: no Q
  } else if constexpr (C::FP8) {
    tile.load_q8(row_ok ? static_cast<const uint8_t*>(a.q) + qoff : nullptr, lane);
  } else {
    tile.load_q(row_ok ? static_cast<const bf16_t*>(a.q) + qoff : nullptr, lane);
  }
  if constexpr (C::QV != 0) {
    const size_t qvoff = (((size_t)b * a.sq + tq) * a.hq + h) * C::DV * C::EB;
    tile.load_qv(row_ok ? static_cast<const char*>(a.qv) + qvoff : nullptr, lane);
  }
  // FP8: descales of (b, kvh) scale the scores and O (1 when not given); the
  // qv . v scores carry v_descale where q . k carry k_descale
  float cscale = a.scale_log2, vscale = 1.f, qv_ratio = 1.f;
  if constexpr (C::FP8) {
    const size_t di = (size_t)b * a.hkv + kvh;
    const float kd = a.k_descale ? a.k_descale[di] : 1.f;
    cscale *= (a.q_descale ? a.q_descale[di] : 1.f) * kd;
    vscale = a.v_descale ? a.v_descale[di] : 1.f;
    qv_ratio = vscale / kd;
  }
  wait_vmcnt<0>();  // Q in registers before any DMA is in flight

  // byte strides of one token's row in the caches and this KV head's column
  const size_t tok_k = (size_t)a.hkv * C::D * C::EB, tok_v = (size_t)a.hkv * C::DV * C::EB;
  const char* kcb = static_cast<const char*>(a.kc) + (size_t)kvh * C::D * C::EB;
  const char* vcb = static_cast<const char*>(C::VSHARED ? a.kc : a.vc) + (size_t)kvh * C::DV * C::EB;
  const int* btb = a.block_table + (size_t)b * a.max_pages;
  const int kv_last = kv1 - 1;
  // lane parts of the saddr-form DMA: bf16 tiles one offset each for K and V;
  // FP8 tiles two (the swizzle depends on one bit of the 8-row group)
  uint32_t klane = 0, vlane = 0, k8[2] = {0, 0};
  if constexpr (C::FP8) {
    k8[0] = T::lane_off8(lane, (uint32_t)tok_k, 0);
    k8[1] = T::lane_off8(lane, (uint32_t)tok_k, 1);
  } else {
    klane = T::k_lane_off(lane, (uint32_t)tok_k);
    vlane = T::v_lane_off(lane, (uint32_t)tok_v);
  }
  auto issue = [&](char* st, int ti) {
    // A 16-row block of a tile lies on one page (pages are multiples of 16
    // rows and splits start on page boundaries). sl[b]: cache slot of tile
    // row 16 b (clamped to the split's last key).
    constexpr int NB = C::BN / 16;
    const int j0 = kv0 + ti * C::BN;
    long sl[NB];
    static_for<NB / 2>([&](auto I) {
      constexpr int bb = 2 * decltype(I)::value;
      const int ja = min(j0 + 16 * bb, kv_last), jb = min(j0 + 16 * (bb + 1), kv_last);
      const int la = ja / a.page, lb = jb / a.page;
      int pa, pb;
      sload2_uniform(btb + la, btb + lb, pa, pb);
      sl[bb] = (long)pa * a.page + (ja - la * a.page);
      sl[bb + 1] = (long)pb * a.page + (jb - lb * a.page);
    });
    const int rmax = kv_last - j0;
    if (rmax >= C::BN - 1) {
      if constexpr (C::FP8) {
        auto kb = [&](int r8) { return kcb + (sl[r8 >> 1] + (r8 & 1) * 8) * (long)tok_k; };
        auto vb = [&](int r8) { return vcb + (sl[r8 >> 1] + (r8 & 1) * 8) * (long)tok_v; };
        T::dma_tile8_sv(st, kb, vb, k8[0], k8[1], k8[0], k8[1]);
      } else {
        T::dma_tile_sv(
            st,
            [&](int rb, int colb) {
              return typename T::Src{kcb + sl[rb] * (long)tok_k + colb, klane};
            },
            [&](int rb, int sub, int colb) {
              return typename T::Src{vcb + (sl[rb] + sub * 8) * (long)tok_v + colb, vlane};
            },
            wave);
      }
    } else {
      // last tile of the split: rows past its last key re-read that key,
      // which is masked; the lane's 16-row block selects its slot
      auto row = [&](int rr) {
        rr = min(rr, rmax);
        long v = sl[0];
        static_for<NB - 1>([&](auto I) {
          if ((rr >> 4) == decltype(I)::value + 1) v = sl[decltype(I)::value + 1];
        });
        return v + (rr & 15);
      };
      if constexpr (C::FP8)
        T::dma_tile8(
            st, [&](int rr) { return kcb + row(rr) * tok_k; },
            [&](int rr) { return vcb + row(rr) * tok_v; }, lane);
      else
        T::dma_tile(
            st, [&](int rr) { return reinterpret_cast<const bf16_t*>(kcb + row(rr) * tok_k); },
            [&](int rr) { return reinterpret_cast<const bf16_t*>(vcb + row(rr) * tok_v); }, wave,
            lane);
    }
  };
  const int first_t = (mt * C::ROWS) / grp;
  const int ntiles = (kv1 - kv0 + C::BN - 1) / C::BN;
  stream_tiles<C>(ring, ntiles, issue, [&](int ti, const char* st) {
    const int j0 = kv0 + ti * C::BN;
    const bool need = j0 + C::BN > kv1 || (a.causal && j0 + C::BN - 1 > first_t + delta);
    f32x4 sc[C::NSB];
    tile.qk(st, lane, sc);
    tile.qv_scores(st, lane, sc, qv_ratio);
    tile.exchange(xchg, wave, lane, sc);
    const int hi_vis = a.causal ? min(kv1 - 1, tq + delta) : kv1 - 1;
    const float m_use = tile.prep(sc, cscale, lane, need,
                                  [&](int jr) { return j0 + jr <= hi_vis; });
    uint32_t pk[C::NSB * 2];
    tile.probs(sc, cscale, m_use, pk);
    tile.pv(st, lane, pk);
  });

  float lse;
  const float inv = tile.finish(false, 0.f, lse) * vscale;
  if (row_ok) {
    const size_t slot_id = (size_t)b * a.max_splits + s;
    const size_t row = slot_id * nrows * a.hkv + (size_t)tq * a.hq + h;
    tile.store(a.o_part + row * C::DV, inv, lane);
    if (lane < 16 && tile.half == 0) a.lse_part[row] = lse;
  }
}

// MLA-absorbed decode on the wide tile: one workgroup = (split, row tile mt)
// of 128 rows (query token, head) of the single latent KV head; the rest as in
// k_decode.
template <class C>
__global__ void __launch_bounds__(C::THREADS)
k_decode_wide(DecodeArgs a) {
  using T = WideTile<C>;
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char xchg[C::XCHG_BYTES];
  __shared__ __attribute__((aligned(16))) char qlds[C::QLDS_BYTES > 0 ? C::QLDS_BYTES : 16];
  const int nrows = a.sq * a.hq;
  const int mtiles = (nrows + C::ROWS - 1) / C::ROWS;
  const int logical = xcd_group(blockIdx.x, mtiles);
  const int total = a.plan[0];
  if (logical >= total * mtiles) return;
  const int mt = logical % mtiles;
  const int split = logical / mtiles;
  const int* tri = a.plan + 3 + a.batch + 3 * split;
  const int b = tri[0], kv0 = tri[1], kv1 = tri[2];
  const int s = split - a.plan[2 + b];
  const int lk = a.lens[b];
  const int delta = lk - a.sq;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = mt * C::ROWS + (wave >> 1) * C::R + (lane & 31);
  const bool row_ok = r < nrows;
  const int tq = row_ok ? r / a.hq : 0;
  const int h = row_ok ? r % a.hq : 0;
  T tile;
  tile.init(wave);
  tile.load_q(row_ok ? static_cast<const bf16_t*>(a.q) + (((size_t)b * a.sq + tq) * a.hq + h) * C::D
                     : nullptr,
              qlds, wave, lane);
  wait_vmcnt<0>();  // Q in registers before any DMA is in flight

  const int* btb = a.block_table + (size_t)b * a.max_pages;
  const int kv_last = kv1 - 1;
  const uint32_t kstride = (uint32_t)(C::D * 2);
  const char* kcb = static_cast<const char*>(a.kc);
  auto issue = [&](char* st, int ti) {
    // 16-row blocks lie on one page each (see k_decode)
    const int j0 = kv0 + ti * C::BN;
    const int j1 = min(j0 + 16, kv_last);
    const int lp0 = j0 / a.page, lp1 = j1 / a.page;
    int p0, p1;
    sload2_uniform(btb + lp0, btb + lp1, p0, p1);
    const long slot0 = (long)p0 * a.page + (j0 - lp0 * a.page);
    const long slot1 = (long)p1 * a.page + (j1 - lp1 * a.page);
    const int rmax = kv_last - j0;
    if (rmax >= C::BN - 1) {
      const uint32_t klane = T::dma_lane_off(fresh_lane(), kstride);
      T::dma_tile_sv(
          st,
          [&](int rb, int colb) {
            return DmaSrc{kcb + (rb ? slot1 : slot0) * (long)kstride + colb, klane};
          },
          wave);
    } else {
      const int lane = fresh_lane();
      // last tile of the split: slot1 is tile row min(16, rmax); lane rows
      // past the split's last key re-read that key (masked), so the lane's
      // row offset from its block's first row is clamped to lim
      const int lim0 = min(rmax, 15), lim1 = max(rmax - 16, 0);
      T::dma_tile_sv(
          st,
          [&](int rb, int colb) {
            const uint32_t lr = min(T::dma_lane_row(lane), (uint32_t)(rb ? lim1 : lim0));
            return DmaSrc{kcb + (rb ? slot1 : slot0) * (long)kstride + colb,
                          lr * kstride + (lane >> 4) * 16};
          },
          wave);
    }
  };
  const int first_t = (mt * C::ROWS) / a.hq;
  const int ntiles = (kv1 - kv0 + C::BN - 1) / C::BN;
  stream_tiles<C>(ring, ntiles, issue, [&](int ti, const char* st) {
    const int j0 = kv0 + ti * C::BN;
    const bool need = j0 + C::BN > kv1 || (a.causal && j0 + C::BN - 1 > first_t + delta);
    f32x16 sc;
    tile.qk(st, qlds, wave, sc);
    tile.exchange(xchg, wave, sc);
    const float m_use = tile.prep(sc, a.scale_log2, need, [&](int jr) {
      // row of this lane, recomputed here rather than kept across the loop
      const int rr = mt * C::ROWS + (wave >> 1) * C::R + (fresh_lane() & 31);
      const int hi_vis = a.causal ? min(kv1 - 1, rr / a.hq + delta) : kv1 - 1;
      return j0 + jr <= hi_vis;
    });
    uint32_t pk[8];
    tile.probs(sc, a.scale_log2, m_use, pk);
    tile.pv(st, pk);
  });

  float lse;
  const float inv = tile.finish(false, 0.f, lse);
  if (row_ok) {
    const size_t slot_id = (size_t)b * a.max_splits + s;
    const size_t row = slot_id * nrows + (size_t)tq * a.hq + h;
    tile.store(a.o_part + row * C::DV, inv, lane);
    if (lane < 32 && tile.half == 0) a.lse_part[row] = lse;
  }
}

// One workgroup = (sequence b, query token t, head tile mt); all heads of a
// token share its key list. Index i names keys i*s .. i*s + s - 1 (s =
// 2^ls, the sparse block size; s = 1: token indices). The keys are taken in
// chunks of kMaxTopk: each chunk's physical rows (paged: through the block
// table) are staged in LDS, invalid keys as -1, whose rows are fetched from
// row 0 of the base (a valid address) and masked; the chunk is then streamed.
constexpr int kMaxTopk = 4096;

template <class C, bool PAGED>
__global__ void __launch_bounds__(C::THREADS)
k_sparse(SparseArgs a) {
  using T = StreamTile<C>;
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * C::STAGE_BYTES];
  __shared__ int sidx[kMaxTopk];
  __shared__ __attribute__((aligned(16))) char xchg[C::XCHG_BYTES > 0 ? C::XCHG_BYTES : 16];
  const int mtiles = (a.hq + C::ROWS - 1) / C::ROWS;
  const int p = blockIdx.x;
  const int mt = p % mtiles;
  const int t = (p / mtiles) % a.sq;
  const int b = p / (mtiles * a.sq);
  if (b >= a.batch) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = mt * C::ROWS + (wave / C::DSPLIT) * C::R + (lane & 15);
  const bool row_ok = h < a.hq;

  const int32_t* ix = a.idx + ((size_t)b * a.sq + t) * a.topk;
  const int lk = PAGED ? a.seqlens[b] : a.sk;
  const int limit = a.mode == 3 ? min(lk - 1, t + lk - a.sq) : lk - 1;
  const int nkeys = a.topk << a.ls;
  T tile;
  tile.init(wave);
  tile.load_q(row_ok ? static_cast<const bf16_t*>(a.q) + (((size_t)b * a.sq + t) * a.hq + h) * C::D
                     : nullptr,
              lane);
  wait_vmcnt<0>();

  // K rows are gathered: the uniform base is the sequence's first row (the
  // pool's first row when paged) and the lane offset the byte offset of its
  // row (fits 32 bits: checked on the host), plus its 16-byte column.
  static_assert(C::VSHARED, "sparse path reads V from the K rows");
  const char* kvb = reinterpret_cast<const char*>(
      static_cast<const bf16_t*>(a.kv) + (PAGED ? 0 : (size_t)b * a.sk * C::D));
  const int* btb = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
  const int lrow = (int)T::k_lane_row(lane);
  const uint32_t lcol = (lane >> 4) * 16;
  auto issue = [&](char* st, int ti) {
    const int* tix = sidx + ti * C::BN;
    const uint32_t r0 = (uint32_t)max(tix[lrow], 0) * (uint32_t)(C::D * 2) + lcol;
    const uint32_t r1 = (uint32_t)max(tix[16 + lrow], 0) * (uint32_t)(C::D * 2) + lcol;
    T::dma_tile_sv(
        st, [&](int rb, int colb) { return typename T::Src{kvb + colb, rb ? r1 : r0}; },
        [&](int, int, int) { return typename T::Src{kvb, 0u}; }, wave);
  };
  const int bmask = (1 << a.ls) - 1;
  for (int c0 = 0; c0 < nkeys; c0 += kMaxTopk) {
    const int n = min(kMaxTopk, nkeys - c0);
    const int ntiles = (n + C::BN - 1) / C::BN;
    __syncthreads();  // every wave is done with the previous chunk's list and ring
    for (int k = threadIdx.x; k < ntiles * C::BN; k += C::THREADS) {
      int row = -1;
      if (k < n) {
        const int key = c0 + k;
        const int id = ix[key >> a.ls];
        if (id >= 0 && id <= (limit >> a.ls)) {
          const int j = (id << a.ls) + (key & bmask);
          if (j <= limit) row = PAGED ? btb[j / a.page] * a.page + j % a.page : j;
        }
      }
      sidx[k] = row;
    }
    __syncthreads();
    stream_tiles<C>(ring, ntiles, issue, [&](int ti, const char* st) {
      const int* tix = sidx + ti * C::BN;
      f32x4 sc[C::NSB];
      tile.qk(st, lane, sc);
      tile.exchange(xchg, wave, lane, sc);
      const float m_use =
          tile.prep(sc, a.scale_log2, lane, true, [&](int jr) { return tix[jr] >= 0; });
      uint32_t pk[C::NSB * 2];
      tile.probs(sc, a.scale_log2, m_use, pk);
      tile.pv(st, lane, pk);
    });
  }

  float lse;
  const float sink2 = (a.sinks && row_ok) ? a.sinks[h] * kLog2e : 0.f;
  const float inv = tile.finish(a.sinks != nullptr, sink2, lse);
  if (row_ok) {
    tile.store(static_cast<bf16_t*>(a.out) + (((size_t)b * a.sq + t) * a.hq + h) * C::DV, inv,
               lane);
    if (a.lse && lane < 16 && tile.half == 0) a.lse[((size_t)b * a.hq + h) * a.sq + t] = lse;
  }
}

template <int QV = 0, int D = 128>
using CfgDecodeGqa = StreamCfg<D, D, 1, 3, false, 1, 0, QV>;
// FP8 tiles of 64 keys: the bytes of a 32-key bf16 tile
template <int FMT, int QV = 0>
using CfgDecodeGqa8 = StreamCfg<128, 128, 1, 3, false, 1, FMT, QV, 64>;
using CfgDecodeMla = WideCfg<576, 512, 3, 2>;
using CfgSparseMla = StreamCfg<576, 512, 8, 3, true, 2>;

}  // namespace

hipError_t launch_decode_gqa(const DecodeArgs& a, int d, hipStream_t s) {
  using C = CfgDecodeGqa<>;
  const int nrows = a.sq * (a.hq / a.hkv);
  const int mt = (nrows + C::ROWS - 1) / C::ROWS;
  const int grid = round_grid((long)a.batch * a.max_splits * a.hkv * mt, mt);
  static_assert(CfgDecodeGqa<0, 64>::ROWS == C::ROWS, "one grid for both head dims");
  if (d == 64)
    hipLaunchKernelGGL((k_decode<CfgDecodeGqa<0, 64>>), dim3(grid), dim3(C::THREADS), 0, s, a);
  else if (a.qv && a.only_qv)
    hipLaunchKernelGGL(k_decode<CfgDecodeGqa<2>>, dim3(grid), dim3(C::THREADS), 0, s, a);
  else if (a.qv)
    hipLaunchKernelGGL(k_decode<CfgDecodeGqa<1>>, dim3(grid), dim3(C::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_gqa_fp8(const DecodeArgs& a, int fmt, hipStream_t s) {
  using C = CfgDecodeGqa8<1>;
  const int nrows = a.sq * (a.hq / a.hkv);
  const int mt = (nrows + C::ROWS - 1) / C::ROWS;
  const int grid = round_grid((long)a.batch * a.max_splits * a.hkv * mt, mt);
  if (a.qv && a.only_qv) {
    if (fmt == 1)
      hipLaunchKernelGGL((k_decode<CfgDecodeGqa8<1, 2>>), dim3(grid), dim3(C::THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((k_decode<CfgDecodeGqa8<2, 2>>), dim3(grid), dim3(C::THREADS), 0, s, a);
  } else if (a.qv) {
    if (fmt == 1)
      hipLaunchKernelGGL((k_decode<CfgDecodeGqa8<1, 1>>), dim3(grid), dim3(C::THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((k_decode<CfgDecodeGqa8<2, 1>>), dim3(grid), dim3(C::THREADS), 0, s, a);
  } else if (fmt == 1) {
    hipLaunchKernelGGL(k_decode<CfgDecodeGqa8<1>>, dim3(grid), dim3(C::THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_decode<CfgDecodeGqa8<2>>, dim3(grid), dim3(C::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s) {
  using C = CfgDecodeMla;
  const int nrows = a.sq * a.hq;
  const int mt = (nrows + C::ROWS - 1) / C::ROWS;
  const int grid = round_grid((long)a.batch * a.max_splits * mt, mt);
  hipLaunchKernelGGL(k_decode_wide<C>, dim3(grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t s) {
  using C = CfgSparseMla;
  const int mt = (a.hq + C::ROWS - 1) / C::ROWS;
  const long grid = (long)a.batch * a.sq * mt;
  if (a.block_table)
    hipLaunchKernelGGL((k_sparse<C, true>), dim3((unsigned)grid), dim3(C::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_sparse<C, false>), dim3((unsigned)grid), dim3(C::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
