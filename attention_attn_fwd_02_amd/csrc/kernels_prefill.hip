// Packed variable-length attention (prefill) for gfx950.
// [MATE "Attention" page, FMHA: flash_attn_varlen_func; CANN flash_attn:
//  cu_seqlens_q / cu_seqlens_kv; lite_boost flash_attention: causal and
//  window_size]
#include "attn_core.h"  // dump_rows
#include "launch.h"
#include "paged.h"
#include "prefill_bf16.h"

namespace attn {

namespace {

// Work order shared by the prefill grids: longest query tiles first (with a
// causal mask the last tile of a sequence sees the most keys), and the query
// heads of one GQA group placed 8 workgroup ids apart so that they run on the
// same XCD (workgroups are dispatched round-robin over the 8 XCDs) and share
// their K/V tiles through that XCD's L2.
struct PrefillWork {
  int b, h, kvh, qt;
};

__device__ __forceinline__ bool decode_prefill_work(int p, int batch, int hq, int hkv, int nqt,
                                                    PrefillWork& w) {
  const int grp = hq / hkv;
  const int rest = (p / (8 * grp)) * 8 + (p & 7);
  const int hg = (p >> 3) % grp;
  const int logical = rest * grp + hg;
  if (logical >= nqt * batch * hq) return false;
  int t = logical / grp;
  w.kvh = t % hkv;
  t /= hkv;
  w.b = t % batch;
  w.qt = nqt - 1 - t / batch;
  w.h = w.kvh * grp + hg;
  return true;
}

// Work order of the cache-plus-current kernels: sequences by their number of
// keys (cache plus current rows, largest first), each sequence's query tiles
// last to first, then its KV heads. Cache lengths vary widely between
// sequences, so the qt-major order above would leave the longest items for
// the end; taking them first is the longest-processing-time rule of list
// scheduling (a list-schedule simulation of the chunked-prefill workload
// over 768 workgroup slots: makespan 414 tiles against 482). The ranks are
// computed by every workgroup from the lengths (batch <= kSortBatch; beyond
// that the sequences keep their order). All threads take part (barriers).
constexpr int kSortBatch = 256;

struct SortScratch {
  int key[kSortBatch];
  int perm[kSortBatch];
};

__device__ __forceinline__ void sort_sequences(const VarlenArgs& a, SortScratch& ss, int tid,
                                               int nthreads) {
  const bool sorted = a.batch <= kSortBatch;
  for (int b = tid; b < a.batch && sorted; b += nthreads)
    ss.key[b] = a.cache_lens[b] + (a.cu_k[b + 1] - a.cu_k[b]);
  __syncthreads();
  for (int b = tid; b < a.batch && sorted; b += nthreads) {
    const int kb = ss.key[b];
    int r = 0;
    for (int c = 0; c < a.batch; ++c) {
      const int kc = ss.key[c];
      r += (kc > kb || (kc == kb && c < b)) ? 1 : 0;
    }
    ss.perm[r] = b;
  }
  __syncthreads();
}

__device__ __forceinline__ bool decode_prefill_work_kvc(int p, const VarlenArgs& a,
                                                        const SortScratch& ss, PrefillWork& w) {
  const int grp = a.hq / a.hkv;
  const int rest = (p / (8 * grp)) * 8 + (p & 7);
  const int hg = (p >> 3) % grp;
  const int logical = rest * grp + hg;
  if (logical >= a.nqt * a.batch * a.hq) return false;
  int t = logical / grp;
  w.kvh = t % a.hkv;
  t /= a.hkv;
  w.qt = a.nqt - 1 - t % a.nqt;
  const int r = t / a.nqt;
  w.b = a.batch <= kSortBatch ? ss.perm[r] : r;
  w.h = w.kvh * grp + hg;
  return true;
}

int prefill_grid(int batch, int hq, int hkv, int nqt) {
  const int unit = 8 * (hq / hkv);
  const long total = (long)nqt * batch * hq;
  return (int)(((total + unit - 1) / unit) * unit);
}

// Key range and masking of one query tile [row0, row_last] of a sequence with
// Lq queries and Lk keys; diagonal of query t is t + (Lk - Lq).
struct Band {
  int lo, hi;       // keys to visit
  int delta, wl, wr;  // wr is -1 (unbounded) or the effective right bound
};

__device__ __forceinline__ Band make_band(int row0, int row_last, int lq, int lk, int causal,
                                          int wl, int wr, int bn) {
  Band bd;
  bd.delta = lk - lq;
  bd.wl = wl;
  bd.wr = causal ? (wr < 0 ? 0 : min(wr, 0)) : wr;
  bd.hi = lk;
  if (bd.wr >= 0) bd.hi = min(bd.hi, row_last + bd.delta + bd.wr + 1);
  bd.lo = 0;
  if (wl >= 0) bd.lo = max(0, row0 + bd.delta - wl);
  bd.lo = (bd.lo / bn) * bn;
  return bd;
}

// KVC: the keys of sequence b are its cache_lens[b] cached rows (paged:
// row j at block_table[b][j / page], slot j % page) followed by its current
// rows [cu_k[b], cu_k[b+1]). Page sizes are multiples of 16, so each 16-row
// block of a tile that lies wholly in the cache sits on one page.
// MASK: an additive bf16 mask (mask_heads, Tq, mask_ld) is added to the scaled
// scores; each wave streams its 32 rows x BN mask entries of every key tile
// into the stage beside K and V (4 lanes per 64-byte row segment, coalesced).
// C::FP8: Q, K and V are FP8 codes; the descales of (sequence, KV head) scale
// the scores (q and k) and the output (v).
// QV: a second query qv is scored against the V rows; each stage also holds
// V in the K layout (a third DMA of the same rows) for that product.
// DUMP: the gather-test instance; the same work items and tile issue, but
// query tile 0 of the first query head of each KV head copies every staged
// K and V tile out (rows of the sequence's keys, cache rows first,
// un-swizzled) instead of computing on it (launched without causal mask or
// window, so that this tile visits every key).
template <class C, bool KVC, bool MASK, bool QV = false, bool DUMP = false>
__device__ __forceinline__ void varlen_body(const VarlenArgs& a) {
  using T = PrefillTile<C, QV>;
  static_assert(C::FP8 == 0 || !MASK, "FP8 tiles: no mask");
  static_assert(!QV || !MASK, "qv: no mask");
  static_assert(!QV || !KVC || C::FP8 == 0, "qv over a cache: bfloat16");
  constexpr int MASK_BAND = C::R * C::BN * 2;              // one wave's rows of a tile
  constexpr int VK_OFF = 2 * C::TILE_BYTES;                // V in the K layout (QV)
  constexpr int MASK_OFF = VK_OFF + (QV ? C::TILE_BYTES : 0);
  constexpr int STAGE = MASK_OFF + (MASK ? C::NW * MASK_BAND : 0);
  constexpr int MASK_DMA = MASK ? C::BN / 16 : 0;          // mask instructions per wave
  // ring of STAGES buffers, each one K tile, one V tile (and the mask tile)
  __shared__ __attribute__((aligned(1024))) char ring[C::STAGES * STAGE];
  PrefillWork w;
  if constexpr (KVC && !DUMP) {
    __shared__ SortScratch ss;
    sort_sequences(a, ss, threadIdx.x, C::THREADS);
    if (!decode_prefill_work_kvc(blockIdx.x, a, ss, w)) return;
  } else {
    if (!decode_prefill_work(blockIdx.x, a.batch, a.hq, a.hkv, a.nqt, w)) return;
  }
  const int q0 = a.cu_q[w.b];
  const int lq = a.cu_q[w.b + 1] - q0;
  const int row0 = w.qt * C::ROWS;
  if (row0 >= lq) return;
  const int k0 = a.cu_k[w.b];
  const int tq_all = a.cu_q[a.batch];  // LSE row stride, read with the bounds
  const int lc = KVC ? a.cache_lens[w.b] : 0;  // cached keys come first
  const int lk = lc + a.cu_k[w.b + 1] - k0;
  const int row_last = min(lq, row0 + C::ROWS) - 1;
  const Band bd = make_band(row0, row_last, lq, lk, a.causal, a.wl, a.wr, C::BN);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int trow = row0 + wave * C::R + (lane & 31);
  const int wrow0 = row0 + wave * C::R;             // this wave's first row
  const int wrow1 = min(lq, wrow0 + C::R) - 1;      // and its last row in the sequence
  const bool row_ok = trow < lq;
  T t;
  t.init();
  const size_t qoff = ((size_t)(q0 + trow) * a.hq + w.h) * C::D * C::EB;  // bytes
  if constexpr (!DUMP) t.load_q(row_ok ? static_cast<const char*>(a.q) + qoff : nullptr, lane);
  if constexpr (QV) t.load_qv(row_ok ? static_cast<const char*>(a.qv) + qoff : nullptr, lane);
  // Q must be in registers before any LDS-DMA is in flight: the compiler
  // cannot count the DMA operations, so any vmcnt wait it placed for Q inside
  // the key loop would also drain the prefetch of the next tile.
  wait_vmcnt<0>();

  // rows of this KV head, row_bytes apart (byte addresses)
  const long row_bytes = (long)a.hkv * C::D * C::EB;
  const size_t head = (size_t)w.kvh * C::D * C::EB;
  const char* kb = static_cast<const char*>(a.k) + (size_t)k0 * row_bytes + head;
  const char* vb = static_cast<const char*>(a.v) + (size_t)k0 * row_bytes + head;
  const int last = lk - 1;  // rows past the sequence re-read its last key (then masked)
  // STAGES-1 tiles are in flight while one is computed; a single barrier per
  // tile both publishes tile i and retires every wave's reads of tile i-1,
  // whose buffer then receives tile i+STAGES-1.
  uint32_t koff[C::NOFF], voff[C::NOFF];
  T::template dma_lane_offs<false>(lane, (uint32_t)row_bytes, wave, koff);
  T::template dma_lane_offs<true>(lane, (uint32_t)row_bytes, wave, voff);
  // cache bases of this KV head (KVC only)
  const char* kcb = KVC ? static_cast<const char*>(a.kc) + head : nullptr;
  const char* vcb = KVC ? static_cast<const char*>(a.vc) + head : nullptr;
  const int* btb = KVC ? a.block_table + (size_t)w.b * a.max_pages : nullptr;
  // mask rows of this wave (rows past the sequence re-read its last row)
  const char* mbase = nullptr;
  const int mrow0 = min(wrow0, lq - 1);  // the wave's first mask row in the sequence
  if constexpr (MASK) {
    const int tq = a.cu_q[a.batch];
    const int hm = a.mask_heads > 1 ? w.h : 0;
    mbase = static_cast<const char*>(a.mask) + ((size_t)hm * tq + q0 + mrow0) * a.mask_ld * 2;
  }
  auto issue = [&](char* buf, int i) {
    const int j0 = bd.lo + i * C::BN;  // key index of tile row 0 (cache rows first)
    if constexpr (MASK) {
      // lane offsets rebuilt per tile from a fresh lane id (a few VALU
      // operations) rather than held in registers across the key loop
      constexpr int UPR = C::BN / 8, RPI = 64 / UPR;  // 16-byte units per row, rows per instr.
      const int ln = fresh_lane();
#pragma unroll
      for (int n = 0; n < MASK_DMA; ++n) {
        const int r = min(wrow0 + n * RPI + ln / UPR, lq - 1);
        const uint32_t off = (uint32_t)(r - mrow0) * (uint32_t)a.mask_ld * 2 + (ln % UPR) * 16;
        lds_dma16_sv(mbase + j0 * 2, off, buf + MASK_OFF + wave * MASK_BAND + n * 1024);
      }
    }
    if (!KVC || j0 >= lc) {
      const int c0 = j0 - lc;  // current row of tile row 0
      if (j0 + C::BN - 1 <= last) {
        T::template dma_tile_sv<false>(buf, kb + c0 * row_bytes, row_bytes, koff, wave);
        T::template dma_tile_sv<true>(buf + C::TILE_BYTES, vb + c0 * row_bytes, row_bytes, voff,
                                      wave);
        if constexpr (QV)
          T::template dma_tile_sv<false>(buf + VK_OFF, vb + c0 * row_bytes, row_bytes, koff,
                                         wave);
      } else {
        // the cache variant holds more state across the key loop: its lane
        // constants are rebuilt here rather than kept live
        const int ln = KVC ? fresh_lane() : lane;
        T::template dma_tile<false>(
            buf, [&](int r) { return kb + (long)(min(j0 + r, last) - lc) * row_bytes; }, wave, ln);
        T::template dma_tile<true>(
            buf + C::TILE_BYTES,
            [&](int r) { return vb + (long)(min(j0 + r, last) - lc) * row_bytes; }, wave, ln);
        if constexpr (QV)
          T::template dma_tile<false>(
              buf + VK_OFF, [&](int r) { return vb + (long)(min(j0 + r, last) - lc) * row_bytes; },
              wave, ln);
      }
      return;
    }
    if constexpr (KVC) {
      // cache slot of the first row of each 16-row block of the tile (blocks
      // past the cache clamp to its last row and are not used)
      constexpr int NB = C::BN / 16;
      long sl[NB];
      paged_block_slots<NB>(btb, a.page, j0, lc - 1, sl);
      auto slot = [&](int rb) { return block_slot(sl, rb); };
      if (j0 + C::BN - 1 < lc) {
        auto kblk = [&](int rb) { return kcb + slot(rb) * row_bytes; };
        auto vblk = [&](int rb) { return vcb + slot(rb) * row_bytes; };
        T::template dma_tile_blk<false>(buf, kblk, row_bytes, koff, wave);
        T::template dma_tile_blk<true>(buf + C::TILE_BYTES, vblk, row_bytes, voff, wave);
        if constexpr (QV) T::template dma_tile_blk<false>(buf + VK_OFF, vblk, row_bytes, koff, wave);
      } else {
        // the tile straddles the end of the cache (or is the last tile):
        // per-lane rows, cached ones through the block slots above
        const int ln = fresh_lane();
        auto row = [&](const char* cb, const char* cur, int r) -> const char* {
          const int j = min(j0 + r, last);
          if (j < lc) return cb + (slot((j - j0) >> 4) + ((j - j0) & 15)) * row_bytes;
          return cur + (long)(j - lc) * row_bytes;
        };
        T::template dma_tile<false>(buf, [&](int r) { return row(kcb, kb, r); }, wave, ln);
        T::template dma_tile<true>(buf + C::TILE_BYTES, [&](int r) { return row(vcb, vb, r); },
                                   wave, ln);
        if constexpr (QV)
          T::template dma_tile<false>(buf + VK_OFF, [&](int r) { return row(vcb, vb, r); }, wave,
                                      ln);
      }
    }
  };
  const int tdiag = trow + bd.delta;
  float cscale = a.scale_log2;
  float vscale = 1.f, qv_ratio = 1.f;
  if constexpr (C::FP8 != 0) {
    const int dsi = w.b * a.hkv + w.kvh;
    const float kd = a.k_descale ? a.k_descale[dsi] : 1.f;
    if (a.q_descale) cscale *= a.q_descale[dsi];
    cscale *= kd;
    if (a.v_descale) vscale = a.v_descale[dsi];
    qv_ratio = vscale / kd;
  }
  const int ntiles = bd.hi > bd.lo ? (bd.hi - bd.lo + C::BN - 1) / C::BN : 0;
  auto stage = [&](int i) { return ring + i * STAGE; };  // i < STAGES
  // DMA instructions per wave per tile
  constexpr int PER_TILE = (QV ? 3 : 2) * C::DMA_PER_WAVE + MASK_DMA;
  static_assert(PER_TILE * (C::STAGES - 1) < 64, "vmcnt range");
#pragma unroll
  for (int i = 0; i < C::STAGES - 1; ++i)
    if (i < ntiles) issue(stage(i), i);
  auto process = [&](int i, char* cur, char* refill) {
    // tile i has landed once at most `after` later tiles are outstanding
    const int after = min(ntiles - 1 - i, C::STAGES - 2);
    static_for<C::STAGES - 1>([&](auto I) {
      if (after == decltype(I)::value) wait_vmcnt<decltype(I)::value * PER_TILE>();
    });
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own reads of tile i-1 retired
    barrier_no_fence();
    if (i + C::STAGES - 1 < ntiles) issue(refill, i + C::STAGES - 1);
    const int j0 = bd.lo + i * C::BN;
    if constexpr (DUMP) {
      if (w.qt == 0 && w.h % (a.hq / a.hkv) == 0) {
        constexpr int UNITS = C::D * C::EB / 16;
        auto dst = [&](void* base, int r) {
          return static_cast<char*>(base) +
                 (((size_t)w.b * a.dump_rows + j0 + r) * a.hkv + w.kvh) * (UNITS * 16);
        };
        const int n = min(C::BN, lk - j0);
        dump_rows<UNITS>(
            cur, n, [](int r, int u) { return T::template lds_unit<false>(r, u); },
            [&](int r) { return dst(a.dump_k, r); }, threadIdx.x, C::THREADS);
        dump_rows<UNITS>(
            cur + C::TILE_BYTES, n, [](int r, int u) { return T::template lds_unit<true>(r, u); },
            [&](int r) { return dst(a.dump_v, r); }, threadIdx.x, C::THREADS);
      }
      return;
    }
    // per wave: skip a tile none of its rows sees (on the causal diagonal or
    // past a window, or rows past the sequence); mask only where some of its
    // rows see part of the tile
    if (wrow1 < wrow0 || (bd.wr >= 0 && j0 > wrow1 + bd.delta + bd.wr) ||
        (bd.wl >= 0 && j0 + C::BN - 1 < wrow0 + bd.delta - bd.wl))
      return;
    const bool need = j0 + C::BN > lk ||
                      (bd.wr >= 0 && j0 + C::BN - 1 > wrow0 + bd.delta + bd.wr) ||
                      (bd.wl >= 0 && j0 < wrow1 + bd.delta - bd.wl);
    f32x16 s[C::NSB];
    t.qk(cur, lane, s);
    t.qv_scores(cur + VK_OFF, lane, s, qv_ratio);
    float cs = cscale;
    if constexpr (MASK) {
      T::add_mask(s, cur + MASK_OFF + wave * MASK_BAND, cs, fresh_lane());
      cs = 1.f;  // the scores are scaled
    }
    if (need) {
      // visible keys of this lane's row, as tile indices
      const int hi = min(lk - 1, bd.wr < 0 ? lk - 1 : tdiag + bd.wr) - j0;
      if (bd.wl < 0) T::template mask<false>(s, lane, 0, hi);
      else T::template mask<true>(s, lane, tdiag - bd.wl - j0, hi);
    }
    uint32_t pk[C::NSB * 8];
    t.softmax(s, cs, pk);
    t.pv(cur + C::TILE_BYTES, lane, pk);
  };
  // unrolled by STAGES so that every buffer address is a constant
  for (int i = 0; i < ntiles; i += C::STAGES) {
#pragma unroll
    for (int k = 0; k < C::STAGES; ++k)
      if (i + k < ntiles)
        process(i + k, ring + k * STAGE, ring + ((k + C::STAGES - 1) % C::STAGES) * STAGE);
  }

  if constexpr (DUMP) return;
  float lse;
  const float inv =
      t.finish(a.sinks != nullptr, a.sinks ? a.sinks[w.h] * kLog2e : 0.f, lse) * vscale;
  if (row_ok) {
    t.store(static_cast<bf16_t*>(a.out) + ((size_t)(q0 + trow) * a.hq + w.h) * C::DV, inv, lane);
    if (a.lse && lane < 32) a.lse[(size_t)w.h * tq_all + q0 + trow] = lse;
  }
}

template <class C, bool KVC, bool MASK = false>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_bf16(VarlenArgs a) {
  varlen_body<C, KVC, MASK>(a);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_fp8(VarlenArgs a) {
  varlen_body<C, false, false>(a);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_fp8_kvc(VarlenArgs a) {
  varlen_body<C, true, false>(a);
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_qv(VarlenArgs a) {
  varlen_body<C, false, false, true>(a);
}

// qv over a paged cache plus the current rows (bfloat16)
template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_qv_kvc(VarlenArgs a) {
  varlen_body<C, true, false, true>(a);
}

// gather test: the cache-plus-current tile issue with the tiles copied out
template <class C>
__global__ void __launch_bounds__(C::THREADS, C::MIN_WAVES) k_varlen_kvc_dump(VarlenArgs a) {
  varlen_body<C, true, false, false, true>(a);
}

// ---------------------------------------------------------------------------
// float32 variant: VALU arithmetic in fp32 throughout (no bf16 rounding of
// inputs or probabilities). LPR = D / 8 lanes share one query row, each
// holding 8 of its head dimensions; a dot product is summed over those lanes
// with log2(LPR) butterfly exchanges. One wave covers 64 / LPR rows, and the
// four waves of a workgroup take the same rows and every fourth 32-key tile
// of their key range each (a split of the keys inside the workgroup, so a
// short problem still spreads over many SIMDs). Each wave stages its own
// tiles in its part of LDS with 16-byte loads; at the end the waves' running
// (max, sum, O) are merged through LDS by wave 0, the merge of [MATE]'s
// combine with weights 2^(m_w - M).
template <int D>
struct F32Cfg {
  static constexpr int DPL = 8;           // head dimensions per lane
  static constexpr int LPR = D / DPL;     // lanes per query row (8 or 16)
  static constexpr int NW = 4;            // waves, one key share each
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = 64 / LPR;   // query rows of the workgroup (and of each wave)
  static constexpr int BN = 32;
  static_assert(64 % LPR == 0, "a row's lanes stay within one wave");
};

template <int D>
__global__ void __launch_bounds__(256) k_varlen_f32(VarlenArgs a) {
  using C = F32Cfg<D>;
  __shared__ __attribute__((aligned(16))) float ks[C::NW][C::BN][D];
  __shared__ __attribute__((aligned(16))) float vs[C::NW][C::BN][D];
  __shared__ __attribute__((aligned(16))) float mo[C::NW - 1][64][C::DPL];
  __shared__ float ml[C::NW - 1][64][2];
  PrefillWork w;
  if (!decode_prefill_work(blockIdx.x, a.batch, a.hq, a.hkv, a.nqt, w)) return;
  const int q0 = a.cu_q[w.b];
  const int lq = a.cu_q[w.b + 1] - q0;
  const int row0 = w.qt * C::ROWS;
  if (row0 >= lq) return;
  const int k0 = a.cu_k[w.b];
  const int lk = a.cu_k[w.b + 1] - k0;
  // the LSE row stride, read with the sequence bounds rather than after the
  // merge, where it would add a memory round trip to this short kernel
  const int tq_all = a.cu_q[a.batch];
  const int row_last = min(lq, row0 + C::ROWS) - 1;
  const Band bd = make_band(row0, row_last, lq, lk, a.causal, a.wl, a.wr, C::BN);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = lane % C::LPR;
  const int trow = row0 + lane / C::LPR;
  const bool row_ok = trow < lq;
  const float* q = static_cast<const float*>(a.q);
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);
  float qr[C::DPL], o[C::DPL];
  {
    f32x4 q4[2] = {f32x4{}, f32x4{}};
    if (row_ok) {
      const f32x4* qp = reinterpret_cast<const f32x4*>(
          q + ((size_t)(q0 + trow) * a.hq + w.h) * D + part * C::DPL);
      q4[0] = qp[0];
      q4[1] = qp[1];
    }
#pragma unroll
    for (int d = 0; d < C::DPL; ++d) {
      qr[d] = q4[d / 4][d % 4];
      o[d] = 0.f;
    }
  }
  float m_run = kNegInf, l_run = 0.f;
  const int tdiag = trow + bd.delta;
  float (*kw)[D] = ks[wave];
  float (*vw)[D] = vs[wave];
  for (int j0 = bd.lo + wave * C::BN; j0 < bd.hi; j0 += C::NW * C::BN) {
    // this wave's tile; only this wave reads it, so the wave's own ordering
    // of LDS operations (and the compiler barrier) is the only sync needed.
    // All of a lane's loads are issued before its first store, so the tile
    // costs one memory latency, not one per 16-byte element.
    constexpr int PER_LANE = C::BN * D / 4 / 64;
    f32x4 kv[PER_LANE], vv[PER_LANE];
#pragma unroll
    for (int n = 0; n < PER_LANE; ++n) {
      const int e = lane + 64 * n;
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      const int j = j0 + r;
      kv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      vv[n] = kv[n];
      if (j < lk) {
        const size_t off = ((size_t)(k0 + j) * a.hkv + w.kvh) * D + c;
        kv[n] = *reinterpret_cast<const f32x4*>(kg + off);
        vv[n] = *reinterpret_cast<const f32x4*>(vg + off);
      }
    }
#pragma unroll
    for (int n = 0; n < PER_LANE; ++n) {
      const int e = lane + 64 * n;
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(&kw[r][c]) = kv[n];
      *reinterpret_cast<f32x4*>(&vw[r][c]) = vv[n];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float s[C::BN];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < C::BN; ++j) {
      const f32x4* kr = reinterpret_cast<const f32x4*>(&kw[j][part * C::DPL]);
      const f32x4 ka = kr[0], kb = kr[1];
      float acc = qr[0] * ka[0];
      acc = fmaf(qr[1], ka[1], acc);
      acc = fmaf(qr[2], ka[2], acc);
      acc = fmaf(qr[3], ka[3], acc);
      acc = fmaf(qr[4], kb[0], acc);
      acc = fmaf(qr[5], kb[1], acc);
      acc = fmaf(qr[6], kb[2], acc);
      acc = fmaf(qr[7], kb[3], acc);
#pragma unroll
      for (int m = 1; m < C::LPR; m <<= 1) acc += __shfl_xor(acc, m);
      const int jj = j0 + j;
      const bool ok = jj < lk && (bd.wr < 0 || jj <= tdiag + bd.wr) && (bd.wl < 0 || jj >= tdiag - bd.wl);
      s[j] = ok ? acc * a.scale_log2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < C::DPL; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < C::BN; ++j) {
      const float p = fast_exp2(s[j] - m_use);
      l_run += p;
      const f32x4* vr = reinterpret_cast<const f32x4*>(&vw[j][part * C::DPL]);
      const f32x4 va = vr[0], vb = vr[1];
      o[0] = fmaf(p, va[0], o[0]);
      o[1] = fmaf(p, va[1], o[1]);
      o[2] = fmaf(p, va[2], o[2]);
      o[3] = fmaf(p, va[3], o[3]);
      o[4] = fmaf(p, vb[0], o[4]);
      o[5] = fmaf(p, vb[1], o[5]);
      o[6] = fmaf(p, vb[2], o[6]);
      o[7] = fmaf(p, vb[3], o[7]);
    }
    // the next tile's stores must not pass this tile's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge: waves 1..NW-1 hand their (m, l, O) to wave 0
  if (wave > 0) {
#pragma unroll
    for (int d = 0; d < C::DPL; ++d) mo[wave - 1][lane][d] = o[d];
    ml[wave - 1][lane][0] = m_run;
    ml[wave - 1][lane][1] = l_run;
  }
  __syncthreads();
  if (wave > 0) return;
  float mw[C::NW], lw[C::NW];
  mw[0] = m_run;
  lw[0] = l_run;
  float mm = m_run;
#pragma unroll
  for (int v = 1; v < C::NW; ++v) {
    mw[v] = ml[v - 1][lane][0];
    lw[v] = ml[v - 1][lane][1];
    mm = fmaxf(mm, mw[v]);
  }
  const float m_ref = mm == kNegInf ? 0.f : mm;
  float l_sum = 0.f;
#pragma unroll
  for (int v = 0; v < C::NW; ++v) {
    const float f = fast_exp2(mw[v] - m_ref);  // 0 for a wave that saw no key
    l_sum += lw[v] * f;
    if (v == 0) {
#pragma unroll
      for (int d = 0; d < C::DPL; ++d) o[d] *= f;
    } else {
#pragma unroll
      for (int d = 0; d < C::DPL; ++d) o[d] = fmaf(mo[v - 1][lane][d], f, o[d]);
    }
  }
  const bool empty = !(l_sum > 0.f);
  const float lse = empty ? kNegInf : (m_ref + fast_log2(l_sum)) * kLn2;
  float inv = empty ? 0.f : 1.f / l_sum;
  if (a.sinks && !empty) {
    const float sink2 = a.sinks[w.h] * kLog2e;
    const float ms = fmaxf(m_ref, sink2);
    const float f = fast_exp2(m_ref - ms);
    inv = f / (l_sum * f + fast_exp2(sink2 - ms));
  }
  if (row_ok) {
    f32x4* orow = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) +
                                           ((size_t)(q0 + trow) * a.hq + w.h) * D +
                                           part * C::DPL);
    orow[0] = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    orow[1] = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    if (a.lse && part == 0) a.lse[(size_t)w.h * tq_all + q0 + trow] = lse;
  }
}

using CfgP64 = PrefillCfg<64, 4, 64>;
// D = 128: a 2-stage ring (one tile in flight while one is computed). At 3
// waves per SIMD the tile DMA needs no deeper prefetch, and the smaller
// stages keep 3 workgroups per CU where a stage also holds the mask band
// (the masked chunked prefill: 0.97 -> 0.73 ms; FP8 chunked 0.54 -> 0.515 ms).
using CfgP128 = PrefillCfg<128, 4, 32, 3, 2>;
// attn_fwd_varlen_mask: its instance needs more registers than 3 waves per
// SIMD allow (the compiler would spill); 2 waves per SIMD and a 3-stage ring
using CfgP128M = PrefillCfg<128, 4, 32, 2, 3>;
static_assert(CfgP128M::ROWS == CfgP128::ROWS, "one grid for both");
template <int FMT>
using CfgP8 = PrefillCfg<128, 4, 32, 3, 2, FMT>;
static_assert(CfgP8<1>::ROWS == CfgP128::ROWS, "FP8 grid sized by varlen_bf16_rows(128)");
// FP8 keys over a paged cache (the same tile, with the cache slots)
template <int FMT>
using CfgP8Kv = PrefillCfg<128, 4, 32, 3, 2, FMT>;
// qv: the second query's fragments take 2 waves per SIMD (bf16 or FP8 codes)
template <int FMT>
using CfgPQv = PrefillCfg<128, 4, 32, 2, 2, FMT>;
static_assert(CfgPQv<0>::ROWS == CfgP128::ROWS, "qv grid sized by varlen_bf16_rows(128)");

}  // namespace

int varlen_bf16_rows(int d) { return d == 64 ? CfgP64::ROWS : CfgP128::ROWS; }
int varlen_f32_rows(int d) { return d == 64 ? F32Cfg<64>::ROWS : F32Cfg<128>::ROWS; }

hipError_t launch_varlen_bf16(const VarlenArgs& a, int d, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (a.mask) {
    if (d == 64)
      hipLaunchKernelGGL((k_varlen_bf16<CfgP64, false, true>), dim3(grid), dim3(CfgP64::THREADS),
                         0, s, a);
    else
      hipLaunchKernelGGL((k_varlen_bf16<CfgP128M, false, true>), dim3(grid),
                         dim3(CfgP128M::THREADS), 0, s, a);
    return hipGetLastError();
  }
  if (d == 64)
    hipLaunchKernelGGL((k_varlen_bf16<CfgP64, false>), dim3(grid), dim3(CfgP64::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_varlen_bf16<CfgP128, false>), dim3(grid), dim3(CfgP128::THREADS), 0, s,
                       a);
  return hipGetLastError();
}

hipError_t launch_varlen_kvcache_bf16(const VarlenArgs& a, int d, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (a.mask) {
    if (d == 64)
      hipLaunchKernelGGL((k_varlen_bf16<CfgP64, true, true>), dim3(grid), dim3(CfgP64::THREADS), 0,
                         s, a);
    else
      hipLaunchKernelGGL((k_varlen_bf16<CfgP128, true, true>), dim3(grid),
                         dim3(CfgP128::THREADS), 0, s, a);
  } else if (d == 64) {
    hipLaunchKernelGGL((k_varlen_bf16<CfgP64, true>), dim3(grid), dim3(CfgP64::THREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_varlen_bf16<CfgP128, true>), dim3(grid), dim3(CfgP128::THREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_varlen_fp8(const VarlenArgs& a, int fmt, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (fmt == 1)
    hipLaunchKernelGGL(k_varlen_fp8<CfgP8<1>>, dim3(grid), dim3(CfgP8<1>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_varlen_fp8<CfgP8<2>>, dim3(grid), dim3(CfgP8<2>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_varlen_kvcache_fp8(const VarlenArgs& a, int fmt, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (fmt == 1)
    hipLaunchKernelGGL(k_varlen_fp8_kvc<CfgP8Kv<1>>, dim3(grid), dim3(CfgP8Kv<1>::THREADS), 0, s,
                       a);
  else
    hipLaunchKernelGGL(k_varlen_fp8_kvc<CfgP8Kv<2>>, dim3(grid), dim3(CfgP8Kv<2>::THREADS), 0, s,
                       a);
  return hipGetLastError();
}

hipError_t launch_dump_kvcache(const VarlenArgs& a, int fmt, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (fmt == 0)
    hipLaunchKernelGGL(k_varlen_kvc_dump<CfgP128>, dim3(grid), dim3(CfgP128::THREADS), 0, s, a);
  else if (fmt == 1)
    hipLaunchKernelGGL(k_varlen_kvc_dump<CfgP8Kv<1>>, dim3(grid), dim3(CfgP8Kv<1>::THREADS), 0, s,
                       a);
  else
    hipLaunchKernelGGL(k_varlen_kvc_dump<CfgP8Kv<2>>, dim3(grid), dim3(CfgP8Kv<2>::THREADS), 0, s,
                       a);
  return hipGetLastError();
}

hipError_t launch_varlen_qv(const VarlenArgs& a, int fmt, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (fmt == 0)
    hipLaunchKernelGGL(k_varlen_qv<CfgPQv<0>>, dim3(grid), dim3(CfgPQv<0>::THREADS), 0, s, a);
  else if (fmt == 1)
    hipLaunchKernelGGL(k_varlen_qv<CfgPQv<1>>, dim3(grid), dim3(CfgPQv<1>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_varlen_qv<CfgPQv<2>>, dim3(grid), dim3(CfgPQv<2>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_varlen_kvcache_qv_bf16(const VarlenArgs& a, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  hipLaunchKernelGGL(k_varlen_qv_kvc<CfgPQv<0>>, dim3(grid), dim3(CfgPQv<0>::THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_varlen_f32(const VarlenArgs& a, int d, hipStream_t s) {
  const int grid = prefill_grid(a.batch, a.hq, a.hkv, a.nqt);
  if (d == 64)
    hipLaunchKernelGGL(k_varlen_f32<64>, dim3(grid), dim3(F32Cfg<64>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(k_varlen_f32<128>, dim3(grid), dim3(F32Cfg<128>::THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
