// Wide streaming tile for MLA-absorbed decode, where every query row of a
// sequence attends to the same single latent KV head: 32 query rows per wave
// pair on v_mfma_f32_32x32x16_bf16 and 128 rows per workgroup of 8 waves.
// Each byte brought into LDS, and each LDS read, then feeds twice as many
// rows as in the 16-row engine of attn_core.h, whose 64-row workgroups are
// bounded by how fast one CU can take tiles in from L2.
//
// Wave pair p (waves 2p and 2p+1) owns rows 32p .. 32p+31 of the workgroup.
// Wave 2p+h holds the head-dimension chunks of parity h (Q K^T over them
// gives a partial S^T, summed with the partner's through LDS) and the value
// columns [DV/2 h, DV/2 (h+1)) of the output.
//
// LDS layout of one tile (BN = 32 rows x D; V is the first DV columns of the
// same rows), 16-byte units, c = chunk index along the row:
//   [row / 16][c][(row % 16) ^ sw(c)],  sw(c) = 8 (c & 1) ^ 4 ((c >> 1) & 1)
// * Q K^T reads (b128): lanes 0-31 read chunk a and lanes 32-63 chunk a+4 of
//   rows 0..31. sw(a) = sw(a+4), so all lanes of an instruction use one row
//   permutation: each 16-lane group reads one 256-byte block, a relabelling
//   of the banks of a plain contiguous read.
// * V reads (ds_read_b64_tr_b16): each 16-lane block reads 4 rows x 2 chunks
//   (128 bytes); sw places blocks 0/1 (and 2/3) in complementary halves of
//   the 64 banks.
#pragma once
#include "attn_core.h"

namespace attn {

// QLDS of each wave's Q fragments are kept in LDS instead of registers (the
// register file holds 2 waves per SIMD only just: 128 accumulator registers
// for O and 72 for Q of a 576-wide head); 0 keeps Q wholly in registers.
template <int D_, int DV_, int STAGES_, int QLDS_ = 2>
struct WideCfg {
  static constexpr int D = D_, DV = DV_, STAGES = STAGES_, QLDS = QLDS_;
  static constexpr int NW = 8, DSPLIT = 2, R = 32, BN = 32;
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW / DSPLIT * R;
  static constexpr int NCH = D / 8;
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int STAGE_BYTES = K_BYTES;  // V shares the K rows
  static constexpr int K_DMA = K_BYTES / 1024;
  static constexpr int DMA_WAVES = NW / DSPLIT;
  static constexpr int DMA_PER_WAVE = K_DMA / DMA_WAVES;
  static constexpr int VM_PER_TILE = DMA_PER_WAVE;  // vector-memory instructions per tile
  static constexpr int NQ = D / 16 / DSPLIT;    // Q fragments (16 head dims each) per wave
  static constexpr int NOB = DV / 32 / DSPLIT;  // 32-column O^T blocks per wave
  static constexpr int XCHG_BYTES = NW * 4 * 64 * 16;  // [wave][quarter][lane] x f32x4
  static constexpr int NQR = NQ - QLDS;                // Q fragments held in registers
  static constexpr int QLDS_BYTES = NW * QLDS * 1024;  // [wave][fragment][lane] x 16 B
  static constexpr int QK_PREFETCH = 3;                 // K fragments read ahead in Q K^T
  static constexpr int PV_PREFETCH = 2;                 // V fragments read ahead in P V
  static constexpr bool SCHED_GROUPS = true;
  static_assert(D % 64 == 0 && NCH % 8 == 0, "chunk classes need D % 64 == 0");
  static_assert(DV % 64 == 0 && DV <= D, "value width");
  static_assert(K_DMA % DMA_WAVES == 0, "tile DMA must split evenly over the waves");
  static_assert(DMA_PER_WAVE * (STAGES - 1) < 64, "vmcnt range");
  static_assert(QLDS >= 0 && QLDS < NQ, "QLDS");
};

template <class C>
struct WideTile {
  using M = Mfma<32>;
  bf16x8 qf[C::NQR];
  f32x16 o[C::NOB];
  float m_ref;  // reference max (base-2 scaled domain), -inf until a key is seen
  float l_run;  // this lane's share of sum 2^(s*c - m_ref)
  int half;     // parity of the head-dimension chunks / half of the value columns

  __device__ __forceinline__ static int sw(int c) { return ((c & 1) << 3) ^ (((c >> 1) & 1) << 2); }

  __device__ __forceinline__ void init(int wave) {
    half = wave & 1;
#pragma unroll
    for (int i = 0; i < C::NOB; ++i) o[i] = f32x16{};
    m_ref = kNegInf;
    l_run = 0.f;
  }

  // Fragment t of half h: lane group g (= lane >> 5) holds chunk
  // 8 (t / 2) + h + 2 (t % 2) + 4 g, 8 head dims.
  __device__ __forceinline__ static int q_chunk(int t, int h, int g) {
    return 8 * (t >> 1) + h + 2 * (t & 1) + 4 * g;
  }

  // Fragments NQR .. NQ-1 go to this wave's part of qlds (read back by the
  // same wave only, so no barrier is needed).
  __device__ __forceinline__ void load_q(const bf16_t* qrow, char* qlds, int wave, int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int t = 0; t < C::NQ; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow) v = *reinterpret_cast<const u32x4*>(qrow + q_chunk(t, half, g) * 8);
      if (t < C::NQR)
        qf[t] = as_bf16x8(v);
      else
        *reinterpret_cast<u32x4*>(qlds + (wave * C::QLDS + t - C::NQR) * 1024 + lane * 16) = v;
    }
  }

  // Byte offset of 16-byte unit u (chunk u of 8 elements) of tile row r in a
  // stage: the layout above (used by the DUMP instance of the gather test).
  __device__ __forceinline__ static int lds_unit(int r, int u) {
    return (r >> 4) * C::NCH * 256 + u * 256 + ((r & 15) ^ sw(u)) * 16;
  }

  // DMA of one tile. Instruction inst covers the 16-row block inst / (NCH/4)
  // and chunks 4 (inst % (NCH/4)) .. +3; lane -> chunk +(lane >> 4), row
  // (lane & 15) ^ sw(lane >> 4) of the block, landing at 16 * lane of the
  // instruction's 1 KB. Waves 0 .. DMA_WAVES-1 issue: one on each SIMD
  // (waves w and w+4 share one), so the other wave of that SIMD keeps its
  // MFMA pipe busy while the issuing wave waits for the address unit.
  __device__ __forceinline__ static uint32_t dma_lane_row(int lane) {
    return (uint32_t)((lane & 15) ^ sw(lane >> 4));
  }
  __device__ __forceinline__ static uint32_t dma_lane_off(int lane, uint32_t row_bytes) {
    return dma_lane_row(lane) * row_bytes + (lane >> 4) * 16;
  }
  // saddr form: ksrc(rb, colb) gives the wave-uniform base of row 16 rb of
  // the tile plus the uniform column offset colb, and the lane's offset.
  template <class KSrc>
  __device__ __forceinline__ static void dma_tile_sv(char* stage, KSrc ksrc, int wave) {
    if (wave >= C::DMA_WAVES) return;
    const int dw = wave;
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      constexpr int IPB = C::NCH / 4;
      const int inst = dw * C::DMA_PER_WAVE + n;
      const DmaSrc a = ksrc(inst / IPB, (inst % IPB) * 64);
      lds_dma16_sv(a.s, a.v, stage + inst * 1024);
    }
  }
  // per-lane form: krow(r) is the global address of tile row r
  template <class KRow>
  __device__ __forceinline__ static void dma_tile(char* stage, KRow krow, int wave, int lane) {
    if (wave >= C::DMA_WAVES) return;
    const int dw = wave;
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      constexpr int IPB = C::NCH / 4;
      const int inst = dw * C::DMA_PER_WAVE + n;
      const int c = (inst % IPB) * 4 + (lane >> 4);
      const int r = (inst / IPB) * 16 + (int)dma_lane_row(lane);
      lds_dma16(krow(r) + c * 8, stage + inst * 1024);
    }
  }

  // Partial S^T (32 keys x this pair's 32 rows) over this wave's chunks.
  __device__ __forceinline__ void qk(const char* stage, const char* qlds, int wave,
                                     f32x16& s) const {
    const int lane = fresh_lane();
    const int g = lane >> 5, key = lane & 31;
    const int rb = key >> 4, slot = key & 15;
    // fragment parity p: chunk a + 4g with a % 4 = half + 2p, sw = 8 half ^ 4p
    const char* kb0 = stage + (rb * C::NCH + half + 4 * g) * 256 + (slot ^ (8 * half)) * 16;
    const char* kb1 = stage + (rb * C::NCH + half + 2 + 4 * g) * 256 + (slot ^ (8 * half ^ 4)) * 16;
    auto kload = [&](int t) {
      const char* kb = (t & 1) ? kb1 : kb0;
      return *reinterpret_cast<const u32x4*>(kb + 8 * (t >> 1) * 256);
    };
    // K fragments are read PF ahead of their MFMA; the schedule groups below
    // keep the compiler from sinking the reads next to their uses.
    constexpr int PF = C::QK_PREFETCH;
    u32x4 ka[C::NQ];
#pragma unroll
    for (int t = 0; t < PF; ++t) ka[t] = kload(t);
    s = f32x16{};
#pragma unroll
    for (int t = 0; t < C::NQ; ++t) {
      if (t + PF < C::NQ) ka[t + PF] = kload(t + PF);
      bf16x8 q;
      if (t < C::NQR)
        q = qf[t];
      else
        q = as_bf16x8(*reinterpret_cast<const u32x4*>(
            qlds + (wave * C::QLDS + t - C::NQR) * 1024 + lane * 16));
      s = M::mma(as_bf16x8(ka[t]), q, s);
    }
    if constexpr (C::SCHED_GROUPS) {
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // PF LDS reads
      static_for<C::NQ>([&](auto I) {
        constexpr int t = decltype(I)::value;
        constexpr int reads = (t + PF < C::NQ) + (t + 1 >= C::NQR && t + 1 < C::NQ);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);
      });
    }
  }

  // Adds the partner's partial S^T. The buffer is reused every tile: the
  // caller's per-tile barrier (after lgkmcnt(0)) orders the partner's reads
  // of one tile before the writes of the next. Float addition commutes, so
  // both waves obtain the same sums.
  __device__ __forceinline__ void exchange(char* xchg, int wave, f32x16& s) const {
    const int lane = fresh_lane();
    f32x4* mine = reinterpret_cast<f32x4*>(xchg) + wave * 4 * 64 + lane;
    const f32x4* other = reinterpret_cast<const f32x4*>(xchg) + (wave ^ 1) * 4 * 64 + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) mine[q * 64] = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own writes done
    barrier_no_fence();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = other[q * 64];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * q + i] += x[i];
    }
  }

  // Masks the scores of tile-relative keys j with !vis(j).
  template <class Vis>
  __device__ __forceinline__ static void mask(f32x16& s, Vis vis) {
    const int g = fresh_lane() >> 5;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!vis(M::mrow(g, r))) s[r] = kNegInf;
  }

  // p = 2^(s*c - m) packed to bf16 pairs: pk[4c .. 4c+3] is the B operand of
  // the P.V instruction over keys 16c .. 16c+15 (in the S^T register order);
  // l += sum p in float32. The reference is checked after the exponentials
  // (see PrefillTile::softmax): a lane whose probabilities sum to more than
  // kSumLimit, or whose row has no reference yet, sends the wave down the
  // rare path that raises the reference to the row maximum (rescaling O and
  // l) and recomputes the tile.
  __device__ __forceinline__ void exps(const f32x16& s, float cscale, uint32_t (&pk)[8],
                                       float& l) const {
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[r], cscale, -m_use));
      const float p1 = fast_exp2(__builtin_fmaf(s[r + 1], cscale, -m_use));
      l = r == 0 ? p0 + p1 : l + (p0 + p1);
      pk[r / 2] = pack_bf16x2(p0, p1);
    }
  }
  __device__ __forceinline__ void softmax(const f32x16& s, float cscale, uint32_t (&pk)[8]) {
    float l;
    exps(s, cscale, pk, l);
    if (__ballot(l > kSumLimit || m_ref == kNegInf) != 0) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const float rmx = M::group_max(mx) * cscale;
      if (rmx > m_ref) {
        const float alpha = fast_exp2(m_ref - rmx);  // m_ref = -inf -> 0
        m_ref = rmx;
        l_run *= alpha;
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob) o[ob] *= alpha;
      }
      exps(s, cscale, pk, l);
    }
    l_run += l;
  }

  // O^T += V^T P^T. Lane l (16-lane block b = l >> 4, i = l & 15, group
  // g = l >> 5) addresses tile row g*4 + i/4 (+8 for the upper half of the
  // A operand) of each 16-key block and 4 value columns starting at
  // 16 (b & 1) + 4 (i % 4), so that it receives column l % 32 of keys
  // g*4 .. g*4+3 (and 8 + g*4 ..): the key order of the S^T registers.
  __device__ __forceinline__ void pv(const char* stage, const uint32_t (&pk)[8]) {
    const int lane = fresh_lane();
    const int b = lane >> 4, i = lane & 15, g = lane >> 5;
    const int cc = half * (C::DV / 16) + 2 * (b & 1) + ((i & 3) >> 1);  // chunk (+ 4 ob)
    const int fs = (((i & 3) >> 1) << 3) ^ ((b & 1) << 2);               // sw(cc)
    const int klo = g * 4 + (i >> 2);
    const char* lo_b = stage + cc * 256 + ((klo ^ fs) * 16) + (i & 1) * 8;
    const char* hi_b = stage + cc * 256 + (((klo + 8) ^ fs) * 16) + (i & 1) * 8;
    // instruction n = c * NOB + ob; V fragments are read PF ahead
    constexpr int N = 2 * C::NOB, PF = C::PV_PREFETCH;
    auto vload = [&](int n) {
      const int off = ((n / C::NOB) * C::NCH + 4 * (n % C::NOB)) * 256;
      const s16x4 lo = lds_read_tr(reinterpret_cast<const bf16_t*>(lo_b + off));
      const s16x4 hi = lds_read_tr(reinterpret_cast<const bf16_t*>(hi_b + off));
      return join_bf16x8(lo, hi);
    };
    bf16x8 va[N];
#pragma unroll
    for (int n = 0; n < PF; ++n) va[n] = vload(n);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (n + PF < N) va[n + PF] = vload(n + PF);
      const int c = n / C::NOB, ob = n % C::NOB;
      const u32x4 p4 = {pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
      o[ob] = M::mma(va[n], as_bf16x8(p4), o[ob]);
    }
    if constexpr (C::SCHED_GROUPS) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 1);  // PF fragments (2 reads each)
      static_for<N>([&](auto I) {
        constexpr int n = decltype(I)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if constexpr (n + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      });
    }
  }

  __device__ __forceinline__ float finish(bool has_sink, float sink2, float& lse) const {
    const float l = M::group_sum(l_run);
    const bool empty = !(l > 0.f);
    lse = empty ? kNegInf : (m_ref + fast_log2(l)) * kLn2;
    if (!has_sink) return empty ? 0.f : 1.f / l;
    if (empty) return 0.f;
    const float ms = fmaxf(m_ref, sink2);
    const float f = fast_exp2(m_ref - ms);
    return f / (l * f + fast_exp2(sink2 - ms));
  }

  // Writes this wave's DV/2 output columns of its row (float32).
  __device__ __forceinline__ void store(float* orow, float inv, int lane) const {
    const int g = lane >> 5;
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = half * (C::DV / 2) + ob * 32 + q * 8 + g * 4;
        const f32x4 w = {o[ob][4 * q] * inv, o[ob][4 * q + 1] * inv, o[ob][4 * q + 2] * inv,
                         o[ob][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + col) = w;
      }
    }
  }
};

}  // namespace attn
