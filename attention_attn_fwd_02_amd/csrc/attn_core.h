// Streaming tile engine for the decode-side kernels on gfx950 (paged GQA
// decode, MLA-absorbed decode, top-k sparse MLA): 16 query rows per wave on
// v_mfma_f32_16x16x32_bf16, keys streamed through an LDS ring.
//
//   S^T = K Q^T   (A = K tile from LDS, B = this wave's Q rows in registers)
//   online softmax per row in the base-2 domain with a reference max
//   checked after the exponentials (see prefill_bf16.h)
//   O^T += V^T P^T (A = V read transposed from LDS, B = P from the S^T
//   registers, which are already in B-operand order)
//
// Keys are consumed in tiles of BN rows (32; 64 for FP8). Each tile is copied global ->
// LDS with global_load_lds_dwordx4 into a ring of STAGES buffers, so up to
// STAGES-1 tiles are in flight per workgroup; the caller supplies the global
// row address of every key of a tile (row(r), always a valid address) and,
// after the ring, waits only on the DMA of the tile it is about to read.
//
// LDS layouts (16-byte units, c = chunk index along the row; 64 banks x 4 B):
//   K, V shared with K (MLA): [row / 16][c][(row % 16) ^ 8*(c & 1)]
//      16 lanes reading 16 rows of one chunk cover 256 contiguous bytes; the
//      parity swizzle makes the transposed V reads of a shared K/V row (MLA)
//      conflict-free too: two 16-lane blocks reading chunks 2k and 2k+1 of
//      8 rows land in opposite 128-byte halves.
//   K, separate V: [row / 16][c / 4][row % 16][(c % 4) ^ ((row % 16) / 4)]
//      the DMA reads each 64-byte row segment with 4 consecutive lanes
//      (coalesced); 16 lanes reading 16 rows of one chunk take the 16
//      combinations of row % 4 (16-bank group) and swizzled slot (4 banks).
//   V (when not shared): [row / 8][c / 2][row % 8][c % 2]
//      two 16-lane ds_read_b64_tr_b16 blocks (8 consecutive rows, one chunk
//      pair) cover 256 contiguous bytes.
#pragma once
#include "device_common.h"
#include "prefill_bf16.h"  // lds_dma16, wait_vmcnt, barrier_no_fence, kSumLimit

namespace attn {

// Source of one DMA instruction in the saddr form: wave-uniform base and the
// lane's byte offset from it.
struct DmaSrc {
  const char* s;
  uint32_t v;
};

// DSPLIT = 2 pairs the waves of a workgroup (waves 2p and 2p+1): both own
// the same 16 query rows, each holds half of every Q row and half of every
// output row, computes the partial S^T over its half of the head dimension,
// and the two partials are summed through LDS so that both waves continue
// with identical scores. Waves 0 .. NW/2-1 issue the DMA. This halves
// the registers a wave needs for wide heads (MLA: 576 / 512), so two waves
// fit on each SIMD and hide each other's LDS latency.
//
// FP8 = 1 (e4m3fn) or 2 (e5m2): Q, K and V hold 8-bit codes. Tiles reach LDS
// as bytes (half the traffic). Q.K^T runs on the FP8 MFMA over the codes
// (exact products, fp32 sums); V fragments are widened to bfloat16 as they
// are read (exact), so P.V, the softmax and the partial outputs are those of
// the bfloat16 path; descales are applied to the scores and to O.
//
// QV = 1: a second query qv (Dv wide) is scored against the value rows of
// the tile, S^T += V Qv^T, read in place from the V layout (no second copy).
// QV = 2: only that score path; tiles hold V alone (no K bytes, no Q).
//
// BN: keys per tile, 32, or a multiple of 32 for FP8 tiles (whose rows are
// half as wide, so 64 keys move the bytes of a 32-key bf16 tile).
//
// MASK: an additive bf16 mask tile (16 rows x BN keys, row-major) follows K
// and V in each stage, brought in by one more DMA instruction per tile; it is
// added to the scaled scores before the softmax (one wave, bf16 only).
template <int D_, int DV_, int NW_, int STAGES_, bool VSHARED_, int DSPLIT_ = 1, int FP8_ = 0,
          int QV_ = 0, int BN_ = 32, bool MASK_ = false>
struct StreamCfg {
  static constexpr int D = D_, DV = DV_, NW = NW_, STAGES = STAGES_;
  static constexpr bool VSHARED = VSHARED_;
  static constexpr int DSPLIT = DSPLIT_;
  static constexpr int FP8 = FP8_;
  static constexpr int QV = QV_;
  static constexpr bool MASK = MASK_;
  static constexpr int EB = FP8 ? 1 : 2;  // bytes per element in memory and LDS
  static constexpr int BN = BN_, R = 16;
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW / DSPLIT * R;
  static constexpr int DMA_WAVES = NW / DSPLIT;
  static constexpr int NCH = D / 8;
  static constexpr int K_BYTES = QV == 2 ? 0 : BN * D * EB;
  static constexpr int V_BYTES = VSHARED ? 0 : BN * DV * EB;
  static constexpr int MASK_BYTES = MASK ? R * BN * 2 : 0;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES + MASK_BYTES;
  static constexpr int K_DMA = K_BYTES / 1024;
  static constexpr int V_DMA = V_BYTES / 1024;
  static constexpr int DMA_PER_WAVE = (K_DMA + V_DMA) / DMA_WAVES;
  // vector-memory instructions per wave per tile (the tile loop's vmcnt waits)
  static constexpr int VM_PER_TILE = DMA_PER_WAVE + (MASK ? 1 : 0);
  static constexpr int NQ = D / 32 / DSPLIT;    // Q fragments held per wave
  static constexpr int NSB = BN / 16;           // S^T blocks per tile
  static constexpr int NOB = DV / 16 / DSPLIT;  // O^T blocks held per wave
  // partial-S^T exchange buffer: [wave][sb][lane] x f32x4
  static constexpr int XCHG_BYTES = DSPLIT == 2 ? NW * NSB * 64 * 16 : 0;
  static_assert(DSPLIT == 1 || DSPLIT == 2, "DSPLIT");
  static_assert(D % 64 == 0 && DV % (16 * DSPLIT) == 0, "head dims");
  static_assert((K_DMA + V_DMA) % DMA_WAVES == 0, "tile DMA must split evenly over the waves");
  static_assert(VSHARED || (NCH / 2) % 4 == 0, "V layout needs whole instructions per row block");
  static_assert(VSHARED ? DV <= D : DV == D, "value width");
  static_assert(VM_PER_TILE * (STAGES - 1) < 64, "vmcnt range");
  static_assert(!MASK || (NW == 1 && FP8 == 0 && QV == 0 && BN == 32 && !VSHARED),
                "decode mask: one wave, bf16 K and V, 32-key tiles");
  static_assert(FP8 == 0 || (D == 128 && DV == 128 && !VSHARED && DSPLIT == 1),
                "FP8 tiles: D = Dv = 128, separate V, whole head per wave");
  static_assert(QV == 0 || (!VSHARED && DSPLIT == 1 && DV == D), "qv: separate V, Dv = D");
  static_assert(BN == 32 || (FP8 != 0 && BN % 32 == 0 && BN <= 64),
                "tiles of 32 keys, or up to 64 with FP8 codes");
};

template <class C>
struct StreamTile {
  using M = Mfma<16>;
  bf16x8 qf[C::NQ];
  i32x8 q8f;  // FP8: the Q row's codes as the B operand of the 16x16x128 FP8 MFMA
  bf16x8 qvf[C::QV ? C::NQ : 1];  // qv fragments, chunks as those of Q
  f32x4 o[C::NOB];
  float m_ref;
  float l_run;
  int half;  // half of the head dimension this wave holds (0 unless DSPLIT = 2)

  __device__ __forceinline__ void init(int wave) {
    half = C::DSPLIT == 2 ? (wave & 1) : 0;
#pragma unroll
    for (int i = 0; i < C::NOB; ++i) o[i] = f32x4{};
    m_ref = kNegInf;
    l_run = 0.f;
  }

  // Fragment dq of this wave covers the head-dimension chunks (8 elements
  // each) c = (f >> 1) * 8 + 2 * g + (f & 1), f = dq * DSPLIT + half, for
  // lane group g = lane >> 4: all four groups of one fragment read chunks of
  // one parity, so the K reads of the swizzled layout stay conflict-free (a
  // uniform XOR of the row slot only relabels banks). With DSPLIT = 2 the
  // two waves of a pair hold the even and the odd chunks.
  __device__ __forceinline__ static int q_chunk(int dq, int half, int g) {
    const int f = dq * C::DSPLIT + half;
    return (f >> 1) * 8 + 2 * g + (f & 1);
  }

  __device__ __forceinline__ void load_q(const bf16_t* qrow, int lane) {
    const int g = lane >> 4;
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow) v = *reinterpret_cast<const u32x4*>(qrow + q_chunk(i, half, g) * 8);
      qf[i] = as_bf16x8(v);
    }
  }

  // FP8 Q: lane group g holds codes 32 g .. 32 g + 31 of its row (the K
  // fragments below hold the same dims, so the 128-deep products pair them).
  __device__ __forceinline__ void load_q8(const uint8_t* qrow, int lane) {
    const int g = lane >> 4;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
    if (qrow) {
      v0 = *reinterpret_cast<const u32x4*>(qrow + g * 32);
      v1 = *reinterpret_cast<const u32x4*>(qrow + g * 32 + 16);
    }
    q8f = join_i32x8(v0, v1);
  }
  __device__ __forceinline__ static void load_frag8(bf16x8 (&f)[C::NQ], const uint8_t* row,
                                                    int lane) {
    const int g = lane >> 4;
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      u32x2 v = {0u, 0u};
      if (row) v = *reinterpret_cast<const u32x2*>(row + (i * 4 + g) * 8);
      f[i] = fp8x8_to_bf16<C::FP8>(v);
    }
  }
  // qv row (bf16 or FP8 codes), in the fragments of Q
  __device__ __forceinline__ void load_qv(const void* row, int lane) {
    if constexpr (C::QV != 0) {
      if constexpr (C::FP8 != 0) {
        load_frag8(qvf, static_cast<const uint8_t*>(row), lane);
      } else {
        const int g = lane >> 4;
#pragma unroll
        for (int i = 0; i < C::NQ; ++i) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row)
            v = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(row) +
                                                q_chunk(i, 0, g) * 8);
          qvf[i] = as_bf16x8(v);
        }
      }
    }
  }

  // FP8 LDS layouts: tile rows of 128 bytes; the 16-byte unit u of row r is
  // stored at unit u ^ f(r), with
  //   K: f(r) = (r / 2) % 8                    (16 consecutive rows of one block)
  //   V: f(r) = (r / 2) % 4 + 4 ((r / 16) % 2)  (rows 4g..4g+3 and 16+4g..16+4g+3
  //                                             of a 32-key chunk)
  // so that the 32 lanes of each read cycle hit 64 distinct banks. A DMA
  // instruction fills 8 rows: lane l reads 16 bytes of row l / 8 (8 lanes
  // per 128-byte row, coalesced); its unit depends on the instruction's rows
  // through one bit, hence two lane offsets each for K and V.
  __device__ __forceinline__ static int swz8_k(int r) { return (r >> 1) & 7; }
  __device__ __forceinline__ static int swz8_v(int r) {
    return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
  }
  // lane offsets for instructions whose 8-row groups r8 have (r8 & 1) = hi
  // (K) or ((r8 >> 1) & 1) = hi (V); rows `stride` bytes apart
  __device__ __forceinline__ static uint32_t lane_off8(int lane, uint32_t stride, int hi) {
    return (uint32_t)(lane >> 3) * stride + (uint32_t)((lane & 7) ^ (hi * 4 + (lane >> 4))) * 16;
  }
  // Saddr form: kbase(r8) / vbase(r8) give the wave-uniform pointer of tile
  // row 8 r8 (r8 < BN / 8; rows 8 r8 .. 8 r8 + 7 are `stride` bytes apart).
  template <class KB, class VB>
  __device__ __forceinline__ static void dma_tile8_sv(char* stage, KB kbase, VB vbase,
                                                      uint32_t koff0, uint32_t koff1,
                                                      uint32_t voff0, uint32_t voff1) {
    if constexpr (C::K_BYTES > 0) {
#pragma unroll
      for (int r8 = 0; r8 < C::BN / 8; ++r8)
        lds_dma16_sv(kbase(r8), (r8 & 1) ? koff1 : koff0, stage + r8 * 1024);
    }
#pragma unroll
    for (int r8 = 0; r8 < C::BN / 8; ++r8)
      lds_dma16_sv(vbase(r8), ((r8 >> 1) & 1) ? voff1 : voff0,
                   stage + C::K_BYTES + r8 * 1024);
  }
  // Per-lane form: krow(r) / vrow(r) are the byte addresses of tile row r.
  template <class KRow, class VRow>
  __device__ __forceinline__ static void dma_tile8(char* stage, KRow krow, VRow vrow, int lane) {
#pragma unroll
    for (int r8 = 0; r8 < C::BN / 8; ++r8) {
      const int r = r8 * 8 + (lane >> 3);
      if constexpr (C::K_BYTES > 0)
        lds_dma16(krow(r) + ((lane & 7) ^ swz8_k(r)) * 16, stage + r8 * 1024);
      lds_dma16(vrow(r) + ((lane & 7) ^ swz8_v(r)) * 16, stage + C::K_BYTES + r8 * 1024);
    }
  }

  // This wave's share of the DMA of one tile into `stage`. krow(r) / vrow(r)
  // give the global address of the K / V row of key r of the tile (r in
  // [0, BN)); vrow is unused when V shares the K row. With DSPLIT = 2 only
  // waves 0 .. DMA_WAVES-1 issue: one on each SIMD of an 8-wave workgroup
  // (waves w and w+4 share one), so the other wave of that SIMD keeps its
  // MFMA pipe busy while the issuing wave waits for the address unit.
  template <class KRow, class VRow>
  __device__ __forceinline__ static void dma_tile(char* stage, KRow krow, VRow vrow, int wave,
                                                  int lane) {
    if (C::DSPLIT == 2 && wave >= C::DMA_WAVES) return;
    const int dw = C::DMA_WAVES == 1 ? 0 : wave;
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      // dw is 0 for single-DMA-wave workgroups and a uniform (SGPR) value
      // otherwise, so the K/V choice below is a scalar branch or constant.
      const int inst = dw * C::DMA_PER_WAVE + n;
      const bool is_k = C::V_DMA == 0 || (C::DMA_WAVES == 1 ? n < C::K_DMA : inst < C::K_DMA);
      if (is_k) {
        constexpr int IPB = C::NCH / 4;  // instructions per 16-row block
        const int rb = inst / IPB, cq = inst % IPB;
        const int c = cq * 4 + (C::VSHARED ? (lane >> 4) : k_lane_col(lane) / 16);
        const int r = rb * 16 + (int)k_lane_row(lane);
        lds_dma16(krow(r) + c * 8, stage + inst * 1024);
      } else {
        const int vi = inst - C::K_DMA;
        const int blk = 4 * vi + (lane >> 4);
        const int r = (blk / (C::NCH / 2)) * 8 + ((lane & 15) >> 1);
        const int c = (blk % (C::NCH / 2)) * 2 + (lane & 1);
        lds_dma16(vrow(r) + c * 8, stage + C::K_BYTES + vi * 1024);
      }
    }
  }

  using Src = DmaSrc;

  // Byte offset within a stage of the 16-byte unit u of tile row r (K rows,
  // or V rows when is_v): the inverse of the DMA placement (FP8: units of 16
  // codes; bf16: chunks of 8 elements). Used by the DUMP instances that copy
  // staged tiles out for the gather test.
  __device__ __forceinline__ static int lds_unit(bool is_v, int r, int u) {
    if constexpr (C::FP8 != 0) {
      return is_v ? C::K_BYTES + r * 128 + ((u ^ swz8_v(r)) * 16) : r * 128 + ((u ^ swz8_k(r)) * 16);
    } else if constexpr (C::VSHARED) {
      return (r >> 4) * C::NCH * 256 + u * 256 + ((r & 15) ^ ((u & 1) * 8)) * 16;
    } else {
      if (is_v)
        return C::K_BYTES + (r >> 3) * (C::NCH / 2) * 256 + (u >> 1) * 256 + (r & 7) * 32 +
               (u & 1) * 16;
      return (r >> 4) * (C::NCH / 4) * 1024 + (u >> 2) * 1024 + (r & 15) * 64 +
             ((u & 3) ^ ((r & 15) >> 2)) * 16;
    }
  }

  // Lane parts of the saddr form (tile-independent): the byte offset of this
  // lane's 16 bytes from the first row of a 16-row block whose rows are
  // kstride / vstride bytes apart, for the K and the (separate) V DMA.
  __device__ __forceinline__ static uint32_t k_lane_row(int lane) {
    if constexpr (C::VSHARED) return (uint32_t)((lane & 15) ^ (((lane >> 4) & 1) * 8));
    return (uint32_t)(lane >> 2);
  }
  __device__ __forceinline__ static uint32_t k_lane_col(int lane) {
    if constexpr (C::VSHARED) return (uint32_t)(lane >> 4) * 16;
    return (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16;
  }
  __device__ __forceinline__ static uint32_t k_lane_off(int lane, uint32_t kstride) {
    return k_lane_row(lane) * kstride + k_lane_col(lane);
  }
  __device__ __forceinline__ static uint32_t v_lane_off(int lane, uint32_t vstride) {
    return (uint32_t)((lane & 15) >> 1) * vstride + ((lane >> 4) * 2 + (lane & 1)) * 16;
  }

  // The same DMA as dma_tile in the saddr form. Every instruction reads rows
  // of one 16-row block rb of the tile. ksrc(rb, colb) returns the source of
  // a K instruction whose uniform column offset is colb bytes (the lane adds
  // its row and (lane >> 4) * 16); vsrc(rb, sub, colb) that of a V
  // instruction covering rows sub*8 .. sub*8+7 of block rb.
  template <class KSrc, class VSrc>
  __device__ __forceinline__ static void dma_tile_sv(char* stage, KSrc ksrc, VSrc vsrc, int wave) {
    if (C::DSPLIT == 2 && wave >= C::DMA_WAVES) return;
    const int dw = C::DMA_WAVES == 1 ? 0 : wave;
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      const int inst = dw * C::DMA_PER_WAVE + n;
      const bool is_k = C::V_DMA == 0 || (C::DMA_WAVES == 1 ? n < C::K_DMA : inst < C::K_DMA);
      if (is_k) {
        constexpr int IPB = C::NCH / 4;
        const Src a = ksrc(inst / IPB, (inst % IPB) * 64);
        lds_dma16_sv(a.s, a.v, stage + inst * 1024);
      } else {
        constexpr int H = C::NCH / 2;
        const int vi = inst - C::K_DMA;
        const int q = 4 * vi / H;  // 8-row group of the instruction
        const Src a = vsrc(q >> 1, q & 1, ((4 * vi) % H) * 32);
        lds_dma16_sv(a.s, a.v, stage + C::K_BYTES + vi * 1024);
      }
    }
  }

  // S^T for one tile.
  __device__ __forceinline__ void qk(const char* stage, int lane, f32x4 (&s)[C::NSB]) const {
    const int g = lane >> 4;
    if constexpr (C::QV == 2) {  // no Q.K^T path: the scores start at zero
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) s[sb] = f32x4{};
    } else if constexpr (C::FP8) {
      // one 16x16x128 FP8 MFMA per 16-key block on the codes themselves
      // (exact products, fp32 sums): key r = lane % 16 gives units 2 g and
      // 2 g + 1 of its row (codes 32 g .. 32 g + 31, as Q), stored at
      // unit ^ swz8_k(r)
      const int r = lane & 15, sw = swz8_k(r);
      const char* k0 = stage + r * 128 + ((2 * g) ^ sw) * 16;
      const char* k1 = stage + r * 128 + ((2 * g + 1) ^ sw) * 16;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        const i32x8 a = join_i32x8(*reinterpret_cast<const u32x4*>(k0 + sb * 16 * 128),
                                   *reinterpret_cast<const u32x4*>(k1 + sb * 16 * 128));
        s[sb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, q8f, f32x4{}, C::FP8 - 1,
                                                                 C::FP8 - 1, 0, 127, 0, 127);
      }
    } else if constexpr (C::VSHARED) {
      // chunk parity p = f & 1; chunk c = (f >> 1) * 8 + 2g + p sits at
      // c * 256 + ((row % 16) ^ 8p) * 16 within a 16-row block
      const char* kb0 = stage + g * 512 + (lane & 15) * 16;
      const char* kb1 = stage + g * 512 + 256 + ((lane & 15) ^ 8) * 16;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        s[sb] = f32x4{};
#pragma unroll
        for (int dq = 0; dq < C::NQ; ++dq) {
          const int f = dq * C::DSPLIT + half;
          const char* kb = (f & 1) ? kb1 : kb0;
          const u32x4 a = *reinterpret_cast<const u32x4*>(kb + (sb * C::NCH + (f >> 1) * 8) * 256);
          s[sb] = M::mma(as_bf16x8(a), qf[dq], s[sb]);
        }
      }
    } else {
      // chunk c = (f >> 1) * 8 + 2g + p: block c / 4 = 2 (f >> 1) + g / 2,
      // slot (2 (g & 1) + p) ^ ((row % 16) / 4)
      constexpr int IPB = C::NCH / 4;
      const int r = lane & 15, sw = (r >> 2) & 3;
      const char* base = stage + (g >> 1) * 1024 + r * 64;
      const char* kb0 = base + ((2 * (g & 1)) ^ sw) * 16;
      const char* kb1 = base + ((2 * (g & 1) + 1) ^ sw) * 16;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        s[sb] = f32x4{};
#pragma unroll
        for (int dq = 0; dq < C::NQ; ++dq) {
          const int f = dq * C::DSPLIT + half;
          const char* kb = (f & 1) ? kb1 : kb0;
          const u32x4 a =
              *reinterpret_cast<const u32x4*>(kb + (sb * IPB + (f >> 1) * 2) * 1024);
          s[sb] = M::mma(as_bf16x8(a), qf[dq], s[sb]);
        }
      }
    }
  }

  // S^T += ratio * V Qv^T: lane (key r = lane % 16 of block sb, group g)
  // reads the chunks of its value row that its Q fragments hold, from the V
  // layout in place. bf16: chunk c of row r at block (r / 8, c / 2), row
  // r % 8, half c % 2 (two rows per 32-byte line: 2-way bank conflicts,
  // which the HBM-bound decode hides). FP8: 8 codes of unit
  // (2 dq + g / 2) ^ swz8_v(r), half g % 2. ratio = v_descale / k_descale
  // for FP8 (a second accumulator), 1 for bf16 (the same MFMA chain).
  __device__ __forceinline__ void qv_scores(const char* stage, int lane, f32x4 (&s)[C::NSB],
                                            float ratio) const {
    if constexpr (C::QV != 0) {
      const int g = lane >> 4, r = lane & 15;
      const char* vbase = stage + C::K_BYTES;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        const int row = sb * 16 + r;
        if constexpr (C::FP8 != 0) {
          const int fv = swz8_v(row);
          const char* base = vbase + row * 128 + (g & 1) * 8;
          f32x4 t = f32x4{};
#pragma unroll
          for (int dq = 0; dq < C::NQ; ++dq) {
            const u32x2 w =
                *reinterpret_cast<const u32x2*>(base + ((2 * dq + (g >> 1)) ^ fv) * 16);
            t = M::mma(fp8x8_to_bf16<C::FP8>(w), qvf[dq], t);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) s[sb][e] = __builtin_fmaf(t[e], ratio, s[sb][e]);
        } else {
          const char* base = vbase + (row >> 3) * (C::NCH / 2) * 256 + (row & 7) * 32;
#pragma unroll
          for (int dq = 0; dq < C::NQ; ++dq) {
            const int c = q_chunk(dq, 0, g);
            const u32x4 a = *reinterpret_cast<const u32x4*>(base + (c >> 1) * 256 + (c & 1) * 16);
            s[sb] = M::mma(as_bf16x8(a), qvf[dq], s[sb]);
          }
        }
      }
    }
  }

  // DSPLIT = 2: adds the partner wave's partial S^T. The exchange buffer is
  // reused every tile; the caller's per-tile barrier (after lgkmcnt(0))
  // orders the partner's reads of tile i before the writes of tile i+1.
  // Float addition commutes, so both waves of a pair obtain the same sums.
  __device__ __forceinline__ void exchange(char* xchg, int wave, int lane, f32x4 (&s)[C::NSB]) const {
    if constexpr (C::DSPLIT == 2) {
      f32x4* mine = reinterpret_cast<f32x4*>(xchg) + wave * C::NSB * 64 + lane;
      const f32x4* other = reinterpret_cast<const f32x4*>(xchg) + (wave ^ 1) * C::NSB * 64 + lane;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) mine[sb * 64] = s[sb];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own writes done
      barrier_no_fence();
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) s[sb] += other[sb * 64];
    }
  }

  // MASK: s = s * cscale + mask * log2(e) from the stage's mask tile, whose
  // row r (this lane's row, lane % 16) holds the tile's keys 0..BN-1; the
  // scores are then in the scaled domain (softmax with cscale = 1).
  __device__ __forceinline__ static void add_mask(f32x4 (&s)[C::NSB], const char* mbuf,
                                                  float cscale, int lane) {
    const char* mrow = mbuf + (lane & 15) * (C::BN * 2) + (lane >> 4) * 8;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(mrow + sb * 32);  // keys 16 sb + 4 g ..
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
        s[sb][e] = __builtin_fmaf(s[sb][e], cscale, __builtin_bit_cast(float, bits) * kLog2e);
      }
    }
  }

  // Masks the scores of tile-relative keys j with !vis(j).
  template <class Vis>
  __device__ __forceinline__ static void mask(f32x4 (&s)[C::NSB], int lane, Vis vis) {
    const int g = lane >> 4;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!vis(sb * 16 + g * 4 + r)) s[sb][r] = kNegInf;
    }
  }

  // p = 2^(s*c - m) packed to bf16 pairs, l += sum p (float32), with the
  // reference checked after the exponentials (see PrefillTile::softmax): a
  // lane whose probabilities sum to more than kSumLimit, or whose row has no
  // reference yet, sends the wave down the rare path that forms the row
  // maximum across the row's lanes, raises the reference to it (rescaling O
  // and l) and recomputes the tile.
  __device__ __forceinline__ void exps(const f32x4 (&s)[C::NSB], float cscale,
                                       uint32_t (&pk)[C::NSB * 2], float& l) const {
    const float m_use = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[sb][r], cscale, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s[sb][r + 1], cscale, -m_use));
        l = (sb == 0 && r == 0) ? p0 + p1 : l + (p0 + p1);
        pk[sb * 2 + r / 2] = pack_bf16x2(p0, p1);
      }
    }
  }
  __device__ __forceinline__ void softmax(const f32x4 (&s)[C::NSB], float cscale,
                                          uint32_t (&pk)[C::NSB * 2]) {
    float l;
    exps(s, cscale, pk, l);
    if (__ballot(l > kSumLimit || m_ref == kNegInf) != 0) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[sb][r]);
      }
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

  // O^T += V^T P^T for one tile (one 32-key chunk; FP8 tiles loop over theirs).
  __device__ __forceinline__ void pv(const char* stage, int lane, const uint32_t (&pk)[C::NSB * 2]) {
    const int g = lane >> 4, i = lane & 15;
    const u32x4 pv4 = {pk[0], pk[1], pk[2], pk[3]};
    const bf16x8 b = as_bf16x8(pv4);
    if constexpr (C::FP8) {
      // Per 32-key chunk c, the B operand (P) of lane group g holds keys
      // 32c + 4g..4g+3 and 32c + 16+4g..16+4g+3 (the S^T accumulator layout
      // of the chunk's two 16-key blocks); the A operand must list the same
      // keys: lane i of block g receives V[key k_j][dv ob*16 + i],
      // k_j = 32c + (j % 4) + 4g + 16 (j / 4), by addressing row k_{i/2},
      // bytes ob*16 + 8 (i % 2) .. + 7 (swz8_v repeats every 32 rows).
      const int jj = i >> 1;
      const int row = (jj & 3) + 4 * g + 16 * (jj >> 2);
      const int fv = swz8_v(row);
      const char* vb = stage + C::K_BYTES + row * 128 + (i & 1) * 8;
#pragma unroll
      for (int c = 0; c < C::BN / 32; ++c) {
        const u32x4 pc = {pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
        const bf16x8 bc = as_bf16x8(pc);
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob)
          o[ob] = M::mma(fp8x8_to_bf16<C::FP8>(lds_read_tr8(vb + c * 32 * 128 + (ob ^ fv) * 16)),
                         bc, o[ob]);
      }
    } else if constexpr (C::VSHARED) {
      const int par = (i >> 1) & 1;
      const char* vb = stage + (par * 256 + ((g * 4 + (i >> 2)) ^ (par * 8)) * 16 + (i & 1) * 8) +
                       half * C::NOB * 2 * 256;
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) {
        const s16x4 lo = lds_read_tr(reinterpret_cast<const bf16_t*>(vb + (0 * C::NCH + ob * 2) * 256));
        const s16x4 hi = lds_read_tr(reinterpret_cast<const bf16_t*>(vb + (1 * C::NCH + ob * 2) * 256));
        o[ob] = M::mma(join_bf16x8(lo, hi), b, o[ob]);
      }
    } else {
      const char* vb = stage + C::K_BYTES + ((g >> 1) * (C::NCH / 2) * 256 + (g & 1) * 128 + i * 8);
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) {
        const s16x4 lo = lds_read_tr(reinterpret_cast<const bf16_t*>(vb + (0 * (C::NCH / 2) + ob) * 256));
        const s16x4 hi = lds_read_tr(reinterpret_cast<const bf16_t*>(vb + (2 * (C::NCH / 2) + ob) * 256));
        o[ob] = M::mma(join_bf16x8(lo, hi), b, o[ob]);
      }
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

  template <class OutT>
  __device__ __forceinline__ void store(OutT* orow, float inv, int lane) const {
    const int g = lane >> 4;
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
      const int col = (half * C::NOB + ob) * 16 + g * 4;
      const float a0 = o[ob][0] * inv, a1 = o[ob][1] * inv;
      const float a2 = o[ob][2] * inv, a3 = o[ob][3] * inv;
      if constexpr (sizeof(OutT) == 2) {
        const u32x2 w = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
      } else {
        const f32x4 w = {a0, a1, a2, a3};
        *reinterpret_cast<f32x4*>(orow + col) = w;
      }
    }
  }
};

// Streams tiles [0, ntiles) through the LDS ring `ring` (STAGES buffers of
// STAGE_BYTES). issue(stage_ptr, t) enqueues the DMA of tile t; compute(t,
// stage_ptr) consumes it. Exactly VM_PER_TILE DMA instructions per wave per
// tile must be issued by issue(). Waits only for the tile about to be read.
template <class C, class Issue, class Compute>
__device__ __forceinline__ void stream_tiles(char* ring, int ntiles, Issue issue, Compute compute) {
  auto stage = [&](int t) { return ring + (t % C::STAGES) * C::STAGE_BYTES; };
#pragma unroll
  for (int t = 0; t < C::STAGES - 1; ++t)
    if (t < ntiles) issue(stage(t), t);
  for (int i = 0; i < ntiles; ++i) {
    // tiles issued after tile i: min(ntiles-1-i, STAGES-2)
    const int after = min(ntiles - 1 - i, C::STAGES - 2);
    if constexpr (C::STAGES >= 4) {
      if (after >= 2) wait_vmcnt<2 * C::VM_PER_TILE>();
      else if (after == 1) wait_vmcnt<C::VM_PER_TILE>();
      else wait_vmcnt<0>();
    } else if constexpr (C::STAGES == 3) {
      if (after >= 1) wait_vmcnt<C::VM_PER_TILE>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own LDS reads of tile i-1 retired
    barrier_no_fence();                  // tile i visible; every wave is done with tile i-1
    if (i + C::STAGES - 1 < ntiles) issue(stage(i + C::STAGES - 1), i + C::STAGES - 1);
    compute(i, stage(i));
  }
}

// DUMP instances (gather test): copies rows [0, nrows) of a staged tile out
// of LDS, un-swizzled: unit u (16 bytes) of row r is read at stage +
// off(r, u) and written to dst(r) + 16 u. Every thread of the workgroup takes
// part; the stores are waited for before returning, so that the vmcnt waits
// of the tile loop count only the DMA.
template <int UNITS, class Off, class Dst>
__device__ __forceinline__ void dump_rows(const char* stage, int nrows, Off off, Dst dst, int tid,
                                          int nthreads) {
  for (int e = tid; e < nrows * UNITS; e += nthreads) {
    const int r = e / UNITS, u = e % UNITS;
    *reinterpret_cast<u32x4*>(dst(r) + u * 16) = *reinterpret_cast<const u32x4*>(stage + off(r, u));
  }
  wait_vmcnt<0>();
}

}  // namespace attn
