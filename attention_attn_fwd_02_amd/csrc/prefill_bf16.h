// Prefill tile engine for gfx950 (32 query rows per wave, 32x32 MFMA), for
// bfloat16 inputs or FP8 codes (FP8 = 1 e4m3fn, 2 e5m2).
//
// Per workgroup: NW waves x 32 rows share one key sequence. Key tiles of BN
// rows are copied HBM/L2 -> LDS by global_load_lds_dwordx4 (no register
// staging) through a ring of STAGES buffers, STAGES-1 tiles in flight.
//
// LDS layouts (16-byte units, c = chunk index along the head dimension). The
// LDS has 64 banks of 4 bytes (256 B per cycle) and serves 16 lanes of a
// 16-byte read per cycle; both layouts put the 16 lanes of every read in 64
// distinct banks:
//   K: [row / 16][c / 4][row % 16][(c % 4) ^ ((row % 16) / 4)]
//      an A-operand read (16 consecutive rows at one chunk) takes the 16
//      combinations of row % 4 (16-bank group) and the swizzled slot
//      (4-bank group).
//   V: [row / 8][c / 4][(row / 4) % 2][row % 4][c % 4]
//      the two 16-lane blocks of a ds_read_b64_tr_b16 that share a cycle
//      (4 rows x 32 B each) interleave into 256 contiguous bytes.
// Every DMA instruction writes 1 KB contiguously (64 lanes x 16 B). Its
// global reads are coalesced: each group of 4 consecutive lanes reads one
// 64-byte row segment (K: 16 rows x 64 B per instruction; V: 8 rows x 2
// segments).
// All MFMA operand addresses are a per-lane base plus a compile-time offset.
//
// FP8 tiles (D = 128: rows of 128 bytes, 8 units): unit u of row r is stored
// at u ^ f(r) within the row, with
//   K: f(r) = (r / 2) % 8            (16 rows of one A-operand read cycle)
//   V: f(r) = 2 ((r / 2) % 2) + 4 ((r / 8) % 2)
//      (the 32 lanes of a ds_read_b64_tr_b8 cycle: rows 0-3 and 8-11, or
//      4-7 and 12-15, of a 16-key chunk, two units each)
// which puts every read cycle in 64 distinct banks. A DMA instruction fills 8
// rows, 8 lanes per 128-byte row (coalesced); f depends on the instruction
// only through its parity. S^T = K Q^T runs on the FP8 MFMA (32x32x64,
// products exact, fp32 sums); V widens to bfloat16 exactly after the
// transposing read, and P.V is the bfloat16 path's.
//
// Softmax runs in the base-2 domain on unscaled scores s: p = 2^(s*c - m),
// c = scale*log2(e). The reference m is checked after the exponentials, from
// the sums of p each lane forms anyway (see PrefillTile::softmax), so no row
// maximum is formed on the common path and the O/l rescale is rare; the
// final O = acc / l and LSE = (m + log2 l) ln 2 are exact for any reference m.
#pragma once
#include "device_common.h"

namespace attn {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// ATTN_LDS_POISON (a debug build, off by default): before each DMA
// instruction the issuing lanes fill their 16 bytes of its LDS destination
// with all-ones bits (NaN as bfloat16, float32 and both FP8 formats) and wait
// for those writes, so that a read of a stage before its DMA has landed (a
// missing vmcnt wait or barrier) turns the results into NaN instead of
// silently reusing the previous tile's data.
#ifndef ATTN_LDS_POISON
#define ATTN_LDS_POISON 0
#endif
__device__ __forceinline__ void lds_poison16(void* lds_dst_uniform) {
  if constexpr (ATTN_LDS_POISON != 0) {
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4_*>(static_cast<char*>(lds_dst_uniform) + lane * 16) =
        u32x4_{~0u, ~0u, ~0u, ~0u};
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the fill lands before the DMA's data
  }
}

// 16 bytes per lane from gsrc into LDS at lds_dst_uniform + 16*lane
// (global_load_lds_dwordx4; the LDS base goes through M0 and must be
// wave-uniform). The instruction has no register results. It is issued from
// asm so that the compiler does not add conservative vmcnt waits before LDS
// reads of the other buffer: callers wait on vmcnt themselves before the
// barrier that publishes a tile.
__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_dst_uniform) {
  lds_poison16(lds_dst_uniform);
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_ptr)(lds_dst_uniform);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}

// Same DMA with the source split into a wave-uniform base (SGPR pair) and the
// lane's 32-bit byte offset from it (the global "saddr" form), so the
// per-lane part can be computed once and reused for every tile.
__device__ __forceinline__ void lds_dma16_sv(const void* sbase_uniform, uint32_t voff,
                                             void* lds_dst_uniform) {
  lds_poison16(lds_dst_uniform);
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_ptr)(lds_dst_uniform);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase_uniform), "{m0}"(m0)
               : "memory");
}

// Two wave-uniform 32-bit loads through the scalar cache, waited for inside
// the asm. The compiler would otherwise emit vector loads here (the DMA asm
// above clobbers memory), and its vmcnt wait for them would also wait for
// every DMA in flight.
__device__ __forceinline__ void sload2_uniform(const int* p0, const int* p1, int& v0, int& v1) {
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1)
      : "s"(p0), "s"(p1));
}

// s_waitcnt with vmcnt = n and the other counters left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): the caller
// has already waited for exactly the memory operations the other waves need
// (LDS-DMA of the current tile), so DMA for the next tile stays in flight.
// The empty asm with a memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Bound on one lane's sum of p over a tile before the reference is raised:
// a sum above it means some p > kSumLimit / 16 = 2^8 (and p < 2^12 always,
// far from float32 and bfloat16 overflow).
constexpr float kSumLimit = 4096.0f;

template <int D_, int NW_, int BN_, int MIN_WAVES_ = 2, int STAGES_ = 3, int FP8_ = 0>
struct PrefillCfg {
  static constexpr int D = D_, DV = D_, NW = NW_, BN = BN_;
  static constexpr int MIN_WAVES = MIN_WAVES_;  // waves per SIMD the registers must allow
  static constexpr int STAGES = STAGES_;        // K+V tile buffers in the LDS ring
  static constexpr int FP8 = FP8_;              // 0 bfloat16, 1 e4m3fn, 2 e5m2 codes
  static constexpr int EB = FP8 ? 1 : 2;        // bytes per element
  static constexpr int R = 32;
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW * R;
  static constexpr int NCH = D * EB / 16;              // 16-byte chunks per row
  static constexpr int TILE_BYTES = BN * D * EB;       // one K (or V) tile
  static constexpr int DMA_PER_TILE = TILE_BYTES / 1024;
  static constexpr int DMA_PER_WAVE = DMA_PER_TILE / NW;  // per wave, per K or V tile
  static constexpr int NOFF = FP8 ? DMA_PER_WAVE : 1;     // DMA lane offsets per wave
  static constexpr int NQ = FP8 ? D / 64 : D / 16;     // Q fragments per row
  static constexpr int NSB = BN / 32;                  // S^T blocks per tile
  static constexpr int NPC = BN / 16;                  // P chunks per tile
  static constexpr int NOB = DV / 32;                  // O^T blocks
  static_assert(DMA_PER_TILE % NW == 0, "tile must split evenly over the waves");
  static_assert(BN % 32 == 0 && D % 64 == 0, "shape");
  static_assert(FP8 == 0 || D == 128, "FP8 tiles: D = 128");
};

// QV: the tile also holds a second query qv (Dv = D wide), scored against
// the V rows of each tile (a copy of V in the K layout) and added to Q.K^T.
template <class C, bool QV = false>
struct PrefillTile {
  using M = Mfma<32>;
  // bfloat16: fragment i = dims 16 i + 8 g .. + 7; FP8: fragment m = dims
  // 64 m + 32 g .. + 31 (the B operand of one 32x32x64 FP8 MFMA)
  using QFrag = std::conditional_t<(C::FP8 != 0), i32x8, bf16x8>;
  QFrag qf[C::NQ];
  QFrag qvf[QV ? C::NQ : 1];
  f32x16 o[C::NOB];
  float m_ref;  // reference max (base-2 scaled domain), -inf until a key is seen
  float m_use;  // exponent offset: m_ref, or 0 while m_ref is -inf
  float l_run;  // this lane's share of sum 2^(s*c - m_ref)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < C::NOB; ++i) o[i] = f32x16{};
    m_ref = kNegInf;
    m_use = 0.f;
    l_run = 0.f;
  }

  // One query row (bf16 elements or FP8 codes) into B-operand fragments.
  __device__ __forceinline__ static void load_frags(QFrag (&f)[C::NQ], const void* row,
                                                    int lane) {
    const int g = lane >> 5;
    if constexpr (C::FP8 != 0) {
      const uint8_t* qrow = static_cast<const uint8_t*>(row);
#pragma unroll
      for (int m = 0; m < C::NQ; ++m) {
        u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
        if (qrow) {
          v0 = *reinterpret_cast<const u32x4*>(qrow + m * 64 + g * 32);
          v1 = *reinterpret_cast<const u32x4*>(qrow + m * 64 + g * 32 + 16);
        }
        f[m] = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                     (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
      }
    } else {
      const bf16_t* qrow = static_cast<const bf16_t*>(row);
#pragma unroll
      for (int i = 0; i < C::NQ; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qrow) v = *reinterpret_cast<const u32x4*>(qrow + i * 16 + g * 8);
        f[i] = as_bf16x8(v);
      }
    }
  }
  __device__ __forceinline__ void load_q(const void* qrow, int lane) { load_frags(qf, qrow, lane); }
  __device__ __forceinline__ void load_qv(const void* row, int lane) {
    if constexpr (QV) load_frags(qvf, row, lane);
  }

  // FP8 unit swizzles (see the header comment)
  __device__ __forceinline__ static constexpr int fk8(int r) { return (r >> 1) & 7; }
  __device__ __forceinline__ static constexpr int fv8(int r) {
    return ((r >> 1) & 1) * 2 + ((r >> 3) & 1) * 4;
  }
  __device__ __forceinline__ static i32x8 join8(u32x4 a, u32x4 b) {
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                 (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  }
  __device__ __forceinline__ static f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
    // operand formats: 0 = e4m3, 1 = e5m2; block scales 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, C::FP8 - 1, C::FP8 - 1, 0,
                                                           127, 0, 127);
  }

  // Byte offset within a K (VLAYOUT = false) or V tile buffer of the 16-byte
  // unit u of tile row r: the inverse of the DMA placement below (bf16: chunk
  // u of 8 elements; FP8: unit u of 16 codes). Used by the DUMP instance that
  // copies staged tiles out for the gather test.
  template <bool VLAYOUT>
  __device__ __forceinline__ static int lds_unit(int r, int u) {
    if constexpr (C::FP8 != 0) return r * 128 + ((u ^ (VLAYOUT ? fv8(r) : fk8(r))) * 16);
    if constexpr (!VLAYOUT)
      return (r >> 4) * (C::NCH / 4) * 1024 + (u >> 2) * 1024 + (r & 15) * 64 +
             ((u & 3) ^ ((r & 15) >> 2)) * 16;
    return (r >> 3) * (C::NCH / 4) * 512 + (u >> 2) * 512 + ((r >> 2) & 1) * 256 + (r & 3) * 64 +
           (u & 3) * 16;
  }

  // Issues this wave's share of the DMA for one K or V tile whose key rows
  // start at row(0); row(r) returns the global byte address of key r's row
  // (always a valid address). V tiles use the V layout.
  template <bool VLAYOUT, class RowPtr>
  __device__ __forceinline__ static void dma_tile(char* buf, RowPtr row, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      const int inst = wave * C::DMA_PER_WAVE + n;
      if constexpr (C::FP8 != 0) {
        const int r = inst * 8 + (lane >> 3);
        const int f = VLAYOUT ? fv8(r) : fk8(r);
        lds_dma16(row(r) + ((lane & 7) ^ f) * 16, buf + inst * 1024);
        continue;
      }
      int r, c;
      if constexpr (!VLAYOUT) {
        // instruction -> (16-row block, 4 chunks); 4 lanes per row, the
        // chunk slot swizzled by the row's quarter of the block
        constexpr int IPB = C::NCH / 4;
        const int rb = inst / IPB, cq = inst % IPB;
        r = rb * 16 + (lane >> 2);
        c = cq * 4 + ((lane & 3) ^ ((lane >> 4) & 3));
      } else {
        // instruction -> two 512 B blocks (8 rows x 4 chunks); lane -> (row, chunk)
        const int blk = 2 * inst + (lane >> 5);
        r = (blk / (C::NCH / 4)) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 2) & 3);
        c = (blk % (C::NCH / 4)) * 4 + (lane & 3);
      }
      lds_dma16(row(r) + c * 16, buf + inst * 1024);
    }
  }

  // The same DMA in the saddr form for a tile whose BN rows are all valid
  // and row_bytes apart from `tile` (a wave-uniform pointer to row 0):
  // every instruction's uniform part (its row block and chunk group) goes
  // into the scalar base and the lane's part is lane_off, computed once by
  // dma_lane_off.
  // FP8: the offset also depends on the parity of the instruction (par).
  template <bool VLAYOUT>
  __device__ __forceinline__ static uint32_t dma_lane_off(int lane, uint32_t row_bytes,
                                                          int par = 0) {
    if constexpr (C::FP8 != 0) {
      const int f = VLAYOUT ? ((lane >> 4) & 1) * 2 + par * 4 : par * 4 + (lane >> 4);
      return (uint32_t)(lane >> 3) * row_bytes + (uint32_t)((lane & 7) ^ f) * 16;
    }
    if constexpr (!VLAYOUT)
      return (uint32_t)(lane >> 2) * row_bytes + ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
    return (uint32_t)(((lane >> 4) & 1) * 4 + ((lane >> 2) & 3)) * row_bytes +
           ((lane >> 5) * 4 + (lane & 3)) * 16;
  }
  // blk(rb): wave-uniform byte pointer of tile row 16 rb; rows of one
  // 16-row block are row_bytes apart (different blocks may lie on different
  // pages).
  // Lane offsets of this wave's instructions, computed once.
  template <bool VLAYOUT>
  __device__ __forceinline__ static void dma_lane_offs(int lane, uint32_t row_bytes, int wave,
                                                       uint32_t (&off)[C::NOFF]) {
#pragma unroll
    for (int n = 0; n < C::NOFF; ++n)
      off[n] = dma_lane_off<VLAYOUT>(lane, row_bytes, (wave * C::DMA_PER_WAVE + n) & 1);
  }
  template <bool VLAYOUT, class Blk>
  __device__ __forceinline__ static void dma_tile_blk(char* buf, Blk blk, long row_bytes,
                                                      const uint32_t (&lane_off)[C::NOFF],
                                                      int wave) {
#pragma unroll
    for (int n = 0; n < C::DMA_PER_WAVE; ++n) {
      const int inst = wave * C::DMA_PER_WAVE + n;
      const char* src;
      if constexpr (C::FP8 != 0) {
        src = blk(inst >> 1) + (inst & 1) * 8 * row_bytes;  // rows 8 inst .. 8 inst + 7
        lds_dma16_sv(src, lane_off[n], buf + inst * 1024);
        continue;
      }
      if constexpr (!VLAYOUT) {
        constexpr int IPB = C::NCH / 4;
        src = blk(inst / IPB) + (inst % IPB) * 64;
      } else {
        // blk = 2 inst + (lane >> 5); NCH / 4 is even, so the 8-row group
        // (2 inst) / (NCH / 4) is uniform
        constexpr int BPR = C::NCH / 4;
        const int q8 = (2 * inst) / BPR;
        src = blk(q8 >> 1) + (q8 & 1) * 8 * row_bytes + ((2 * inst) % BPR) * 64;
      }
      lds_dma16_sv(src, lane_off[0], buf + inst * 1024);
    }
  }
  template <bool VLAYOUT>
  __device__ __forceinline__ static void dma_tile_sv(char* buf, const char* tile, long row_bytes,
                                                     const uint32_t (&lane_off)[C::NOFF],
                                                     int wave) {
    dma_tile_blk<VLAYOUT>(
        buf, [&](int rb) { return tile + rb * 16 * row_bytes; }, row_bytes, lane_off, wave);
  }

  // S^T = K Q^T for one tile. Lane (key k = lane % 32, group g = lane / 32)
  // reads chunk 2 dq + g of key k: block (k / 16, dq / 2), row k % 16, slot
  // (2 (dq % 2) + g) ^ ((k % 16) / 4); the two slot patterns of even and odd
  // dq give two per-lane bases.
  __device__ __forceinline__ void qk(const char* kbuf, int lane, f32x16 (&s)[C::NSB]) const {
    qk_frags<false>(kbuf, qf, lane, s, 1.f);
  }
  // S^T += ratio * V Qv^T from the copy of V in the K layout at vkbuf (bf16:
  // the same MFMA chain, ratio 1; FP8: a second accumulator, ratio =
  // v_descale / k_descale, as the score scale carries k_descale).
  __device__ __forceinline__ void qv_scores(const char* vkbuf, int lane, f32x16 (&s)[C::NSB],
                                            float ratio) const {
    if constexpr (QV) qk_frags<true>(vkbuf, qvf, lane, s, ratio);
  }
  // ACC = false: S^T = K F^T; ACC = true: S^T += ratio * K F^T.
  template <bool ACC>
  __device__ __forceinline__ void qk_frags(const char* kbuf, const QFrag (&fr)[C::NQ], int lane,
                                           f32x16 (&s)[C::NSB], float ratio) const {
    if constexpr (C::FP8 != 0) {
      // key k = lane % 32 of block sb: dims 64 m + 32 g .. + 31 are units
      // 4 m + 2 g + t (t = 0, 1) of its row, stored at unit ^ fk8(k); A and B
      // hold the same dims in the same registers, so any assignment of the
      // 64 reduction indices to registers gives the same dot products
      const int k = lane & 31, g = lane >> 5, f = fk8(k);
      const char* base = kbuf + k * 128;
      const char* kp[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) kp[m][t2] = base + ((4 * m + 2 * g + t2) ^ f) * 16;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
        i32x8 kf[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
          kf[m] = join8(*reinterpret_cast<const u32x4*>(kp[m][0] + sb * 32 * 128),
                        *reinterpret_cast<const u32x4*>(kp[m][1] + sb * 32 * 128));
        f32x16 acc = f32x16{};
#pragma unroll
        for (int m = 0; m < 2; ++m) acc = mma8(kf[m], fr[m], acc);
        if constexpr (ACC) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s[sb][e] = __builtin_fmaf(acc[e], ratio, s[sb][e]);
        } else {
          s[sb] = acc;
        }
      }
      return;
    } else {
    constexpr int IPB = C::NCH / 4;
    const int g = lane >> 5, r = lane & 15, sw = (r >> 2) & 3;
    const char* base = kbuf + ((lane >> 4) & 1) * IPB * 1024 + r * 64;
    const char* kb0 = base + (g ^ sw) * 16;
    const char* kb1 = base + ((2 + g) ^ sw) * 16;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
      bf16x8 kf[C::NQ];
#pragma unroll
      for (int dq = 0; dq < C::NQ; ++dq)
        kf[dq] = as_bf16x8(*reinterpret_cast<const u32x4*>((dq & 1 ? kb1 : kb0) +
                                                           (sb * 2 * IPB + dq / 2) * 1024));
      if constexpr (!ACC) s[sb] = f32x16{};
#pragma unroll
      for (int dq = 0; dq < C::NQ; ++dq) s[sb] = M::mma(kf[dq], fr[dq], s[sb]);
    }
    }
  }

  // Masks the scores of keys this lane's row must not see: key = tile key
  // index (sb * 32 + mrow(g, r)); the row sees keys lo <= key <= hi (tile
  // indices, possibly out of range). HAS_LO = false skips the lower bound.
  template <bool HAS_LO>
  __device__ __forceinline__ static void mask(f32x16 (&s)[C::NSB], int lane, int lo, int hi) {
    const int g4 = (lane >> 5) * 4;  // mrow(g, r) = (r/4)*8 + 4g + r%4
    const int h = hi - g4, l = lo - g4;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = sb * 32 + (r >> 2) * 8 + (r & 3);
        bool hide = k > h;
        if constexpr (HAS_LO) hide |= k < l;
        if (hide) s[sb][r] = kNegInf;
      }
    }
  }

  // Additive mask: s <- s * c + mask * log2(e) (the base-2 scaled domain).
  // The wave's mask band in LDS is row-major, 32 rows x BN bf16; this lane
  // reads its row's keys mrow(g, r) in four 8-byte groups per 32-key block.
  __device__ __forceinline__ static void add_mask(f32x16 (&s)[C::NSB], const char* mbuf,
                                                  float cscale, int lane) {
    const int g = lane >> 5;
    const char* mrow = mbuf + (lane & 31) * (C::BN * 2) + g * 8;
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int q8 = 0; q8 < 4; ++q8) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(mrow + (sb * 32 + q8 * 8) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
          const int r = q8 * 4 + e;                  // mrow(g, r) = 8 q8 + 4 g + e
          s[sb][r] = __builtin_fmaf(s[sb][r], cscale,
                                    __builtin_bit_cast(float, bits) * kLog2e);
        }
      }
    }
  }

  // p = 2^(s*c - m) for one tile, packed to bf16 pairs in B-operand order,
  // and l += sum p in float32 (summing the bf16-rounded p instead would move
  // LSE by up to 2^-8 on rows with few keys).
  //
  // The reference m is checked after the exponentials rather than before,
  // so no row maximum is formed on the common path: a lane whose 16
  // probabilities sum to more than kSumLimit (so one of them exceeds 2^8),
  // or whose row has no reference yet, sends the wave down the rare path,
  // which forms the row maximum across the lane pair, raises the reference
  // to it (rescaling O and l) and recomputes the tile. The final
  // O = acc / l and LSE = m + log2 l are exact for any reference.
  __device__ __forceinline__ void exps(const f32x16 (&s)[C::NSB], float cscale,
                                       uint32_t (&pk)[C::NSB * 8], float& l0, float& l1) const {
#pragma unroll
    for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(s[sb][r], cscale, -m_use));
        const float p1 = fast_exp2(__builtin_fmaf(s[sb][r + 1], cscale, -m_use));
        pk[sb * 8 + r / 2] = pack_bf16x2(p0, p1);
        float& l = ((r >> 1) & 1) ? l1 : l0;
        l = (sb == 0 && r < 4) ? p0 + p1 : l + (p0 + p1);
      }
    }
  }
  __device__ __forceinline__ void softmax(const f32x16 (&s)[C::NSB], float cscale,
                                          uint32_t (&pk)[C::NSB * 8]) {
    float l0, l1;
    exps(s, cscale, pk, l0, l1);
    if (__ballot(l0 + l1 > kSumLimit || m_ref == kNegInf) != 0) {
      float mx = kNegInf;
#pragma unroll
      for (int sb = 0; sb < C::NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      }
      const float rmx = M::group_max(mx) * cscale;
      if (rmx > m_ref) {
        const float alpha = fast_exp2(m_ref - rmx);  // m_ref = -inf -> 0
        m_ref = rmx;
        m_use = rmx;
        l_run *= alpha;
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob) o[ob] *= alpha;
      }
      exps(s, cscale, pk, l0, l1);
    }
    l_run += l0 + l1;
  }

  // O^T += V^T P^T with V read transposed.
  __device__ __forceinline__ void pv(const char* vbuf, int lane, const uint32_t (&pk)[C::NSB * 8]) {
    if constexpr (C::FP8 != 0) {
      // P (B operand) of lane group g holds, for k-index j = 0..7 of chunk
      // c, key 16 c + 8 (j / 4) + 4 g + j % 4. Lane i of each 16-lane block
      // must receive V[key_j][dv] for dv = 32 ob + 16 hb + i: the
      // transposing read gives it byte i % 8 of lane 2 j + i / 8, so lane m
      // addresses row key_{m/2}, bytes 32 ob + 16 hb + 8 (m % 2) .. + 7.
      const int g = lane >> 5, hb = (lane >> 4) & 1, i = lane & 15, jj = i >> 1;
      const int row = (jj >> 2) * 8 + 4 * g + (jj & 3);
      const int fh = fv8(row) >> 1;  // fv8 is even: it flips units in pairs
      const char* vb = vbuf + row * 128 + hb * 16 + (i & 1) * 8;
#pragma unroll
      for (int c = 0; c < C::NPC; ++c) {
        const u32x4 pv4 = {pk[c * 4], pk[c * 4 + 1], pk[c * 4 + 2], pk[c * 4 + 3]};
        const bf16x8 b = as_bf16x8(pv4);
#pragma unroll
        for (int ob = 0; ob < C::NOB; ++ob)
          o[ob] = M::mma(fp8x8_to_bf16<C::FP8>(lds_read_tr8(vb + c * 16 * 128 + (ob ^ fh) * 32)),
                         b, o[ob]);
      }
      return;
    }
    const int g = lane >> 5;
    const char* vb = vbuf + (g * 256 + ((lane & 15) >> 2) * 64 + ((lane >> 4) & 1) * 32 + (lane & 3) * 8);
#pragma unroll
    for (int c = 0; c < C::NPC; ++c) {
      const u32x4 pv4 = {pk[c * 4], pk[c * 4 + 1], pk[c * 4 + 2], pk[c * 4 + 3]};
      const bf16x8 b = as_bf16x8(pv4);
#pragma unroll
      for (int ob = 0; ob < C::NOB; ++ob) {
        const s16x4 lo = lds_read_tr(reinterpret_cast<const bf16_t*>(
            vb + ((c * 2 + 0) * (C::NCH / 4) + ob) * 512));
        const s16x4 hi = lds_read_tr(reinterpret_cast<const bf16_t*>(
            vb + ((c * 2 + 1) * (C::NCH / 4) + ob) * 512));
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

  __device__ __forceinline__ void store(bf16_t* orow, float inv, int lane) const {
    const int g = lane >> 5;
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int col = ob * 32 + M::mrow(g, r);
        const u32x2 w = {pack_bf16x2(o[ob][r] * inv, o[ob][r + 1] * inv),
                         pack_bf16x2(o[ob][r + 2] * inv, o[ob][r + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
    }
  }
};

}  // namespace attn
