// Device helpers shared by the gfx950 attention kernels: vector types, bf16
// conversion, MFMA wrappers with their lane layouts, wave reductions and the
// transposing LDS read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <utility>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest even (values are finite here).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 pair (lo in bits 0..15), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// --- MFMA layouts (checked on gfx950 hardware) ------------------------------
// 32x32x16 bf16: A lane l holds A[m=l%32][k=(l/32)*8+j], B lane l holds
//   B[k=(l/32)*8+j][n=l%32], C lane l reg r holds C[m=(r/4)*8+(l/32)*4+r%4][n=l%32].
// 16x16x32 bf16: A lane l holds A[m=l%16][k=(l/16)*8+j], B likewise with n,
//   C lane l reg r holds C[m=(l/16)*4+r][n=l%16].
template <int R> struct Mfma;

template <> struct Mfma<32> {
  static constexpr int R = 32;      // query rows per wave (the N side of S^T = K Q^T)
  static constexpr int KSTEP = 16;  // reduction depth of one instruction
  static constexpr int SB = 32;     // keys per S^T block (the M side)
  static constexpr int SREG = 16;   // accumulator registers per block
  static constexpr int PVK = 16;    // keys consumed by one P.V instruction
  static constexpr int NGRP = 2;    // lane groups sharing one row
  typedef f32x16 acc_t;
  __device__ static __forceinline__ int row(int l) { return l & 31; }
  __device__ static __forceinline__ int grp(int l) { return l >> 5; }
  // block-relative M index (key, or value column) held in register r by lane group g
  __device__ static __forceinline__ constexpr int mrow(int g, int r) { return (r >> 2) * 8 + g * 4 + (r & 3); }
  __device__ static __forceinline__ acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // column offset of this lane's 16-lane block inside an A-operand tile
  __device__ static __forceinline__ int tr_col(int l) { return ((l >> 4) & 1) * 16; }
  // Reductions over the two lane groups of a row (lanes l and l ^ 32):
  // v_permlane32_swap exchanges the upper half of its first operand with the
  // lower half of its second, so with both set to x the two results hold
  // x[l] and x[l ^ 32] (in some order) in every lane.
  __device__ static __forceinline__ float group_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  }
  __device__ static __forceinline__ float group_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  }
};

template <> struct Mfma<16> {
  static constexpr int R = 16;
  static constexpr int KSTEP = 32;
  static constexpr int SB = 16;
  static constexpr int SREG = 4;
  static constexpr int PVK = 32;
  static constexpr int NGRP = 4;
  typedef f32x4 acc_t;
  __device__ static __forceinline__ int row(int l) { return l & 15; }
  __device__ static __forceinline__ int grp(int l) { return l >> 4; }
  __device__ static __forceinline__ constexpr int mrow(int g, int r) { return g * 4 + r; }
  __device__ static __forceinline__ acc_t mma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int tr_col(int) { return 0; }
  // Reductions over the four lane groups of a row (lanes l ^ 16, l ^ 32):
  // v_permlane16_swap pairs 16-lane rows 0<->1 and 2<->3, then
  // v_permlane32_swap pairs the two halves (see Mfma<32>).
  __device__ static __forceinline__ float group_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    x = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    return Mfma<32>::group_max(x);
  }
  __device__ static __forceinline__ float group_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    x = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    return Mfma<32>::group_sum(x);
  }
};

// --- LDS access ---------------------------------------------------------------
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing read (ds_read_b64_tr_b16). Within each block of 16 lanes, lane i
// must address row (i/4) and column 4*(i%4) of a 4 x 16 tile of 16-bit
// elements; it then receives column i of that tile, rows 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two 16-byte halves as one 8-register MFMA operand (FP8 codes).
__device__ __forceinline__ i32x8 join_i32x8(u32x4 a, u32x4 b) {
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2],
               (int)b[3]};
}

// Transposing read of 8-bit elements (ds_read_b64_tr_b8). Within each block of
// 16 lanes, lane m addresses 8 bytes; lane i receives byte i % 8 of the bytes
// lane 2j + i/8 addressed, for j = 0..7 (so if lane m addresses row m/2,
// bytes 8(m%2) .. 8(m%2)+7 of an 8 x 16 byte tile, lane i gets column i).
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p)));
}

// Eight FP8 codes (bytes 0..7 of w) -> eight bfloat16 values, exactly (every
// e4m3 / e5m2 value is a bfloat16 value): v_cvt_scalef32_pk_bf16_{fp8,bf8}
// with scale 1, two codes per instruction. FMT 1 = e4m3fn, 2 = e5m2.
template <int FMT>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 w) {
  auto cvt = [](uint32_t x, auto hi) {
    if constexpr (FMT == 1)
      return __builtin_bit_cast(uint32_t,
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, decltype(hi)::value));
    else
      return __builtin_bit_cast(uint32_t,
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x, 1.0f, decltype(hi)::value));
  };
  const u32x4 r = {cvt(w[0], std::false_type{}), cvt(w[0], std::true_type{}),
                   cvt(w[1], std::false_type{}), cvt(w[1], std::true_type{})};
  return as_bf16x8(r);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, with i usable as a
// constant expression (schedule-group sizes must be constants).
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Lane id recomputed where it is used (volatile, so not hoisted out of the
// key loop): lane-dependent addresses are then rebuilt with a few VALU
// operations per tile instead of occupying registers across the loop, which
// near the register limit would be spilled and reloaded through scratch
// memory (and scratch loads share vmcnt with the tile DMA).
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ bf16x8 join_bf16x8(s16x4 lo, s16x4 hi) {
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace attn
