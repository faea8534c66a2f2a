// Tiled online-softmax attention engine for gfx950 (bf16 MFMA, fp32 accumulate).
//
// One workgroup owns NW*R query rows that share one key sequence; each wave
// owns R rows. Keys are consumed in tiles of BN rows staged through LDS:
//
//   S^T = K Q^T   (A = K tile from LDS, B = this wave's Q rows in registers)
//   online softmax per row in the base-2 domain: m' = max(m, max_j s_j),
//       p_j = 2^(s_j - m'), l = l 2^(m - m') + sum p_j, O *= 2^(m - m')
//   O^T += V^T P^T (A = V tile read transposed from LDS, B = P in registers)
//
// Computing the transposed products makes every lane own exactly one query
// row: the row statistics are per-lane scalars (reduced across the 2 or 4 lane
// groups that share the row), and the S^T accumulator registers are already
// laid out as the B operand of the P.V product, so P never leaves registers.
// V stays row-major in LDS and is read with ds_read_b64_tr_b16, which also
// lets a shared K/V row (MLA) be staged once.
//
// The score matrix is never materialised; the result per row is
// O = sum_j e^{S_j - m} v_j / sum_j e^{S_j - m} and LSE = m + log sum e^{S_j - m}
// (attention and softmax_lse formulas of the CANN "flash_attn" page), with the
// optional sink of its sink formulas applied in finish().
#pragma once
#include "device_common.h"

namespace attn {

template <int R_, int D_, int DV_, int NW_, int BN_, bool VSHARED_, bool KEYMASK_ = false>
struct TileCfg {
  static constexpr int R = R_, D = D_, DV = DV_, NW = NW_, BN = BN_;
  static constexpr bool VSHARED = VSHARED_;   // V row = first DV entries of the K row
  static constexpr bool KEYMASK = KEYMASK_;   // per-key validity flags staged with the tile
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW * R;
  static constexpr int KS = D + 8;                     // K row stride in LDS (elements)
  static constexpr int VS = VSHARED ? KS : DV + 16;    // V row stride in LDS (elements)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = VSHARED ? 0 : BN * VS;
  static constexpr int FLAG_BYTES = KEYMASK ? BN * 4 : 0;
  static constexpr int LDS_BYTES = (K_ELEMS + V_ELEMS) * 2 + FLAG_BYTES;
  static constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
  static constexpr int NKL = (BN * KCH + THREADS - 1) / THREADS;
  static constexpr int NVL = VSHARED ? 0 : (BN * VCH + THREADS - 1) / THREADS;
  static_assert(D % Mfma<R>::KSTEP == 0, "head dim must be a multiple of the MFMA depth");
  static_assert(DV % Mfma<R>::SB == 0, "value dim must be a multiple of the MFMA width");
  static_assert(BN % Mfma<R>::SB == 0 && BN % Mfma<R>::PVK == 0, "tile must hold whole MFMA blocks");
};

template <class C>
struct TileCore {
  using M = Mfma<C::R>;
  using acc_t = typename M::acc_t;
  static constexpr int NQ = C::D / M::KSTEP;    // Q fragments (B operands) per row
  static constexpr int NSB = C::BN / M::SB;     // S^T blocks per tile
  static constexpr int NPC = C::BN / M::PVK;    // P chunks (B operands of P.V) per tile
  static constexpr int NOB = C::DV / M::SB;     // O^T blocks
  static constexpr int NP = NSB * M::SREG / 2;  // packed bf16 pairs of P

  struct Stage {
    u32x4 k[C::NKL];
    u32x4 v[C::NVL > 0 ? C::NVL : 1];
    uint32_t kflag;  // bit i: K chunk i came from a valid key
  };

  bf16x8 qf[NQ];
  acc_t o[NOB];
  float m_run;  // running max of this row, base-2 scaled domain
  float l_run;  // this lane's share of the running denominator

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < NOB; ++i) o[i] = acc_t{};
    m_run = kNegInf;
    l_run = 0.f;
  }

  // qrow: this lane's query row (D elements) or nullptr for a padding row.
  __device__ __forceinline__ void load_q(const bf16_t* qrow, int lane) {
    const int g = M::grp(lane);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow) v = *reinterpret_cast<const u32x4*>(qrow + i * M::KSTEP + g * 8);
      qf[i] = as_bf16x8(v);
    }
  }

  // Global -> registers for the tile starting at key j0. kptr(j) / vptr(j)
  // return the row of key j or nullptr (invalid key: zeros are staged, so a
  // masked key never injects NaN/Inf garbage into P.V).
  template <class KP, class VP>
  __device__ __forceinline__ void gload(Stage& st, int j0, int tid, KP kptr, VP vptr) const {
    st.kflag = 0;
#pragma unroll
    for (int i = 0; i < C::NKL; ++i) {
      const int q = tid + i * C::THREADS;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < C::BN * C::KCH) {
        const int r = q / C::KCH, c = q % C::KCH;
        const bf16_t* p = kptr(j0 + r);
        if (p) {
          v = *reinterpret_cast<const u32x4*>(p + c * 8);
          st.kflag |= 1u << i;
        }
      }
      st.k[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::NVL; ++i) {
      const int q = tid + i * C::THREADS;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < C::BN * C::VCH) {
        const int r = q / C::VCH, c = q % C::VCH;
        const bf16_t* p = vptr(j0 + r);
        if (p) v = *reinterpret_cast<const u32x4*>(p + c * 8);
      }
      st.v[i] = v;
    }
  }

  __device__ __forceinline__ void sstore(const Stage& st, bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < C::NKL; ++i) {
      const int q = tid + i * C::THREADS;
      if (q < C::BN * C::KCH) {
        const int r = q / C::KCH, c = q % C::KCH;
        *reinterpret_cast<u32x4*>(lds + r * C::KS + c * 8) = st.k[i];
        if (C::KEYMASK && c == 0)
          reinterpret_cast<float*>(lds + C::K_ELEMS + C::V_ELEMS)[r] =
              (st.kflag >> i) & 1u ? 0.f : kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVL; ++i) {
      const int q = tid + i * C::THREADS;
      if (q < C::BN * C::VCH) {
        const int r = q / C::VCH, c = q % C::VCH;
        *reinterpret_cast<u32x4*>(lds + C::K_ELEMS + r * C::VS + c * 8) = st.v[i];
      }
    }
  }

  // One key tile. cscale = softmax scale * log2(e). vis(j) decides whether
  // key j (absolute index) is visible to this lane's row; it is only
  // consulted when need_mask is true.
  template <class Vis>
  __device__ __forceinline__ void tile(const bf16_t* lds, int j0, bool need_mask, Vis vis,
                                       float cscale, int lane) {
    const int g = M::grp(lane);
    const int rr = M::row(lane);
    acc_t s[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      s[sb] = acc_t{};
      const bf16_t* krow = lds + (sb * M::SB + rr) * C::KS + g * 8;
#pragma unroll
      for (int dq = 0; dq < NQ; ++dq) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + dq * M::KSTEP);
        s[sb] = M::mma(as_bf16x8(a), qf[dq], s[sb]);
      }
    }
    // scale, mask, row max
    float mx = kNegInf;
    const float* kbias = reinterpret_cast<const float*>(lds + C::K_ELEMS + C::V_ELEMS);
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < M::SREG; ++r) {
        float x = s[sb][r] * cscale;
        if (need_mask) {
          const int jl = sb * M::SB + M::mrow(g, r);
          if (C::KEYMASK) x += kbias[jl];
          if (!vis(j0 + jl)) x = kNegInf;
        }
        s[sb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = M::group_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) o[ob] *= alpha;
    // probabilities, packed to bf16 pairs in B-operand order
    uint32_t pk[NP];
    float lsum = 0.f;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < M::SREG; r += 2) {
        const float p0 = fast_exp2(s[sb][r] - m_use);
        const float p1 = fast_exp2(s[sb][r + 1] - m_use);
        lsum += p0 + p1;
        pk[(sb * M::SREG + r) / 2] = pack_bf16x2(p0, p1);
      }
    }
    l_run += lsum;
    // O^T += V^T P^T
    const bf16_t* vt = lds + (C::VSHARED ? 0 : C::K_ELEMS);
    const int i16 = lane & 15;
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      const u32x4 pb = {pk[c * 4], pk[c * 4 + 1], pk[c * 4 + 2], pk[c * 4 + 3]};
      const bf16x8 b = as_bf16x8(pb);
      const bf16_t* vrow = vt + (c * M::PVK + g * 4 + (i16 >> 2)) * C::VS + M::tr_col(lane) +
                           (i16 & 3) * 4;
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) {
        const s16x4 lo = lds_read_tr(vrow + ob * M::SB);
        const s16x4 hi = lds_read_tr(vrow + (M::PVK / 2) * C::VS + ob * M::SB);
        o[ob] = M::mma(join_bf16x8(lo, hi), b, o[ob]);
      }
    }
  }

  // Final normalisation. Returns the factor that turns the accumulator into
  // the output row, and the row's LSE (natural log, sink-free, -inf for a row
  // that saw no key). With a sink (base-2 scaled logit sink2) the denominator
  // gains 2^(sink2 - m) measured against m* = max(m, sink2).
  __device__ __forceinline__ float finish(bool has_sink, float sink2, float& lse) const {
    const float l = M::group_sum(l_run);
    const bool empty = !(l > 0.f);
    lse = empty ? kNegInf : (m_run + fast_log2(l)) * kLn2;
    if (!has_sink) return empty ? 0.f : 1.f / l;
    if (empty) return 0.f;
    const float ms = fmaxf(m_run, sink2);
    const float f = fast_exp2(m_run - ms);
    return f / (l * f + fast_exp2(sink2 - ms));
  }

  // Writes this lane's share of the output row: NOB blocks x SREG values,
  // four consecutive columns at a time. OutT is bf16_t or float.
  template <class OutT>
  __device__ __forceinline__ void store(OutT* orow, float inv, int lane) const {
    const int g = M::grp(lane);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int r = 0; r < M::SREG; r += 4) {
        const int col = ob * M::SB + M::mrow(g, r);
        const float a0 = o[ob][r] * inv, a1 = o[ob][r + 1] * inv;
        const float a2 = o[ob][r + 2] * inv, a3 = o[ob][r + 3] * inv;
        if constexpr (sizeof(OutT) == 2) {
          const u32x2 w = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
          *reinterpret_cast<u32x2*>(orow + col) = w;
        } else {
          const f32x4 w = {a0, a1, a2, a3};
          *reinterpret_cast<f32x4*>(orow + col) = w;
        }
      }
    }
  }
};

// Runs the whole key loop [lo, hi) for one workgroup with register-staged
// prefetch of the next tile while the current one is computed.
// need(j0) -> bool says whether tile j0 may contain keys that some row of
// the workgroup must not see.
template <class C, class KP, class VP, class Need, class Vis>
__device__ __forceinline__ void run_keys(TileCore<C>& core, bf16_t* lds, int lo, int hi,
                                         float cscale, KP kptr, VP vptr, Need need, Vis vis) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (lo >= hi) return;
  typename TileCore<C>::Stage st;
  core.gload(st, lo, tid, kptr, vptr);
  for (int j0 = lo; j0 < hi; j0 += C::BN) {
    core.sstore(st, lds, tid);
    __syncthreads();
    if (j0 + C::BN < hi) core.gload(st, j0 + C::BN, tid, kptr, vptr);
    core.tile(lds, j0, need(j0), vis, cscale, lane);
    __syncthreads();
  }
}

}  // namespace attn
