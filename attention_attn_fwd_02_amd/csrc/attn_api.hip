// C ABI of libattn_mi355.so (declared in include/attn.h): host-side argument
// checks, instance selection and launches on the caller's stream. Checks run
// before anything is enqueued; device tensor contents are never inspected.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>

#include "../../include/attn.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The kernels move 16-byte vectors of every element tensor; NULL (an absent
// optional tensor) passes.
template <class... P>
bool aligned16(const P*... p) {
  return ((((uintptr_t)p & 15) == 0) && ...);
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

}  // namespace

namespace attn {

int32_t set_error(int32_t code, const char* msg) { return fail(code, "%s", msg); }

// Host checks of attn_decode_paged apart from its plan and partial buffers
// (shared with attn_decode_paged_noalloc, which supplies those itself).
int32_t check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                          int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                          int32_t dtype, float scale, int32_t max_splits) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 && page_size > 0 &&
              max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  // d = 576, dv = 512: the MLA-absorbed row (value = its first 512 entries)
  const bool mla = d == 576 && dv == 512;
  REQUIRE(q && k_cache && (v_cache || mla) && block_table && cache_seqlens, ATTN_EINVAL,
          "null tensor pointer");
  REQUIRE(aligned16(q, k_cache, v_cache), ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(dtype == ATTN_BF16, ATTN_EUNSUPPORTED, "decode supports bf16 only");
  REQUIRE((d == dv && (d == 64 || d == 128)) || mla, ATTN_EUNSUPPORTED,
          "decode supports d = dv in {64, 128} and d = 576, dv = 512 (got %d, %d)", d, dv);
  REQUIRE(!mla || v_cache == nullptr || v_cache == k_cache, ATTN_EUNSUPPORTED,
          "d = 576, dv = 512 reads the values from the key rows: v_cache must be NULL or k_cache");
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 cache rows are 32-bit)");
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

const char* attn_status_string(int32_t status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_EINVAL: return "ATTN_EINVAL";
    case ATTN_EUNSUPPORTED: return "ATTN_EUNSUPPORTED";
    case ATTN_EEMPTY: return "ATTN_EEMPTY";
    case ATTN_EHIP: return "ATTN_EHIP";
    default: return "ATTN_UNKNOWN";
  }
}

const char* attn_last_error(void) { return g_err; }

int32_t attn_device_info(int32_t device, int32_t* num_cu) {
  REQUIRE(num_cu, ATTN_EINVAL, "num_cu is NULL");
  int v = 0;
  hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute");
  *num_cu = v;
  return ok();
}

// attn_fwd_varlen and attn_fwd_varlen_mask: host checks, then the launch
// (mask NULL: the plain kernel).
static int32_t varlen_launch(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                             int32_t hkv, int32_t d, int32_t dv, int32_t dtype, float scale,
                             int32_t causal, int32_t window_left, int32_t window_right,
                             const float* sinks, const void* mask, int32_t mask_heads,
                             int32_t mask_ld, void* out, float* lse, void* stream,
                             const char* what) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0, ATTN_EEMPTY,
          "empty dimension (batch=%d max_seqlen_q=%d hq=%d hkv=%d d=%d dv=%d)", batch,
          max_seqlen_q, hq, hkv, d, dv);
  REQUIRE(max_seqlen_k >= 0, ATTN_EINVAL, "max_seqlen_k < 0");
  REQUIRE(q && k && v && cu_seqlens_q && cu_seqlens_k && out, ATTN_EINVAL,
          "null tensor pointer");
  REQUIRE(aligned16(q, k, v, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(dtype == ATTN_BF16 || dtype == ATTN_F32, ATTN_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(!mask || dtype == ATTN_BF16, ATTN_EUNSUPPORTED, "the additive mask needs bf16 inputs");
  REQUIRE(d == dv && (d == 64 || d == 128), ATTN_EUNSUPPORTED,
          "head dims d=%d dv=%d not supported (d == dv in {64, 128})", d, dv);
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.mask = mask;
  a.mask_heads = mask_heads;
  a.mask_ld = mask_ld;
  a.kc = nullptr;
  a.vc = nullptr;
  a.block_table = nullptr;
  a.cache_lens = nullptr;
  a.max_pages = 0;
  a.page = 0;
  const int rows = dtype == ATTN_BF16 ? attn::varlen_bf16_rows(d) : attn::varlen_f32_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  hipError_t e = dtype == ATTN_BF16 ? attn::launch_varlen_bf16(a, d, as_stream(stream))
                                    : attn::launch_varlen_f32(a, d, as_stream(stream));
  return hip_status(e, what);
}

int32_t attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                        int32_t max_seqlen_k, int32_t hq, int32_t hkv, int32_t d, int32_t dv,
                        int32_t dtype, float scale, int32_t causal, int32_t window_left,
                        int32_t window_right, const float* sinks, void* out, float* lse,
                        void* stream) {
  return varlen_launch(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                       hq, hkv, d, dv, dtype, scale, causal, window_left, window_right, sinks,
                       nullptr, 0, 0, out, lse, stream, "attn_fwd_varlen launch");
}

int32_t attn_fwd_varlen_mask(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                             int32_t hkv, int32_t d, int32_t dv, float scale, int32_t causal,
                             int32_t window_left, int32_t window_right, const float* sinks,
                             const void* mask, int32_t mask_heads, int32_t mask_ld, void* out,
                             float* lse, void* stream) {
  REQUIRE(mask, ATTN_EINVAL, "null mask (attn_fwd_varlen computes the unmasked case)");
  REQUIRE(mask_heads == 1 || mask_heads == hq, ATTN_EINVAL,
          "mask_heads must be 1 or hq (got %d)", mask_heads);
  REQUIRE(mask_ld > 0 && mask_ld % 64 == 0, ATTN_EINVAL,
          "mask_ld must be a positive multiple of 64 (got %d)", mask_ld);
  REQUIRE((long)mask_ld * 2 * 32 < (1L << 32), ATTN_EUNSUPPORTED, "mask_ld too large");
  REQUIRE(max_seqlen_k <= mask_ld, ATTN_EINVAL,
          "mask_ld (%d) is below max_seqlen_k (%d)", mask_ld, max_seqlen_k);
  REQUIRE(aligned16(mask), ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  return varlen_launch(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                       hq, hkv, d, dv, ATTN_BF16, scale, causal, window_left, window_right, sinks,
                       mask, mask_heads, mask_ld, out, lse, stream, "attn_fwd_varlen_mask launch");
}

int32_t attn_fwd_varlen_fp8(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t fp8_format,
                            const float* q_descale, const float* k_descale,
                            const float* v_descale, float scale, int32_t causal,
                            int32_t window_left, int32_t window_right, const float* sinks,
                            void* out, float* lse, void* stream) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0, ATTN_EEMPTY,
          "empty dimension (batch=%d max_seqlen_q=%d hq=%d hkv=%d d=%d dv=%d)", batch,
          max_seqlen_q, hq, hkv, d, dv);
  REQUIRE(max_seqlen_k >= 0, ATTN_EINVAL, "max_seqlen_k < 0");
  REQUIRE(q && k && v && cu_seqlens_q && cu_seqlens_k && out, ATTN_EINVAL,
          "null tensor pointer");
  REQUIRE(aligned16(q, k, v, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(fp8_format == ATTN_FP8_E4M3 || fp8_format == ATTN_FP8_E5M2, ATTN_EUNSUPPORTED,
          "fp8_format %d (expected ATTN_FP8_E4M3 or ATTN_FP8_E5M2)", fp8_format);
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED, "FP8 varlen supports d = dv = 128 (got %d, %d)",
          d, dv);
  REQUIRE((long)hkv * d * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  const int rows = attn::varlen_bf16_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  return hip_status(attn::launch_varlen_fp8(a, fp8_format == ATTN_FP8_E4M3 ? 1 : 2,
                                            as_stream(stream)),
                    "attn_fwd_varlen_fp8 launch");
}

int32_t attn_fwd_varlen_qv(const void* q, const void* qv, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                           int32_t hkv, int32_t d, int32_t dv, int32_t dtype,
                           const float* q_descale, const float* k_descale,
                           const float* v_descale, float scale, int32_t causal,
                           int32_t window_left, int32_t window_right, const float* sinks,
                           int32_t only_qv, void* out, float* lse, void* stream) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0, ATTN_EEMPTY,
          "empty dimension (batch=%d max_seqlen_q=%d hq=%d hkv=%d d=%d dv=%d)", batch,
          max_seqlen_q, hq, hkv, d, dv);
  REQUIRE(max_seqlen_k >= 0, ATTN_EINVAL, "max_seqlen_k < 0");
  REQUIRE(qv && v && cu_seqlens_q && cu_seqlens_k && out, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, qv, k, v, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(only_qv || (q && k), ATTN_EINVAL, "q and k are required unless only_qv");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2,
          ATTN_EUNSUPPORTED, "dtype %d (expected ATTN_BF16, ATTN_FP8_E4M3 or ATTN_FP8_E5M2)",
          dtype);
  const int fmt = dtype == ATTN_BF16 ? 0 : (dtype == ATTN_FP8_E4M3 ? 1 : 2);
  REQUIRE(fmt != 0 || (!q_descale && !k_descale && !v_descale), ATTN_EINVAL,
          "descales apply to FP8 inputs only");
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED, "qv supports d = dv = 128 (got %d, %d)", d,
          dv);
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  attn::VarlenArgs a{};
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.q_descale = q_descale;
  a.v_descale = v_descale;
  const int rows = attn::varlen_bf16_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  hipError_t e;
  if (only_qv) {
    // scores qv . v_j alone: the plain prefill with qv as its query and the
    // value rows in the role of the keys (k_descale -> v_descale)
    a.q = qv;
    a.k = v;
    a.v = v;
    a.k_descale = v_descale;
    e = fmt == 0 ? attn::launch_varlen_bf16(a, d, as_stream(stream))
                 : attn::launch_varlen_fp8(a, fmt, as_stream(stream));
  } else {
    a.q = q;
    a.qv = qv;
    a.k = k;
    a.v = v;
    a.k_descale = k_descale;
    e = attn::launch_varlen_qv(a, fmt, as_stream(stream));
  }
  return hip_status(e, "attn_fwd_varlen_qv launch");
}

int32_t attn_fwd_varlen_kvcache(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* cache_seqlens, int32_t page_size, int32_t batch,
                                int32_t max_seqlen_q, int32_t hq, int32_t hkv, int32_t d,
                                int32_t dv, int32_t dtype, float scale, int32_t causal,
                                int32_t window_left, int32_t window_right, const float* sinks,
                                const void* mask, int32_t mask_heads, int32_t mask_ld,
                                void* out, float* lse, void* stream) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 &&
              page_size > 0 && max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  // k and v may be NULL when no sequence has current rows (they are then never read)
  REQUIRE(q && cu_seqlens_q && cu_seqlens_k && k_cache && v_cache && block_table &&
              cache_seqlens && out,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, k, v, k_cache, v_cache, out, mask), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(dtype == ATTN_BF16, ATTN_EUNSUPPORTED, "cache + current attention supports bf16 only");
  REQUIRE(d == dv && (d == 64 || d == 128), ATTN_EUNSUPPORTED,
          "head dims d=%d dv=%d not supported (d == dv in {64, 128})", d, dv);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  if (mask) {
    REQUIRE(mask_heads == 1 || mask_heads == hq, ATTN_EINVAL,
            "mask_heads must be 1 or hq (got %d)", mask_heads);
    REQUIRE(mask_ld > 0 && mask_ld % 64 == 0, ATTN_EINVAL,
            "mask_ld must be a positive multiple of 64 (got %d)", mask_ld);
    REQUIRE((long)mask_ld * 2 * 32 < (1L << 32), ATTN_EUNSUPPORTED, "mask_ld too large");
  }
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.mask = mask;
  a.mask_heads = mask_heads;
  a.mask_ld = mask_ld;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.cache_lens = cache_seqlens;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  const int rows = attn::varlen_bf16_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  return hip_status(attn::launch_varlen_kvcache_bf16(a, d, as_stream(stream)),
                    "attn_fwd_varlen_kvcache launch");
}

int32_t attn_fwd_varlen_kvcache_qv(const void* q, const void* qv, const void* k, const void* v,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_pages_per_seq,
                                   const int32_t* cache_seqlens, int32_t page_size,
                                   int32_t batch, int32_t max_seqlen_q, int32_t hq, int32_t hkv,
                                   int32_t d, int32_t dv, float scale, int32_t causal,
                                   int32_t window_left, int32_t window_right,
                                   const float* sinks, int32_t only_qv, void* out, float* lse,
                                   void* stream) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 &&
              page_size > 0 && max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  // current rows may be NULL when no sequence has any (they are then never read)
  REQUIRE(qv && cu_seqlens_q && cu_seqlens_k && v_cache && block_table && cache_seqlens && out,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(only_qv || (q && k_cache), ATTN_EINVAL, "q and k_cache are required unless only_qv");
  REQUIRE(aligned16(q, qv, k, v, k_cache, v_cache, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED,
          "qv over a cache supports d = dv = 128 (got %d, %d)", d, dv);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  attn::VarlenArgs a{};
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.block_table = block_table;
  a.cache_lens = cache_seqlens;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  const int rows = attn::varlen_bf16_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  hipError_t e;
  if (only_qv) {
    // scores qv . v_j alone: the cache-plus-current prefill with qv as its
    // query and the value rows (cached and current) in the role of the keys
    a.q = qv;
    a.k = v;
    a.v = v;
    a.kc = v_cache;
    a.vc = v_cache;
    e = attn::launch_varlen_kvcache_bf16(a, d, as_stream(stream));
  } else {
    a.q = q;
    a.qv = qv;
    a.k = k;
    a.v = v;
    a.kc = k_cache;
    a.vc = v_cache;
    e = attn::launch_varlen_kvcache_qv_bf16(a, as_stream(stream));
  }
  return hip_status(e, "attn_fwd_varlen_kvcache_qv launch");
}

int32_t attn_fwd_varlen_kvcache_fp8(const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, int32_t max_pages_per_seq,
                                    const int32_t* cache_seqlens, int32_t page_size,
                                    int32_t batch, int32_t max_seqlen_q, int32_t hq, int32_t hkv,
                                    int32_t d, int32_t dv, int32_t fp8_format,
                                    const float* q_descale, const float* k_descale,
                                    const float* v_descale, float scale, int32_t causal,
                                    int32_t window_left, int32_t window_right,
                                    const float* sinks, void* out, float* lse, void* stream) {
  REQUIRE(batch > 0 && max_seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 &&
              page_size > 0 && max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  // k and v may be NULL when no sequence has current rows (they are then never read)
  REQUIRE(q && cu_seqlens_q && cu_seqlens_k && k_cache && v_cache && block_table &&
              cache_seqlens && out,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, k, v, k_cache, v_cache, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(window_left >= -1 && window_right >= -1, ATTN_EINVAL, "window bounds must be >= -1");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(fp8_format == ATTN_FP8_E4M3 || fp8_format == ATTN_FP8_E5M2, ATTN_EUNSUPPORTED,
          "fp8_format %d (expected ATTN_FP8_E4M3 or ATTN_FP8_E5M2)", fp8_format);
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED,
          "FP8 cache + current supports d = dv = 128 (got %d, %d)", d, dv);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 key rows are 32-bit)");
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.causal = causal ? 1 : 0;
  a.wl = window_left;
  a.wr = window_right;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.cache_lens = cache_seqlens;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  const int rows = attn::varlen_bf16_rows(d);
  a.nqt = (max_seqlen_q + rows - 1) / rows;
  REQUIRE((long)a.nqt * batch * hq < (1L << 31), ATTN_EUNSUPPORTED, "grid too large");
  return hip_status(attn::launch_varlen_kvcache_fp8(a, fp8_format == ATTN_FP8_E4M3 ? 1 : 2,
                                                    as_stream(stream)),
                    "attn_fwd_varlen_kvcache_fp8 launch");
}

size_t attn_plan_words(int32_t batch, int32_t max_splits) {
  if (batch <= 0 || max_splits <= 0) return 0;
  return 3 + (size_t)batch + 4 * (size_t)batch * max_splits;
}

int32_t attn_plan_splits(const int32_t* cache_seqlens, int32_t batch, int32_t page_size,
                         int32_t units_per_block, int32_t num_cu, int32_t waves,
                         int32_t max_splits, int32_t min_blocks, int32_t* plan, void* stream) {
  REQUIRE(batch > 0, ATTN_EEMPTY, "batch is 0");
  REQUIRE(cache_seqlens && plan, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(page_size > 0 && units_per_block > 0 && num_cu > 0 && waves > 0 && min_blocks > 0,
          ATTN_EINVAL, "page_size, units_per_block, num_cu, waves, min_blocks must be > 0");
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  return hip_status(attn::launch_plan(cache_seqlens, batch, page_size, units_per_block, num_cu,
                                      waves, max_splits, min_blocks, plan, as_stream(stream)),
                    "attn_plan_splits launch");
}

int32_t attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                          int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                          int32_t dtype, float scale, int32_t causal, const int32_t* plan,
                          int32_t max_splits, float* o_partial, float* lse_partial,
                          void* stream) {
  const int32_t st = attn::check_decode_args(q, k_cache, v_cache, block_table,
                                             max_pages_per_seq, cache_seqlens, batch, seqlen_q,
                                             hq, hkv, d, dv, page_size, dtype, scale, max_splits);
  if (st != ATTN_OK) return st;
  const bool mla = d == 576 && dv == 512;
  REQUIRE(plan && o_partial && lse_partial, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(o_partial), ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  attn::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.hkv = hkv;
  a.page = page_size;
  a.causal = causal ? 1 : 0;
  a.max_splits = max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  if (mla) {
    a.vc = nullptr;
    return hip_status(attn::launch_decode_mla(a, as_stream(stream)), "attn_decode_paged launch");
  }
  return hip_status(attn::launch_decode_gqa(a, d, as_stream(stream)), "attn_decode_paged launch");
}

int32_t attn_decode_paged_mask(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                               int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                               float scale, int32_t causal, const void* mask, int32_t mask_heads,
                               int32_t mask_ld, const int32_t* plan, int32_t max_splits,
                               float* o_partial, float* lse_partial, void* stream) {
  const int32_t st = attn::check_decode_args(q, k_cache, v_cache, block_table,
                                             max_pages_per_seq, cache_seqlens, batch, seqlen_q,
                                             hq, hkv, d, dv, page_size, ATTN_BF16, scale,
                                             max_splits);
  if (st != ATTN_OK) return st;
  REQUIRE(d == dv && (d == 64 || d == 128) && v_cache, ATTN_EUNSUPPORTED,
          "the decode mask supports d == dv in {64, 128} with a separate V cache");
  REQUIRE(plan && o_partial && lse_partial && mask, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(o_partial, mask), ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  REQUIRE(mask_heads == 1 || mask_heads == hq, ATTN_EINVAL,
          "mask_heads must be 1 or hq (got %d)", mask_heads);
  REQUIRE(mask_ld > 0 && mask_ld % 64 == 0, ATTN_EINVAL,
          "mask_ld must be a positive multiple of 64 (got %d)", mask_ld);
  attn::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.hkv = hkv;
  a.page = page_size;
  a.causal = causal ? 1 : 0;
  a.max_splits = max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.mask = mask;
  a.mask_heads = mask_heads;
  a.mask_ld = mask_ld;
  return hip_status(attn::launch_decode_gqa(a, d, as_stream(stream)),
                    "attn_decode_paged_mask launch");
}

int32_t attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int32_t max_pages_per_seq,
                              const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                              int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                              int32_t fp8_format, const float* q_descale,
                              const float* k_descale, const float* v_descale, float scale,
                              int32_t causal, const int32_t* plan, int32_t max_splits,
                              float* o_partial, float* lse_partial, void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 && page_size > 0 &&
              max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(q && k_cache && v_cache && block_table && cache_seqlens && plan && o_partial &&
              lse_partial,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, k_cache, v_cache, o_partial), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(fp8_format == ATTN_FP8_E4M3 || fp8_format == ATTN_FP8_E5M2, ATTN_EUNSUPPORTED,
          "fp8_format %d (expected ATTN_FP8_E4M3 or ATTN_FP8_E5M2)", fp8_format);
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED, "decode supports d = dv = 128 (got %d, %d)",
          d, dv);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 cache rows are 32-bit)");
  attn::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.hkv = hkv;
  a.page = page_size;
  a.causal = causal ? 1 : 0;
  a.max_splits = max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  return hip_status(attn::launch_decode_gqa_fp8(a, fp8_format == ATTN_FP8_E4M3 ? 1 : 2,
                                                as_stream(stream)),
                    "attn_decode_paged_fp8 launch");
}

int32_t attn_decode_paged_qv(const void* q, const void* qv, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* cache_seqlens,
                             int32_t batch, int32_t seqlen_q, int32_t hq, int32_t hkv, int32_t d,
                             int32_t dv, int32_t page_size, int32_t dtype,
                             const float* q_descale, const float* k_descale,
                             const float* v_descale, float scale, int32_t causal,
                             int32_t only_qv, const int32_t* plan, int32_t max_splits,
                             float* o_partial, float* lse_partial, void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && hkv > 0 && d > 0 && dv > 0 && page_size > 0 &&
              max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(qv && v_cache && block_table && cache_seqlens && plan && o_partial && lse_partial,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, qv, k_cache, v_cache, o_partial), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(only_qv || (q && k_cache), ATTN_EINVAL, "q and k_cache are required unless only_qv");
  REQUIRE(hq % hkv == 0, ATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", hq, hkv);
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2,
          ATTN_EUNSUPPORTED, "dtype %d (expected ATTN_BF16, ATTN_FP8_E4M3 or ATTN_FP8_E5M2)",
          dtype);
  const bool fp8 = dtype != ATTN_BF16;
  REQUIRE(fp8 || (!q_descale && !k_descale && !v_descale), ATTN_EINVAL,
          "descales apply to FP8 inputs only");
  REQUIRE(d == 128 && dv == 128, ATTN_EUNSUPPORTED, "decode supports d = dv = 128 (got %d, %d)",
          d, dv);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  REQUIRE((long)hkv * d * 2 * 16 < (1L << 32), ATTN_EUNSUPPORTED,
          "hkv * d too large (byte offsets within 16 cache rows are 32-bit)");
  attn::DecodeArgs a{};
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.hkv = hkv;
  a.page = page_size;
  a.causal = causal ? 1 : 0;
  a.max_splits = max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.q_descale = q_descale;
  a.v_descale = v_descale;
  if (only_qv) {
    // scores qv . v_j alone: tiles of V only; the score scale takes the V
    // descale where the QK path takes the K descale (q and K are not read)
    a.q = qv;
    a.qv = qv;
    a.only_qv = 1;
    a.kc = v_cache;
    a.vc = v_cache;
    a.k_descale = v_descale;
  } else {
    a.q = q;
    a.qv = qv;
    a.kc = k_cache;
    a.vc = v_cache;
    a.k_descale = k_descale;
  }
  const hipError_t e =
      fp8 ? attn::launch_decode_gqa_fp8(a, dtype == ATTN_FP8_E4M3 ? 1 : 2, as_stream(stream))
          : attn::launch_decode_gqa(a, d, as_stream(stream));
  return hip_status(e, "attn_decode_paged_qv launch");
}

int32_t attn_combine(const float* o_partial, const float* lse_partial, const int32_t* plan,
                     int32_t batch, int32_t seqlen_q, int32_t hq, int32_t dv, int32_t max_splits,
                     const float* sinks, int32_t out_dtype, void* out, float* lse,
                     void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && dv > 0, ATTN_EEMPTY, "empty dimension");
  REQUIRE(o_partial && lse_partial && plan && out, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(o_partial, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(out_dtype == ATTN_BF16 || out_dtype == ATTN_F32, ATTN_EUNSUPPORTED, "out_dtype %d",
          out_dtype);
  REQUIRE(dv % 4 == 0 && dv <= 1024, ATTN_EUNSUPPORTED, "dv must be a multiple of 4, <= 1024");
  attn::CombineArgs a{};
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  a.plan = plan;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.dv = dv;
  a.max_splits = max_splits;
  a.out_bf16 = out_dtype == ATTN_BF16;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  return hip_status(attn::launch_combine(a, as_stream(stream)), "attn_combine launch");
}

int32_t mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_table,
                         int32_t max_pages_per_seq, const int32_t* cache_seqlens, int32_t batch,
                         int32_t seqlen_q, int32_t hq, int32_t page_size, float scale,
                         int32_t causal, const int32_t* plan, int32_t max_splits,
                         float* o_partial, float* lse_partial, void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && page_size > 0 && max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(q && kv_cache && block_table && cache_seqlens && plan && o_partial && lse_partial,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, kv_cache, o_partial), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  attn::DecodeArgs a{};
  a.q = q;
  a.kc = kv_cache;
  a.vc = nullptr;
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = seqlen_q;
  a.hq = hq;
  a.hkv = 1;
  a.page = page_size;
  a.causal = causal ? 1 : 0;
  a.max_splits = max_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_partial;
  a.lse_part = lse_partial;
  return hip_status(attn::launch_decode_mla(a, as_stream(stream)), "mla_decode_paged launch");
}

int32_t mla_sparse_fwd(const void* q, const void* kv, const int32_t* sparse_indices, int32_t topk,
                       int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t hq, float scale,
                       int32_t sparse_mode, const float* sinks, void* out, float* lse,
                       void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && seqlen_k > 0 && hq > 0 && topk > 0, ATTN_EEMPTY,
          "empty dimension");
  REQUIRE(q && kv && sparse_indices && out, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(q, kv, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(sparse_mode == 0 || sparse_mode == 3, ATTN_EINVAL, "sparse_mode must be 0 or 3");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  REQUIRE(hq % 16 == 0, ATTN_EUNSUPPORTED, "hq must be a multiple of 16");
  REQUIRE((long)batch * seqlen_q * ((hq + 63) / 64) < (1L << 31), ATTN_EUNSUPPORTED,
          "grid too large");
  REQUIRE((long)seqlen_k * 576 * 2 <= (1L << 32), ATTN_EUNSUPPORTED,
          "seqlen_k %d above %ld (row byte offsets are 32-bit)", seqlen_k, (1L << 32) / 1152);
  attn::SparseArgs a{};
  a.q = q;
  a.kv = kv;
  a.idx = sparse_indices;
  a.topk = topk;
  a.batch = batch;
  a.sq = seqlen_q;
  a.sk = seqlen_k;
  a.hq = hq;
  a.mode = sparse_mode;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  return hip_status(attn::launch_sparse_mla(a, as_stream(stream)), "mla_sparse_fwd launch");
}

int32_t mla_sparse_paged_fwd(const void* q, const void* kv_cache, int32_t num_blocks,
                             int32_t page_size, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seqlens_kv,
                             const int32_t* sparse_indices, int32_t topk,
                             int32_t sparse_block_size, int32_t batch, int32_t seqlen_q,
                             int32_t hq, float scale, int32_t sparse_mode, const float* sinks,
                             void* out, float* lse, void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && hq > 0 && topk > 0 && num_blocks > 0 && page_size > 0 &&
              max_pages_per_seq > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(q && kv_cache && block_table && seqlens_kv && sparse_indices && out, ATTN_EINVAL,
          "null tensor pointer");
  REQUIRE(aligned16(q, kv_cache, out), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(sparse_mode == 0 || sparse_mode == 3, ATTN_EINVAL, "sparse_mode must be 0 or 3");
  REQUIRE(std::isfinite(scale) && scale > 0.f, ATTN_EINVAL,
          "scale must be positive and finite");
  int ls = 0;
  while (ls < 8 && (1 << ls) < sparse_block_size) ++ls;
  REQUIRE(sparse_block_size >= 1 && sparse_block_size <= 128 && (1 << ls) == sparse_block_size,
          ATTN_EINVAL, "sparse_block_size %d is not a power of two in [1, 128]",
          sparse_block_size);
  REQUIRE((long)topk * sparse_block_size < (1L << 31), ATTN_EUNSUPPORTED, "too many keys");
  REQUIRE(hq % 16 == 0, ATTN_EUNSUPPORTED, "hq must be a multiple of 16");
  REQUIRE((long)batch * seqlen_q * ((hq + 63) / 64) < (1L << 31), ATTN_EUNSUPPORTED,
          "grid too large");
  REQUIRE((long)num_blocks * page_size * 576 * 2 <= (1L << 32), ATTN_EUNSUPPORTED,
          "page pool above %ld rows (row byte offsets are 32-bit)", (1L << 32) / 1152);
  attn::SparseArgs a{};
  a.q = q;
  a.kv = kv_cache;
  a.idx = sparse_indices;
  a.block_table = block_table;
  a.seqlens = seqlens_kv;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  a.ls = ls;
  a.topk = topk;
  a.batch = batch;
  a.sq = seqlen_q;
  a.sk = 0;
  a.hq = hq;
  a.mode = sparse_mode;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sinks = sinks;
  a.out = out;
  a.lse = lse;
  return hip_status(attn::launch_sparse_mla(a, as_stream(stream)), "mla_sparse_paged_fwd launch");
}

int32_t attn_debug_gather_paged(int32_t kernel, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* cache_seqlens, int32_t batch, int32_t hkv, int32_t d,
                                int32_t page_size, int32_t dtype, const int32_t* plan,
                                int32_t max_splits, int32_t dump_rows, void* k_dst, void* v_dst,
                                void* stream) {
  REQUIRE(batch > 0 && hkv > 0 && d > 0 && page_size > 0 && max_pages_per_seq > 0 &&
              dump_rows > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(kernel == ATTN_GATHER_DECODE || kernel == ATTN_GATHER_MLA, ATTN_EINVAL,
          "kernel %d (expected ATTN_GATHER_DECODE or ATTN_GATHER_MLA)", kernel);
  const bool mla = kernel == ATTN_GATHER_MLA;
  REQUIRE(k_cache && (v_cache || mla) && block_table && cache_seqlens && plan && k_dst &&
              (v_dst || mla),
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(k_cache, v_cache, k_dst, v_dst), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(max_splits >= 1 && max_splits <= 16, ATTN_EINVAL, "max_splits %d not in [1, 16]",
          max_splits);
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  int fmt = 0;
  if (mla) {
    REQUIRE(d == 576 && dtype == ATTN_BF16, ATTN_EUNSUPPORTED, "MLA rows are 576 bf16");
  } else {
    REQUIRE(dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2,
            ATTN_EUNSUPPORTED, "dtype %d", dtype);
    fmt = dtype == ATTN_BF16 ? 0 : (dtype == ATTN_FP8_E4M3 ? 1 : 2);
    REQUIRE(fmt == 0 ? (d == 64 || d == 128) : d == 128, ATTN_EUNSUPPORTED,
            "head dim %d not supported by the decode kernel for dtype %d", d, dtype);
  }
  attn::DecodeArgs a{};
  a.kc = k_cache;
  a.vc = mla ? nullptr : v_cache;
  a.block_table = block_table;
  a.lens = cache_seqlens;
  a.plan = plan;
  a.max_pages = max_pages_per_seq;
  a.batch = batch;
  a.sq = 1;
  a.hq = hkv;  // one row tile per (split, KV head)
  a.hkv = hkv;
  a.page = page_size;
  a.max_splits = max_splits;
  a.dump_k = k_dst;
  a.dump_v = v_dst;
  a.dump_rows = dump_rows;
  const hipError_t e = mla ? attn::launch_dump_mla(a, as_stream(stream))
                           : attn::launch_dump_decode(a, d, fmt, as_stream(stream));
  return hip_status(e, "attn_debug_gather_paged launch");
}

int32_t attn_debug_gather_kvcache(const void* k, const void* v, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int32_t max_pages_per_seq, const int32_t* cache_seqlens,
                                  int32_t page_size, int32_t batch, int32_t hkv, int32_t d,
                                  int32_t dtype, int32_t dump_rows, void* k_dst, void* v_dst,
                                  void* stream) {
  REQUIRE(batch > 0 && hkv > 0 && d > 0 && page_size > 0 && max_pages_per_seq > 0 &&
              dump_rows > 0,
          ATTN_EEMPTY, "empty dimension");
  REQUIRE(cu_seqlens_q && cu_seqlens_k && k_cache && v_cache && block_table && cache_seqlens &&
              k_dst && v_dst,
          ATTN_EINVAL, "null tensor pointer");
  REQUIRE(aligned16(k, v, k_cache, v_cache, k_dst, v_dst), ATTN_EINVAL,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(dtype == ATTN_BF16 || dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E5M2,
          ATTN_EUNSUPPORTED, "dtype %d", dtype);
  REQUIRE(d == 128, ATTN_EUNSUPPORTED, "the cache-plus-current gather test covers d = 128");
  REQUIRE(page_size % 16 == 0, ATTN_EUNSUPPORTED, "page_size must be a multiple of 16");
  attn::VarlenArgs a{};
  a.k = k;
  a.v = v;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.hq = hkv;  // one query head per KV head: every (sequence, KV head) dumps once
  a.hkv = hkv;
  a.nqt = 1;   // query tile 0 only
  a.causal = 0;
  a.wl = -1;
  a.wr = -1;
  a.kc = k_cache;
  a.vc = v_cache;
  a.block_table = block_table;
  a.cache_lens = cache_seqlens;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  a.dump_k = k_dst;
  a.dump_v = v_dst;
  a.dump_rows = dump_rows;
  const int fmt = dtype == ATTN_BF16 ? 0 : (dtype == ATTN_FP8_E4M3 ? 1 : 2);
  return hip_status(attn::launch_dump_kvcache(a, fmt, as_stream(stream)),
                    "attn_debug_gather_kvcache launch");
}

int32_t attn_debug_gather_sparse(const void* kv, int32_t seqlen_k, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seqlens_kv,
                                 int32_t page_size, const int32_t* sparse_indices, int32_t topk,
                                 int32_t sparse_block_size, int32_t batch, int32_t seqlen_q,
                                 int32_t sparse_mode, int32_t dump_rows, void* dst, void* stream) {
  REQUIRE(batch > 0 && seqlen_q > 0 && topk > 0 && dump_rows > 0, ATTN_EEMPTY,
          "empty dimension");
  REQUIRE(kv && sparse_indices && dst, ATTN_EINVAL, "null tensor pointer");
  REQUIRE(!block_table || (seqlens_kv && page_size > 0 && max_pages_per_seq > 0), ATTN_EINVAL,
          "a paged pool needs seqlens_kv, page_size and max_pages_per_seq");
  REQUIRE(block_table || seqlen_k > 0, ATTN_EEMPTY, "seqlen_k is 0");
  REQUIRE(aligned16(kv, dst), ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  REQUIRE(sparse_mode == 0 || sparse_mode == 3, ATTN_EINVAL, "sparse_mode must be 0 or 3");
  int ls = 0;
  while (ls < 8 && (1 << ls) < sparse_block_size) ++ls;
  REQUIRE(sparse_block_size >= 1 && sparse_block_size <= 128 && (1 << ls) == sparse_block_size,
          ATTN_EINVAL, "sparse_block_size %d is not a power of two in [1, 128]",
          sparse_block_size);
  REQUIRE((long)topk * sparse_block_size <= dump_rows, ATTN_EINVAL,
          "dump_rows must hold topk * sparse_block_size keys");
  attn::SparseArgs a{};
  a.kv = kv;
  a.idx = sparse_indices;
  a.block_table = block_table;
  a.seqlens = seqlens_kv;
  a.max_pages = max_pages_per_seq;
  a.page = page_size;
  a.ls = ls;
  a.topk = topk;
  a.batch = batch;
  a.sq = seqlen_q;
  a.sk = block_table ? 0 : seqlen_k;
  a.hq = 16;  // one head tile per token
  a.mode = sparse_mode;
  a.dump_k = dst;
  a.dump_rows = dump_rows;
  return hip_status(attn::launch_dump_sparse(a, as_stream(stream)),
                    "attn_debug_gather_sparse launch");
}

}  // extern "C"
