// attn_decode_paged_noalloc: plan + split decode + combine in one call, with
// the plan and the per-split partial results in a fixed device array of this
// library instead of caller workspaces, for callers that cannot allocate
// device memory. The kernels are those of attn_plan_splits,
// attn_decode_paged and attn_combine.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = (size_t)ATTN_NOALLOC_SCRATCH_BYTES;
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

// One copy per GPU, alive until the process ends. Host code never uses the
// array's name as an address: the kernels receive the per-device pointer from
// hipGetSymbolAddress below.
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t code, const char* fmt, ...) {
  char msg[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof(msg), fmt, ap);
  va_end(ap);
  return attn::set_error(code, msg);
}

// The device address of `scratch` on the current device, looked up once per
// device (on the first call there), with that device current.
int32_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_EUNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ATTN_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_paged_noalloc_bytes(int32_t batch, int32_t seqlen_q, int32_t hq, int32_t dv,
                                       int32_t max_splits) {
  if (batch <= 0 || seqlen_q <= 0 || hq <= 0 || dv <= 0 || max_splits <= 0) return 0;
  const size_t rows = (size_t)batch * max_splits * seqlen_q * hq;
  return round_up(attn_plan_words(batch, max_splits) * sizeof(int32_t)) +
         round_up(rows * dv * sizeof(float)) + round_up(rows * sizeof(float));
}

int32_t attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_pages_per_seq,
                                  const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t dv,
                                  int32_t page_size, int32_t dtype, float scale, int32_t causal,
                                  const float* sinks, int32_t num_cu, int32_t waves,
                                  int32_t max_splits, int32_t min_blocks, void* out, float* lse,
                                  void* stream) {
  // every host check (those of the three calls below, and the size) comes
  // before any HIP call or device work
  int32_t st = attn::check_decode_args(q, k_cache, v_cache, block_table, max_pages_per_seq,
                                       cache_seqlens, batch, seqlen_q, hq, hkv, d, dv, page_size,
                                       dtype, scale, max_splits);
  if (st != ATTN_OK) return st;
  if (!out) return fail(ATTN_EINVAL, "null tensor pointer");
  if ((uintptr_t)out & 15) return fail(ATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  if (num_cu <= 0 || waves <= 0 || min_blocks <= 0)
    return fail(ATTN_EINVAL, "num_cu, waves, min_blocks must be > 0");
  const size_t need = attn_decode_paged_noalloc_bytes(batch, seqlen_q, hq, dv, max_splits);
  if (need > kScratchBytes)
    return fail(ATTN_EINVAL,
                "plan and partials need %zu bytes, above the %zu-byte scratch of the "
                "no-allocation decode (lower max_splits or the batch)",
                need, kScratchBytes);
  void* base = nullptr;
  st = scratch_ptr(&base);
  if (st != ATTN_OK) return st;
  char* p = static_cast<char*>(base);
  int32_t* plan = reinterpret_cast<int32_t*>(p);
  float* o_part = reinterpret_cast<float*>(p + round_up(attn_plan_words(batch, max_splits) * 4));
  const size_t rows = (size_t)batch * max_splits * seqlen_q * hq;
  float* lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(o_part) +
                                             round_up(rows * dv * sizeof(float)));
  // rows of one KV head per decode workgroup: 16 (GQA tile), 128 (MLA tile)
  const int tile_rows = (d == 576 && dv == 512) ? 128 : 16;
  const int units = hkv * ((seqlen_q * (hq / hkv) + tile_rows - 1) / tile_rows);
  st = attn_plan_splits(cache_seqlens, batch, page_size, units, num_cu, waves, max_splits,
                        min_blocks, plan, stream);
  if (st != ATTN_OK) return st;
  st = attn_decode_paged(q, k_cache, v_cache, block_table, max_pages_per_seq, cache_seqlens,
                         batch, seqlen_q, hq, hkv, d, dv, page_size, dtype, scale, causal, plan,
                         max_splits, o_part, lse_part, stream);
  if (st != ATTN_OK) return st;
  return attn_combine(o_part, lse_part, plan, batch, seqlen_q, hq, dv, max_splits, sinks,
                      ATTN_BF16, out, lse, stream);
}

}  // extern "C"
