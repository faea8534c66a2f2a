// Kernel argument blocks and launchers (host side). The C ABI in attn_api.hip
// validates arguments and then calls these; each returns hipSuccess or the
// launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct VarlenArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch, hq, hkv, nqt;   // nqt: query tiles per sequence (grid bound)
  int32_t causal, wl, wr;
  float scale_log2;              // softmax scale * log2(e)
  const float* sinks;
  void* out;
  float* lse;
  // keys of sequence b = cache rows [0, cache_lens[b]) followed by its current
  // rows (attn_fwd_varlen_kvcache); unused by attn_fwd_varlen
  const void* kc;
  const void* vc;
  const int32_t* block_table;
  const int32_t* cache_lens;
  int32_t max_pages, page;
  // optional additive mask (mask_heads, Tq, mask_ld) bf16 added to the scaled
  // scores; column = key position of the query's sequence
  const void* mask;
  int32_t mask_heads, mask_ld;
  // FP8 inputs (attn_fwd_varlen_fp8): descales (batch, hkv) float32, NULL = 1
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  // second query (Tq, hq, dv) scored against the value rows (launch_varlen_qv)
  const void* qv;
  // gather test: the DUMP instances copy every staged tile to dump_k / dump_v
  // (key rows of sequence b at row b * dump_rows + key, heads interleaved)
  void* dump_k;
  void* dump_v;
  int32_t dump_rows;
};

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;               // unused when K and V share the cache row
  const int32_t* block_table;
  const int32_t* lens;
  const int32_t* plan;
  int32_t max_pages, batch, sq, hq, hkv, page, causal, max_splits;
  float scale_log2;
  float* o_part;
  float* lse_part;
  // FP8 caches: descales (batch, hkv) float32, NULL = 1
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  // second query (B, Sq, Hq, Dv) scored against the value rows, or NULL;
  // only_qv: that score path alone (q and the K cache are not read)
  const void* qv;
  int32_t only_qv;
  // additive bf16 mask (batch, mask_heads, sq, mask_ld) over the cache keys,
  // or NULL
  const void* mask;
  int32_t mask_heads, mask_ld;
  // gather test: the DUMP instances copy every staged tile to dump_k / dump_v
  // (key rows of sequence b at row b * dump_rows + key, heads interleaved)
  void* dump_k;
  void* dump_v;
  int32_t dump_rows;
};

struct SparseArgs {
  const void* q;
  const void* kv;               // (B, sk, 1, D), or the page pool when block_table is set
  const int32_t* idx;
  const int32_t* block_table;   // NULL: dense layout; else (B, max_pages)
  const int32_t* seqlens;       // paged: keys per sequence
  int32_t max_pages, page;
  int32_t ls;                   // log2 of the sparse block size
  int32_t topk, batch, sq, sk, hq, mode;
  float scale_log2;
  const float* sinks;
  void* out;
  float* lse;
  // gather test: the DUMP instances copy every staged tile to dump_k / dump_v
  // (key rows of sequence b at row b * dump_rows + key, heads interleaved)
  void* dump_k;
  void* dump_v;
  int32_t dump_rows;
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  const int32_t* plan;
  int32_t batch, sq, hq, dv, max_splits, out_bf16;
  const float* sinks;
  void* out;
  float* lse;
};

// Host-side helpers of the C ABI (attn_api.hip): sets the message that
// attn_last_error() returns and passes the status through; the host checks
// of attn_decode_paged other than its plan and partial buffers.
int32_t set_error(int32_t code, const char* msg);
int32_t check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                          int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                          int32_t dtype, float scale, int32_t max_splits);

// rows per workgroup of each instance (sizes the grids)
int varlen_bf16_rows(int d);  // also the FP8 instance (d = 128)
int varlen_f32_rows(int d);

hipError_t launch_varlen_bf16(const VarlenArgs& a, int d, hipStream_t s);
hipError_t launch_varlen_f32(const VarlenArgs& a, int d, hipStream_t s);
hipError_t launch_varlen_kvcache_bf16(const VarlenArgs& a, int d, hipStream_t s);  // mask: a.mask
hipError_t launch_varlen_kvcache_qv_bf16(const VarlenArgs& a, hipStream_t s);  // d = dv = 128
hipError_t launch_varlen_fp8(const VarlenArgs& a, int fmt, hipStream_t s);  // d = 128
hipError_t launch_varlen_kvcache_fp8(const VarlenArgs& a, int fmt, hipStream_t s);  // d = 128
// q.k + qv.v scores; fmt 0 bf16, 1 e4m3, 2 e5m2; d = dv = 128
hipError_t launch_varlen_qv(const VarlenArgs& a, int fmt, hipStream_t s);
hipError_t launch_decode_gqa(const DecodeArgs& a, int d, hipStream_t s);  // d = dv in {64, 128}
hipError_t launch_decode_gqa_fp8(const DecodeArgs& a, int fmt, hipStream_t s);  // fmt 1 e4m3, 2 e5m2
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t s);
hipError_t launch_sparse_mla(const SparseArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_plan(const int32_t* lens, int batch, int page, int upb, int num_cu, int waves,
                       int max_splits, int min_blocks, int32_t* plan, hipStream_t s);
// DUMP instances of the paged kernels (gather test): the same grids and
// tile issue as the kernels above, with the staged tiles copied out.
hipError_t launch_dump_decode(const DecodeArgs& a, int d, int fmt, hipStream_t s);  // fmt 0 bf16
hipError_t launch_dump_mla(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dump_sparse(const SparseArgs& a, hipStream_t s);
hipError_t launch_dump_kvcache(const VarlenArgs& a, int fmt, hipStream_t s);  // d = 128

}  // namespace attn
