/*
 * attn.h - C ABI of libattn_mi355.so: fused scaled-dot-product attention
 * forward for AMD Instinct MI355X (gfx950).
 *
 * Every entry point computes, tile by tile and without materialising the
 * score matrix,
 *     S = scale * Q K^T,  O = softmax(S) V,  LSE = log sum exp(S - max S) + max S
 * (attention and softmax_lse formulas of the CANN ops-transformer "flash_attn"
 * page), with the masks and layouts described per function.
 *
 * Conventions shared by all calls
 *  - Tensor arguments are DEVICE pointers, allocated and owned by the caller,
 *    dense row-major in the shapes given. The library never allocates device
 *    memory and keeps no pointer after the call returns. Element tensors
 *    (Q, K, V, caches, masks, outputs, partials) must be 16-byte aligned
 *    (ATTN_EINVAL otherwise): the kernels move 16-byte vectors.
 *  - Scalar arguments (sizes, flags, scale) are host values. scale must be
 *    positive and finite (ATTN_EINVAL otherwise): the kernels track the row
 *    maximum of the scaled scores through the maximum of the raw ones.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it and returns without synchronising.
 *  - bfloat16 tensors hold raw 16-bit patterns; results are rounded to
 *    bfloat16 to nearest-even. LSE is float32, natural log.
 *  - Query head h reads KV head h / (Hq / Hkv) (grouping (N2, N1/N2) of the
 *    MindSpore "sparse_flash_attention" page).
 *  - Causal masks are bottom-right aligned: query t of a sequence with Lq
 *    queries and Lk keys sees key j iff j <= t + (Lk - Lq) (rightDownCausal
 *    mode of the same page). A row that sees no key gets O = 0, LSE = -inf.
 *  - Errors: host-side argument checks return an error before any device
 *    work is enqueued. A zero-sized required dimension is ATTN_EEMPTY (the
 *    flash_attn page rejects empty tensors). The CONTENTS of device tensors
 *    (cu_seqlens, block_table, cache_seqlens, indices, plan) are not checked:
 *    out-of-range values are undefined behaviour, as on the flash_attn page.
 *    attn_last_error() returns a thread-local message for the last failure.
 */
#ifndef ATTN_MI355_H
#define ATTN_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* bad argument (null pointer, inconsistent sizes) */
  ATTN_EUNSUPPORTED = 2,  /* valid but not implemented (head dims, dtype)    */
  ATTN_EEMPTY = 3,        /* a required dimension is zero                    */
  ATTN_EHIP = 4           /* HIP runtime error (launch, device query)        */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1, ATTN_FP8_E4M3 = 2, ATTN_FP8_E5M2 = 3 } attn_dtype;

/* kernels whose page gather attn_debug_gather_paged runs (test only) */
typedef enum { ATTN_GATHER_DECODE = 0, ATTN_GATHER_MLA = 1 } attn_gather_kernel;

/* Human-readable name of a status code. Never NULL. */
const char* attn_status_string(int32_t status);

/* Message describing the last failing call on this thread ("" if none). */
const char* attn_last_error(void);

/* Number of compute units of `device` (host output). */
int32_t attn_device_info(int32_t device, int32_t* num_cu);

/*
 * attn_fwd_varlen - packed variable-length attention (prefill).
 * [MATE "Attention" page, FMHA: flash_attn_varlen_func; CANN flash_attn:
 *  cu_seqlens_q / cu_seqlens_kv; lite_boost flash_attention: causal,
 *  window_size]
 *
 *  q   (Tq, hq, d)     k (Tk, hkv, d)     v (Tk, hkv, dv)     dtype elements
 *  cu_seqlens_q, cu_seqlens_k: int32 (batch+1) prefix sums, [0] = 0; sequence
 *      b owns query rows [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]).
 *  max_seqlen_q: host upper bound of the per-sequence query length (sizes the
 *      grid; rows past it are not computed). max_seqlen_k: host upper bound
 *      of the key length (informational, must be >= 0).
 *  window_left / window_right: inclusive band around the causal diagonal,
 *      -1 = unbounded; causal != 0 is the same as window_right = 0.
 *  sinks: NULL or float32 (hq) sink logits (scaled-score domain): the output
 *      becomes sum e^{S-m} V / (sum e^{S-m} + e^{sink-m}), m = max(sink, max S)
 *      [CANN flash_attn sink formulas]; LSE stays sink-free.
 *  out (Tq, hq, dv) dtype;  lse: NULL or float32 (hq, Tq).
 *  Supported: dtype BF16 with d = dv in {64, 128}; dtype F32 with d = dv in
 *  {64, 128}. Others return ATTN_EUNSUPPORTED.
 */
int32_t attn_fwd_varlen(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t dtype,
                        float scale, int32_t causal, int32_t window_left, int32_t window_right,
                        const float* sinks, void* out, float* lse, void* stream);

/*
 * attn_fwd_varlen_fp8 - attn_fwd_varlen with FP8 Q, K and V.
 * [MATE "Attention" page, FMHA forward dtype notes: float8_e4m3fn and
 *  float8_e5m2 inputs of flash_attn_varlen_func; optional float32 q_descale,
 *  k_descale, v_descale of shape (batch_size, num_heads_kv); FP8 inputs give
 *  bfloat16 outputs]
 *
 *  q (Tq, hq, 128), k (Tk, hkv, 128), v (Tk, hkv, 128): 8-bit codes of
 *  fp8_format (ATTN_FP8_E4M3 or ATTN_FP8_E5M2, as in attn_decode_paged_fp8).
 *  q_descale, k_descale, v_descale: NULL (= 1) or float32 (batch, hkv); the
 *  real value of a code of sequence b and KV head g is code * descale[b][g],
 *  query head h using its KV head g = h / (hq / hkv). Descales must be
 *  positive and finite (not checked).
 *  out (Tq, hq, 128) bfloat16; lse NULL or float32 (hq, Tq). Sequences,
 *  masks, sinks and errors are as in attn_fwd_varlen.
 *  Supported: d = dv = 128. Scores are exact products of the codes summed in
 *  float32; the probabilities and V are used as in the bfloat16 path.
 */
int32_t attn_fwd_varlen_fp8(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t fp8_format,
                            const float* q_descale, const float* k_descale,
                            const float* v_descale, float scale, int32_t causal,
                            int32_t window_left, int32_t window_right, const float* sinks,
                            void* out, float* lse, void* stream);

/*
 * attn_fwd_varlen_qv - attn_fwd_varlen with a second query qv scored against
 * the value rows (bf16 or FP8 inputs).
 * [MATE "Attention" page, FMHA forward notes: optional qv input on the FMHA
 *  forward path, also with FP8 inputs (q_descale then applies to both query
 *  tensors); only_qv skips the QK score path]
 *
 *  q (Tq, hq, 128), qv (Tq, hq, 128), k (Tk, hkv, 128), v (Tk, hkv, 128),
 *  sequences as in attn_fwd_varlen. The score of key j for query head h
 *  (KV head g = h / (hq / hkv)) is
 *      scale * (q . k_j + qv . v_j)     (only_qv = 0)
 *      scale * (qv . v_j)               (only_qv != 0; q and k are then not
 *                                        read and may be NULL)
 *  on the real values; masks, sinks, output and LSE are those of
 *  attn_fwd_varlen over these scores. out (Tq, hq, 128) bfloat16; lse NULL or
 *  float32 (hq, Tq).
 *  dtype: ATTN_BF16 (descales must be NULL), ATTN_FP8_E4M3 or ATTN_FP8_E5M2
 *  (codes; descales as in attn_fwd_varlen_fp8, qv using q_descale).
 *  Errors as in attn_fwd_varlen. Supported: d = dv = 128.
 */
int32_t attn_fwd_varlen_qv(const void* q, const void* qv, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                           int32_t hkv, int32_t d, int32_t dv, int32_t dtype,
                           const float* q_descale, const float* k_descale,
                           const float* v_descale, float scale, int32_t causal,
                           int32_t window_left, int32_t window_right, const float* sinks,
                           int32_t only_qv, void* out, float* lse, void* stream);

/*
 * attn_fwd_varlen_mask - attn_fwd_varlen (bfloat16) with an additive mask.
 * [Modular flash_attention_split_kv: input_mask_fn loads additive mask
 *  values; CANN flash_attn: attn_mask (its tables are garbled, so only the
 *  additive form is taken)]
 *
 *  Arguments as attn_fwd_varlen with dtype ATTN_BF16, plus
 *  mask: bf16 (mask_heads, Tq, mask_ld), 16-byte aligned: query row r
 *      (packed index) of head h adds mask[h or 0][r][j] to its scaled score
 *      with key j of its sequence (0 <= j < Lk); -inf removes the key, and a
 *      row with every key removed is empty (O = 0, LSE = -inf). It is added
 *      after the causal and window masks.
 *  mask_heads: 1 (shared by all heads) or hq.
 *  mask_ld: a multiple of 64, at least max_seqlen_k (columns up to every
 *      sequence's Lk rounded up to 32 are read).
 *  Errors: EINVAL for a NULL mask or the mask arguments above, the rest as
 *  attn_fwd_varlen; supported d = dv in {64, 128}.
 */
int32_t attn_fwd_varlen_mask(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t hq,
                             int32_t hkv, int32_t d, int32_t dv, float scale, int32_t causal,
                             int32_t window_left, int32_t window_right, const float* sinks,
                             const void* mask, int32_t mask_heads, int32_t mask_ld, void* out,
                             float* lse, void* stream);

/*
 * attn_fwd_varlen_kvcache - packed queries over a paged cache of earlier
 * tokens followed by the current K/V rows, without concatenating them
 * (chunked / append prefill).
 * [Modular flash_attention_split_kv: the previous KV cache and the current
 *  K/V are separate inputs; MATE flash_attn_with_kvcache: paged k_cache with
 *  block_table and cache_seqlens]
 *
 *  q (Tq, hq, d); k (Tk, hkv, d), v (Tk, hkv, dv): the current tokens, as in
 *      attn_fwd_varlen (cu_seqlens_q, cu_seqlens_k); k and v may be NULL when
 *      Tk = 0 (queries over cached keys only).
 *  k_cache (P, page_size, hkv, d), v_cache (P, page_size, hkv, dv); int32
 *      block_table (batch, max_pages_per_seq); int32 cache_seqlens (batch):
 *      sequence b has cache_seqlens[b] earlier tokens, row j at page
 *      block_table[b][j / page_size], slot j % page_size; the current tokens
 *      are not in the cache.
 *  The keys of b are its cached rows 0 .. Lc-1 followed by its current rows,
 *  Lk = Lc + Ln; causal and window masks are those of attn_fwd_varlen over
 *  that sequence (bottom-right: query t sits at position t + Lk - Lq).
 *  out (Tq, hq, dv); lse NULL or float32 (hq, Tq); sinks as attn_fwd_varlen.
 *  mask: NULL or a bf16 additive mask (mask_heads, Tq, mask_ld) [Modular
 *  flash_attention_split_kv input_mask_fn: additive mask values]: query row
 *  r (packed index) of head h adds mask[h or 0][r][j] to its scaled score
 *  with key j of its sequence (cache rows first); -inf removes the key.
 *  mask_heads is 1 (shared by all heads) or hq; mask_ld is a multiple of 64
 *  and at least every sequence's Lk rounded up to 64 (columns up to that are
 *  read); the mask is 16-byte aligned.
 *  Supported: dtype BF16, d = dv in {64, 128}, page_size a multiple of 16.
 *  Block-table entries past ceil(Lc / page_size) are never read. Device
 *  values are not checked: the caller keeps 0 <= cache_seqlens[b] <=
 *  max_pages_per_seq * page_size and every referenced entry a page of the
 *  pool. Host arguments are checked as for attn_fwd_varlen (EEMPTY, EINVAL,
 *  EUNSUPPORTED) before anything is enqueued.
 */
int32_t attn_fwd_varlen_kvcache(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* cache_seqlens, int32_t page_size, int32_t batch,
                                int32_t max_seqlen_q, int32_t hq, int32_t hkv, int32_t d,
                                int32_t dv, int32_t dtype, float scale, int32_t causal,
                                int32_t window_left, int32_t window_right, const float* sinks,
                                const void* mask, int32_t mask_heads, int32_t mask_ld,
                                void* out, float* lse, void* stream);

/*
 * attn_fwd_varlen_kvcache_qv - attn_fwd_varlen_kvcache (bfloat16) with a
 * second query qv scored against the value rows, cached and current.
 * [MATE "Attention" page, FMHA notes: the optional qv input and only_qv
 *  flag of the forward functions; Modular flash_attention_split_kv: cache and
 *  current K/V as separate inputs]
 *
 *  qv (Tq, hq, dv) bf16: the score of query row r with key j is
 *      scale * (q_r . k_j + qv_r . v_j), or scale * qv_r . v_j with
 *      only_qv != 0 (q, k and k_cache are then not read and may be NULL).
 *  The other arguments, the key sequence (cached rows first), the masks,
 *  sinks, outputs and errors are those of attn_fwd_varlen_kvcache without
 *  an additive mask.
 *  Supported: d = dv = 128, page_size a multiple of 16.
 */
int32_t attn_fwd_varlen_kvcache_qv(const void* q, const void* qv, const void* k, const void* v,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_pages_per_seq,
                                   const int32_t* cache_seqlens, int32_t page_size,
                                   int32_t batch, int32_t max_seqlen_q, int32_t hq, int32_t hkv,
                                   int32_t d, int32_t dv, float scale, int32_t causal,
                                   int32_t window_left, int32_t window_right,
                                   const float* sinks, int32_t only_qv, void* out, float* lse,
                                   void* stream);

/*
 * attn_fwd_varlen_kvcache_fp8 - attn_fwd_varlen_kvcache with FP8 Q, K, V and
 * caches (chunked / append prefill on FP8 inputs).
 * [MATE "Attention" page, FMHA forward dtype notes: the varlen and KV-cache
 *  forward paths take float8_e4m3fn / float8_e5m2 with optional float32
 *  q/k/v_descale of shape (batch, num_heads_kv), bf16 output; Modular
 *  flash_attention_split_kv: cache and current K/V as separate inputs]
 *
 *  Arguments as attn_fwd_varlen_kvcache, with q, k, v, k_cache and v_cache
 *  uint8 codes of fp8_format (ATTN_FP8_E4M3 or ATTN_FP8_E5M2) and no mask.
 *  q_descale, k_descale, v_descale: NULL (= 1) or float32 (batch, hkv). The
 *  real value of an element of sequence b is its FP8 value times the descale
 *  of (b, its KV head), for cached and current rows alike (the descale belongs
 *  to the sequence, not to the page); a query head uses its KV head's
 *  q_descale. out (Tq, hq, 128) bf16; lse NULL or float32 (hq, Tq).
 *  Supported: d = dv = 128, page_size a multiple of 16. Device values are not
 *  checked (as attn_fwd_varlen_kvcache); host arguments are checked before
 *  anything is enqueued (EEMPTY, EINVAL, EUNSUPPORTED).
 */
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
                                    const float* sinks, void* out, float* lse, void* stream);

/*
 * Split-KV plan for paged decode.
 * [MATE: get_scheduler_metadata / get_mla_metadata precompute the work split;
 *  CANN flash_attn_metadata does the same before the main call. The rule
 *  below is this library's own.]
 *
 *  attn_plan_words: number of int32 words of a plan buffer.
 *  attn_plan_splits: enqueues one small kernel that reads cache_seqlens
 *  (device int32, batch) and writes `plan` (device int32, attn_plan_words):
 *    plan[0] = total splits, plan[1] = pages per split target (bps),
 *    plan[2 .. 2+batch] = split_ptr (exclusive prefix sum, batch+1 words),
 *    then one (batch, kv_start, kv_end) triple per split, batch-major
 *    (batch * max_splits triples reserved), then the work order: batch *
 *    max_splits words of which the first plan[0] are the split indices in
 *    the order the decode workgroups take them, longest split
 *    (kv_end - kv_start) first and ties in split order, or in split order
 *    when there are more than 4096 splits.
 *  Rule: nblk = ceil(len / page_size) (0 if len <= 0);
 *        bps  = max(min_blocks, ceil(sum nblk * units_per_block / (num_cu * waves)));
 *        ns   = min(max_splits, max(1, ceil(nblk / bps))), pps = ceil(nblk / ns),
 *        ns   = ceil(nblk / pps); split s = tokens [s*pps*page, min((s+1)*pps*page, len)).
 *  Empty sequences get no split. max_splits must be in [1, 16].
 *  The same plan must be passed unchanged to the decode and combine calls.
 */
size_t attn_plan_words(int32_t batch, int32_t max_splits);
int32_t attn_plan_splits(const int32_t* cache_seqlens, int32_t batch, int32_t page_size,
                         int32_t units_per_block, int32_t num_cu, int32_t waves,
                         int32_t max_splits, int32_t min_blocks, int32_t* plan, void* stream);

/*
 * attn_decode_paged - split-KV attention of a few query tokens against a
 * paged KV cache; writes per-split partial results for attn_combine.
 * [MATE FMHA: flash_attn_with_kvcache with k_cache (pages, page_size, Hkv, D),
 *  block_table and cache_seqlens; a non-empty block_table enables paged
 *  attention (CANN flash_attn)]
 *
 *  q (batch, seqlen_q, hq, d); k_cache (P, page_size, hkv, d);
 *  v_cache (P, page_size, hkv, dv); block_table int32 (batch, max_pages_per_seq):
 *  logical page i of sequence b is physical page block_table[b*max_pages_per_seq+i];
 *  cache_seqlens int32 (batch): keys 0..len-1 (the cache already holds the
 *  current tokens). causal: bottom-right over (seqlen_q, len).
 *  plan: from attn_plan_splits with the same cache_seqlens and max_splits.
 *  o_partial float32 (batch*max_splits, seqlen_q*hq, dv), lse_partial float32
 *  (batch*max_splits, seqlen_q*hq): split s of b writes slot b*max_splits+s,
 *  row t*hq+h, normalised within the split. Unused slots are untouched.
 *  Supported: BF16, d = dv in {64, 128}, page_size a multiple of 16; and the
 *  MLA-absorbed row d = 576, dv = 512 for any hkv (the MATE MLA example has
 *  Hkv = 2): the key is the whole cached row, the value its first 512
 *  entries, and v_cache must then be NULL or equal to k_cache.
 */
int32_t attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                          int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                          int32_t dtype, float scale, int32_t causal, const int32_t* plan,
                          int32_t max_splits, float* o_partial, float* lse_partial,
                          void* stream);

/*
 * attn_decode_paged_mask - attn_decode_paged (bfloat16, GQA) with an
 * additive mask on the scores.
 * [Modular flash_attention_split_kv: input_mask_fn loads additive mask
 *  values; MATE flash_attn_with_kvcache: paged k_cache / v_cache]
 *
 *  Arguments as attn_decode_paged with dtype bfloat16, plus
 *  mask: bf16 (batch, mask_heads, seqlen_q, mask_ld), 16-byte aligned: query
 *      token t of sequence b and head h add mask[b][h or 0][t][j] to the
 *      scaled score with cached key j (0 <= j < cache_seqlens[b]); -inf
 *      removes the key. Added after the causal mask; partials and the
 *      combine as attn_decode_paged.
 *  mask_heads: 1 (shared by all heads) or hq.
 *  mask_ld: a multiple of 64; the caller keeps it >= every cache_seqlens[b]
 *      (columns up to cache_seqlens[b] rounded up to 32 are read; device
 *      values are not checked).
 *  Supported: d = dv in {64, 128}, separate V cache. Errors: EINVAL for a
 *  NULL mask or the mask arguments above, the rest as attn_decode_paged.
 */
int32_t attn_decode_paged_mask(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t max_pages_per_seq,
                               const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                               int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                               float scale, int32_t causal, const void* mask, int32_t mask_heads,
                               int32_t mask_ld, const int32_t* plan, int32_t max_splits,
                               float* o_partial, float* lse_partial, void* stream);

/*
 * attn_decode_paged_fp8 - attn_decode_paged with FP8 query and cache.
 * [MATE "Attention" page, FMHA forward dtype notes: float8_e4m3fn and
 *  float8_e5m2 inputs of flash_attn_with_kvcache; optional float32 q_descale,
 *  k_descale, v_descale of shape (batch_size, num_heads_kv); FP8 inputs give
 *  bfloat16 outputs]
 *
 *  q (B, Sq, Hq, 128), k_cache / v_cache (P, page_size, Hkv, 128) hold 8-bit
 *  codes of fp8_format: ATTN_FP8_E4M3 (e4m3fn: bias 7, no infinities, max
 *  448) or ATTN_FP8_E5M2 (bias 15, IEEE-style infinities and NaN).
 *  q_descale, k_descale, v_descale: NULL (= 1) or float32 (B, Hkv). The real
 *  value of a code of sequence b and KV head g is code * descale[b][g]; query
 *  head h uses the descale of its KV head g = h / (Hq / Hkv). Descales must
 *  be positive and finite (not checked).
 *  Everything else (block table, plan, partial layouts, masks, errors) is as
 *  in attn_decode_paged; attn_combine then gives the bfloat16 O and the LSE.
 *  Supported: d = dv = 128, page_size a multiple of 16.
 */
int32_t attn_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, int32_t max_pages_per_seq,
                              const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                              int32_t hq, int32_t hkv, int32_t d, int32_t dv, int32_t page_size,
                              int32_t fp8_format, const float* q_descale,
                              const float* k_descale, const float* v_descale, float scale,
                              int32_t causal, const int32_t* plan, int32_t max_splits,
                              float* o_partial, float* lse_partial, void* stream);

/*
 * attn_decode_paged_qv - attn_decode_paged with a second query qv scored
 * against the value rows (bf16 or FP8 inputs).
 * [MATE "Attention" page, FMHA forward notes: optional qv input, also with
 *  FP8 inputs (q_descale then applies to both query tensors);
 *  flash_attn_with_kvcache(only_qv=True) skips the QK score path, q and
 *  k_cache may then be None]
 *
 *  qv (B, Sq, Hq, dv), same element type as the caches. The score of key j
 *  for query head h (KV head g = h / (Hq / Hkv)) is
 *      scale * (q . k_j + qv . v_j)       (only_qv = 0)
 *      scale * (qv . v_j)                 (only_qv != 0; q and k_cache are
 *                                          then not read and may be NULL)
 *  on the real values; softmax, output (the partials, then attn_combine) and
 *  LSE are those of attn_decode_paged over these scores.
 *  dtype: ATTN_BF16 (descales must be NULL), ATTN_FP8_E4M3 or ATTN_FP8_E5M2
 *  (codes, descales as in attn_decode_paged_fp8; qv uses q_descale).
 *  Everything else (block table, plan, partial layouts, causal, errors) is
 *  as in attn_decode_paged. Supported: d = dv = 128, page_size a multiple of
 *  16.
 */
int32_t attn_decode_paged_qv(const void* q, const void* qv, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* cache_seqlens,
                             int32_t batch, int32_t seqlen_q, int32_t hq, int32_t hkv, int32_t d,
                             int32_t dv, int32_t page_size, int32_t dtype,
                             const float* q_descale, const float* k_descale,
                             const float* v_descale, float scale, int32_t causal,
                             int32_t only_qv, const int32_t* plan, int32_t max_splits,
                             float* o_partial, float* lse_partial, void* stream);

/*
 * attn_combine - LSE-weighted merge of split results.
 * [MATE FMHA: flash_attn_combine merges partial outputs and LSE buffers;
 *  CANN flash_attn: softmax_lse definition]
 *  For each output row: M = max_s LSE_s, w_s = e^{LSE_s - M},
 *  LSE = M + log sum w_s, O = sum w_s O_s / sum w_s. With sinks (float32 hq,
 *  or NULL) the sink of the row's head adds e^{sink - M*} to the denominator,
 *  M* = max(M, sink); LSE stays sink-free. No split or all LSE_s = -inf gives
 *  O = 0, LSE = -inf.
 *  out (batch, seqlen_q, hq, dv) in out_dtype (BF16 or F32);
 *  lse: NULL or float32 (batch, hq, seqlen_q).
 */
int32_t attn_combine(const float* o_partial, const float* lse_partial, const int32_t* plan,
                     int32_t batch, int32_t seqlen_q, int32_t hq, int32_t dv, int32_t max_splits,
                     const float* sinks, int32_t out_dtype, void* out, float* lse, void* stream);

/*
 * mla_decode_paged - MLA-absorbed split-KV decode: one KV head, each cached
 * row holds the 512-wide latent followed by the 64-wide rope part (d = 576);
 * the key is the whole row and the value is its first 512 entries.
 * [MATE MLA example: flash_mla_with_kvcache(q (B,Sq,Hq,576), k_cache
 *  (P,page,Hkv,576), head_dim_v=512); MindSpore sparse_flash_attention:
 *  MLA-absorb concat of nope and rope along D; CANN flash_attn: shared KV]
 *  q (batch, seqlen_q, hq, 576) bf16; kv_cache (P, page_size, 1, 576) bf16;
 *  other arguments and the partial layout (dv = 512) as attn_decode_paged;
 *  follow with attn_combine(dv = 512). page_size must be a multiple of 16.
 *  This is attn_decode_paged with hkv = 1, d = 576, dv = 512.
 */
int32_t mla_decode_paged(const void* q, const void* kv_cache, const int32_t* block_table,
                         int32_t max_pages_per_seq, const int32_t* cache_seqlens, int32_t batch,
                         int32_t seqlen_q, int32_t hq, int32_t page_size, float scale,
                         int32_t causal, const int32_t* plan, int32_t max_splits,
                         float* o_partial, float* lse_partial, void* stream);

/*
 * mla_sparse_fwd - top-k sparse MLA attention with optional sinks.
 * [MindSpore sparse_flash_attention: sparse_indices (B, Q_S, N2, 2048) select
 *  K~ = V~ rows, N2 = 1, D = 512 + 64 rope, sparse_mode 0 (all) / 3
 *  (rightDownCausal); CANN flash_attn sink formulas]
 *  q (batch, seqlen_q, hq, 576) bf16; kv (batch, seqlen_k, 1, 576) bf16;
 *  sparse_indices int32 (batch, seqlen_q, 1, topk): key rows of each query
 *  token, shared by all its heads; entries < 0 or >= seqlen_k are skipped,
 *  mode 3 also skips keys after t + (seqlen_k - seqlen_q); duplicates count
 *  each time; order is irrelevant. sinks: NULL or float32 (hq).
 *  out (batch, seqlen_q, hq, 512) bf16; lse: NULL or float32 (batch, hq, seqlen_q).
 *  hq must be a multiple of 16; seqlen_k at most 3728270 (row byte offsets
 *  inside one sequence are 32-bit). Skipped entries are fetched from row 0
 *  of the sequence and masked, so row 0 must hold finite values.
 */
int32_t mla_sparse_fwd(const void* q, const void* kv, const int32_t* sparse_indices, int32_t topk,
                       int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t hq, float scale,
                       int32_t sparse_mode, const float* sinks, void* out, float* lse,
                       void* stream);

/*
 * mla_sparse_paged_fwd - block-sparse MLA over a paged latent cache.
 * [MindSpore sparse_flash_attention: layout_kv "PA_BSND" with key of shape
 *  (block_num, block_size, N2, D) and block_table, actual_seq_lengths_kv,
 *  sparse_block_size in [1, 128], a power of two]
 *  q, out, lse, sinks, scale, sparse_mode as mla_sparse_fwd.
 *  kv_cache (num_blocks, page_size, 1, 576) bf16; int32 block_table (batch,
 *  max_pages_per_seq): key j of sequence b is row j % page_size of page
 *  block_table[b][j / page_size]; int32 seqlens_kv (batch): keys of each
 *  sequence (Lk_b).
 *  sparse_indices int32 (batch, seqlen_q, 1, topk): index i >= 0 selects the
 *  sparse_block_size keys i*s .. i*s + s - 1 (s = sparse_block_size; s = 1
 *  selects token i); keys >= Lk_b, and in mode 3 keys after
 *  t + (Lk_b - seqlen_q), are skipped; duplicates count each time.
 *  Supported: hq a multiple of 16, num_blocks * page_size at most 3728270
 *  rows (32-bit row byte offsets into the pool). Skipped keys are fetched
 *  from pool row 0 and masked, so it must hold finite values. Device values
 *  are not checked: referenced block-table entries must name pool pages.
 */
int32_t mla_sparse_paged_fwd(const void* q, const void* kv_cache, int32_t num_blocks,
                             int32_t page_size, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* seqlens_kv,
                             const int32_t* sparse_indices, int32_t topk,
                             int32_t sparse_block_size, int32_t batch, int32_t seqlen_q,
                             int32_t hq, float scale, int32_t sparse_mode, const float* sinks,
                             void* out, float* lse, void* stream);

/*
 * attn_decode_paged_noalloc - plan + attn_decode_paged + attn_combine in one
 * call that allocates nothing and takes no workspace: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 *  Arguments as attn_decode_paged (incl. the MLA row d = 576, dv = 512),
 *  with the planner arguments of attn_plan_splits (num_cu, waves,
 *  max_splits, min_blocks; units per block are derived from the shape) and
 *  the outputs of attn_combine: sinks NULL or float32 (hq); out (batch,
 *  seqlen_q, hq, dv) bf16; lse NULL or float32 (batch, hq, seqlen_q). The
 *  result equals that of the three calls made with the same arguments.
 *  The plan and the per-split partial results live in a device array of the
 *  library of ATTN_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs
 *  on, held until the process ends; attn_decode_paged_noalloc_bytes gives a
 *  call's need, and a call that needs more returns ATTN_EINVAL before any
 *  device work. Every call on one GPU uses that GPU's array: calls whose
 *  work overlaps on one GPU (other streams, other threads) race and must be
 *  serialised by the caller. The array keeps the last call's contents;
 *  nothing in it has to start at zero (the plan kernel writes every word the
 *  decode and the combine read). The current device must be the stream's.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
size_t attn_decode_paged_noalloc_bytes(int32_t batch, int32_t seqlen_q, int32_t hq, int32_t dv,
                                       int32_t max_splits);
int32_t attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_pages_per_seq,
                                  const int32_t* cache_seqlens, int32_t batch, int32_t seqlen_q,
                                  int32_t hq, int32_t hkv, int32_t d, int32_t dv,
                                  int32_t page_size, int32_t dtype, float scale, int32_t causal,
                                  const float* sinks, int32_t num_cu, int32_t waves,
                                  int32_t max_splits, int32_t min_blocks, void* out, float* lse,
                                  void* stream);

/*
 * Test-only gather checks. Each runs a DUMP instance of a kernel that reads
 * a paged (or index-gathered) cache: the kernel's own work split, page-slot
 * computation, tile DMA and LDS ring, with every staged tile copied back out
 * of LDS (un-swizzled) instead of being computed on. A test compares the
 * copies bit for bit with the rows the page table names.
 * [MATE "Attention" page, FMHA: k_cache (num_blocks, page_block_size, Hkv, D)
 *  addressed through block_table and cache_seqlens]
 *
 * attn_debug_gather_paged - the decode kernels. kernel = ATTN_GATHER_DECODE
 *  (the GQA decode of attn_decode_paged / attn_decode_paged_fp8: dtype
 *  ATTN_BF16 with d in {64, 128}, or ATTN_FP8_E4M3 / ATTN_FP8_E5M2 with
 *  d = 128) or ATTN_GATHER_MLA (the wide MLA tile of mla_decode_paged: bf16
 *  rows of d = 576, v_cache and v_dst unused). Caches and block table as in
 *  attn_decode_paged; plan from attn_plan_splits(max_splits) over the same
 *  cache_seqlens. k_dst / v_dst (batch, dump_rows, hkv, d) elements of the
 *  cache type: key j < cache_seqlens[b] of KV head g is written to row
 *  (b, j, g); other rows are untouched. dump_rows >= max cache_seqlens.
 *
 * attn_debug_gather_kvcache - the cache-plus-current prefill of
 *  attn_fwd_varlen_kvcache (dtype ATTN_BF16) and attn_fwd_varlen_kvcache_fp8
 *  (ATTN_FP8_E4M3 / ATTN_FP8_E5M2), d = 128. Arguments as those calls (k, v
 *  the current rows, cu_seqlens_q the query rows per sequence: a sequence
 *  with no query row is not gathered). k_dst / v_dst (batch, dump_rows, hkv,
 *  d): key j of sequence b (its cache rows first, then its current rows) is
 *  written to row (b, j, g). dump_rows >= the longest key sequence.
 *
 * attn_debug_gather_sparse - the key gather of mla_sparse_fwd (block_table
 *  NULL: kv (batch, seqlen_k, 1, 576)) or mla_sparse_paged_fwd (kv the page
 *  pool, block_table, seqlens_kv, page_size). dst (batch, seqlen_q,
 *  dump_rows, 576) bf16: the expanded key list of token (b, t) (index i of
 *  a block size s names keys i*s .. i*s + s - 1), in order; a skipped key
 *  (negative index, past the length, or past the causal limit in mode 3)
 *  holds row 0 of the sequence (dense) or of the pool (paged), which the
 *  kernel fetches and masks. dump_rows >= topk * sparse_block_size.
 *
 *  Host checks as the calls they mirror; device contents are not checked.
 */
int32_t attn_debug_gather_paged(int32_t kernel, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* cache_seqlens, int32_t batch, int32_t hkv, int32_t d,
                                int32_t page_size, int32_t dtype, const int32_t* plan,
                                int32_t max_splits, int32_t dump_rows, void* k_dst, void* v_dst,
                                void* stream);
int32_t attn_debug_gather_kvcache(const void* k, const void* v, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int32_t max_pages_per_seq, const int32_t* cache_seqlens,
                                  int32_t page_size, int32_t batch, int32_t hkv, int32_t d,
                                  int32_t dtype, int32_t dump_rows, void* k_dst, void* v_dst,
                                  void* stream);
int32_t attn_debug_gather_sparse(const void* kv, int32_t seqlen_k, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const int32_t* seqlens_kv,
                                 int32_t page_size, const int32_t* sparse_indices, int32_t topk,
                                 int32_t sparse_block_size, int32_t batch, int32_t seqlen_q,
                                 int32_t sparse_mode, int32_t dump_rows, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355_H */
