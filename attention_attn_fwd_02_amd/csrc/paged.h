// Paged KV-cache addressing, shared by the decode kernels and the gather used
// to test it bit for bit.
#pragma once
#include "device_common.h"

namespace attn {

// Element offset of the row (one token, one KV head) holding logical key j of
// sequence b: logical page j / page_size of b maps to physical page
// block_table[b * max_pages + j / page_size]; the key sits in slot
// j % page_size of it. A physical page is page_size tokens x hkv heads x
// row_elems contiguous elements (k_cache (pages, page_size, Hkv, D) of the
// MATE flash_attn_with_kvcache interface).
__device__ __forceinline__ size_t paged_row_offset(const int32_t* __restrict__ block_table,
                                                   int max_pages, int b, int j, int page_size,
                                                   int hkv, int kvh, int row_elems) {
  const int lp = j / page_size;
  const int slot = j - lp * page_size;
  const int phys = block_table[(size_t)b * max_pages + lp];
  return ((size_t)phys * page_size + slot) * (size_t)hkv * row_elems + (size_t)kvh * row_elems;
}

}  // namespace attn
