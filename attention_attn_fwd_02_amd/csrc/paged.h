// Paged KV-cache addressing. Every kernel that reads a paged cache (the GQA
// and MLA decodes, the cache-plus-current prefill, block-sparse MLA) takes
// its cache rows from the two functions below, and so do their DUMP
// instances, which copy the staged tiles out for the bit-exact gather test.
//
// [MATE "Attention" page, FMHA: flash_attn_with_kvcache with k_cache
//  (num_blocks, page_block_size, Hkv, D) and block_table (B, max_pages):
//  logical key j of sequence b sits in physical page block_table[b][j / page],
//  slot j % page.] The cache slot of a key is its row index in the pool
// viewed as (num_blocks * page) token rows: phys * page + j % page.
#pragma once
#include "device_common.h"
#include "prefill_bf16.h"  // sload2_uniform

namespace attn {

// Cache slot of logical key j, given the physical page that holds it.
__device__ __forceinline__ long slot_in_page(int phys, int j, int page) {
  return (long)phys * page + j % page;
}

// Per-lane form: btb is the sequence's block-table row, read with a vector
// load (used where the key differs per lane, e.g. staging a sparse key list).
__device__ __forceinline__ long paged_slot(const int32_t* __restrict__ btb, int j, int page) {
  return slot_in_page(btb[j / page], j, page);
}

// Wave-uniform form for a key tile: sl[k] is the cache slot of tile row 16 k,
// the first key of the tile's k-th 16-row block, with keys past jlast clamped
// to jlast. Page sizes are multiples of 16 and tiles start at multiples of 16
// from a page boundary, so each block lies on one page and row 16 k + r of the
// tile (r < 16, key <= jlast) is slot sl[k] + r. The block-table entries are
// read through the scalar cache, two per asm block with their own lgkmcnt wait
// (sload2_uniform): a vector load here would be followed by a vmcnt wait that
// also waits for every tile DMA in flight.
template <int NB>
__device__ __forceinline__ void paged_block_slots(const int32_t* __restrict__ btb, int page, int j0,
                                                  int jlast, long (&sl)[NB]) {
  static_assert(NB % 2 == 0, "blocks are read in pairs");
  static_for<NB / 2>([&](auto I) {
    constexpr int k = 2 * decltype(I)::value;
    const int ja = min(j0 + 16 * k, jlast), jb = min(j0 + 16 * (k + 1), jlast);
    int pa, pb;
    sload2_uniform(btb + ja / page, btb + jb / page, pa, pb);
    sl[k] = slot_in_page(pa, ja, page);
    sl[k + 1] = slot_in_page(pb, jb, page);
  });
}

// sl[rb] for a block index rb known only at run time (a select chain over the
// compile-time indices, so sl stays in registers).
template <int NB>
__device__ __forceinline__ long block_slot(const long (&sl)[NB], int rb) {
  long v = sl[0];
  static_for<NB - 1>([&](auto I) {
    if (rb == decltype(I)::value + 1) v = sl[decltype(I)::value + 1];
  });
  return v;
}

}  // namespace attn
