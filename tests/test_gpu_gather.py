"""Bit-exact checks of the gather every paged kernel runs.

Each case calls a DUMP instance of a kernel through the C ABI: the kernel's
own work split, page-slot computation (paged.h), tile DMA and LDS ring, with
every staged tile copied back out of LDS un-swizzled instead of being
computed on. The copies must equal, bit for bit, the rows the page table
names: the oracle's gather_paged (logical key j of sequence b is row
j % page of page block_table[b, j // page]) [MATE "Attention" page, FMHA:
flash_attn_with_kvcache with k_cache and block_table].
"""
import numpy as np
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu


def host_bits(t):
    """Raw element bits of a device tensor (uint16 for bf16, uint8 codes)."""
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dev_bits(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint8:
        return torch.from_numpy(x).cuda()
    return dev(x)


def check_rows(name, got, lens, ref_rows):
    """got (B, rows, ...): rows [0, len_b) equal ref_rows(b) bit for bit and
    the rows after them were never written (still zero)."""
    for b, n in enumerate(lens):
        n = int(n)
        ref = ref_rows(b)
        assert ref.shape == got[b, :n].shape, (name, b, ref.shape, got[b, :n].shape)
        bad = np.nonzero(np.any((got[b, :n] != ref).reshape(n, -1), axis=1))[0]
        assert bad.size == 0, f"{name}: sequence {b} rows {bad[:8]} differ from the page table"
        assert not got[b, n:].any(), f"{name}: sequence {b} has rows written past its length"


# lens end mid-page and mid-tile; many pages per split and splits per sequence
GQA_CASES = [
    # name, lens, page, d, fmt (None = bf16), plan (max_splits, waves, min_blocks)
    ("bf16_d128_page16", [1, 15, 17, 200, 1000], 16, 128, None, (16, 64, 1)),
    ("bf16_d128_page32", [31, 32, 33, 640, 2049], 32, 128, None, (16, 16, 1)),
    ("bf16_d128_page64", [63, 64, 65, 3000], 64, 128, None, (4, 8, 2)),
    ("bf16_d64_page16", [5, 48, 777], 16, 64, None, (16, 64, 1)),
    # 64-key FP8 tiles: four 16-row pages per tile
    ("fp8_e4m3_page16", [3, 64, 65, 129, 1500], 16, 128, "e4m3", (16, 64, 1)),
    ("fp8_e5m2_page64", [70, 1024, 4097], 64, 128, "e5m2", (16, 16, 2)),
    ("fp8_e4m3_page32", [1, 95, 96, 2500], 32, 128, "e4m3", (16, 32, 1)),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_gather_gqa_decode(case):
    name, lens, page, d, fmt, (ms, waves, mb) = case
    log("case gather", name)
    hkv = 2
    if fmt is None:
        w = inputs.paged(8100 + len(name), lens, hq=hkv, hkv=hkv, d=d, page=page)
    else:
        w = inputs.paged_fp8(8200 + len(name), lens, fmt, hq=hkv, hkv=hkv, d=d, page=page,
                             descale=False)
    kc, vc = dev_bits(w.k_cache), dev_bits(w.v_cache)
    bt, ln = dev(w.block_table), dev(w.cache_seqlens)
    plan = B.attn_plan_splits(ln, page, hkv, B.attn_device_info(0), waves, ms, mb)
    kd, vd = B.attn_debug_gather_paged(B.ATTN_GATHER_DECODE, kc, vc, bt, ln, plan, ms,
                                       int(max(lens)), fmt or "e4m3")
    torch.cuda.synchronize()
    splits = int(plan[0].item())
    log(f"[{name}] {splits} splits over {len(lens)} sequences")
    assert splits > len(lens), "the case must split sequences"
    kd, vd = host_bits(kd), host_bits(vd)
    check_rows(name + "_k", kd, lens,
               lambda b: orc.gather_paged(w.k_cache, w.block_table, b, int(lens[b]), page))
    check_rows(name + "_v", vd, lens,
               lambda b: orc.gather_paged(w.v_cache, w.block_table, b, int(lens[b]), page))


MLA_CASES = [
    # name, lens, page, hkv, plan
    ("mla_page16_hkv1", [1, 17, 31, 33, 700], 16, 1, (16, 64, 1)),
    ("mla_page64_hkv2", [64, 65, 2049], 64, 2, (8, 8, 2)),
    ("mla_page32_hkv1", [100, 1000], 32, 1, (16, 32, 1)),
]


@pytest.mark.parametrize("case", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_gather_mla_decode(case):
    name, lens, page, hkv, (ms, waves, mb) = case
    log("case gather", name)
    w = inputs.paged(8300 + len(name), lens, hq=hkv, hkv=hkv, d=576, dv=512, page=page,
                     shared_kv=True)
    kc, bt, ln = dev(w.k_cache), dev(w.block_table), dev(w.cache_seqlens)
    plan = B.attn_plan_splits(ln, page, hkv, B.attn_device_info(0), waves, ms, mb)
    kd, _ = B.attn_debug_gather_paged(B.ATTN_GATHER_MLA, kc, None, bt, ln, plan, ms,
                                      int(max(lens)))
    torch.cuda.synchronize()
    log(f"[{name}] {int(plan[0].item())} splits")
    check_rows(name, host_bits(kd), lens,
               lambda b: orc.gather_paged(w.k_cache, w.block_table, b, int(lens[b]), page))


KVC_CASES = [
    # name, current rows, cache rows, page, fmt
    ("kvc_bf16_page16", [1, 40, 200], [0, 17, 300], 16, None),
    ("kvc_bf16_page64", [33, 5], [64, 1000], 64, None),
    ("kvc_fp8_page32", [7, 100, 1], [95, 31, 0], 32, "e4m3"),
    ("kvc_fp8_e5m2_page16", [64, 3], [48, 129], 16, "e5m2"),
]


@pytest.mark.parametrize("case", KVC_CASES, ids=[c[0] for c in KVC_CASES])
def test_gather_kvcache_prefill(case):
    name, lens_new, lens_cache, page, fmt = case
    log("case gather", name)
    hkv = 2
    if fmt is None:
        w = inputs.varlen_kvcache(8400 + len(name), lens_new, lens_new, lens_cache, hq=hkv,
                                  hkv=hkv, d=128, page=page)
    else:
        w = inputs.varlen_kvcache_fp8(8500 + len(name), lens_new, lens_new, lens_cache, fmt,
                                      hq=hkv, hkv=hkv, d=128, page=page, descale=False)
    lk = [int(a) + int(c) for a, c in zip(lens_new, lens_cache)]
    kd, vd = B.attn_debug_gather_kvcache(
        dev_bits(w.k), dev_bits(w.v), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k),
        dev_bits(w.k_cache), dev_bits(w.v_cache), dev(w.block_table), dev(w.cache_seqlens),
        max(lk), fmt or "e4m3")
    torch.cuda.synchronize()

    def keys(cache, cur):
        def f(b):
            lc = int(w.cache_seqlens[b])
            c0, c1 = int(w.cu_seqlens_k[b]), int(w.cu_seqlens_k[b + 1])
            return np.concatenate([orc.gather_paged(cache, w.block_table, b, lc, page),
                                   cur[c0:c1]])
        return f

    check_rows(name + "_k", host_bits(kd), lk, keys(w.k_cache, w.k))
    check_rows(name + "_v", host_bits(vd), lk, keys(w.v_cache, w.v))


def expanded_rows(idx_row, lk, t, sq, mode, s, rows_of, row0):
    """Reference staging of one token's key list: position i*s + e holds the
    row of key idx*s + e when that key is selected (index >= 0, key < lk, and
    in mode 3 key <= t + lk - sq), else row0 (the masked filler row)."""
    out = []
    limit = min(lk - 1, t + lk - sq) if mode == 3 else lk - 1
    for i in idx_row:
        for e in range(s):
            key = int(i) * s + e
            ok = int(i) >= 0 and key <= limit
            out.append(rows_of(key) if ok else row0)
    return np.stack(out)


def test_gather_sparse_dense():
    s = inputs.sparse_mla(8600, batch=2, sq=5, sk=300, hq=16, topk=64, sparse_mode=3)
    rng = np.random.default_rng(3)
    # plant skipped entries: -1, out of range, and past the causal limit
    s.indices[0, 1, 0, :6] = [-1, 300, 299, -7, 296, 0]
    s.indices[1, 4, 0, 10:14] = [299, 298, 1000, -1]
    s.indices[1, 0, 0, :] = rng.integers(-3, 310, size=64)
    log("case gather sparse_dense")
    got = host_bits(B.attn_debug_gather_sparse(dev(s.kv), dev(s.indices), 3))
    torch.cuda.synchronize()
    b_, sq, _, topk = s.indices.shape
    nsel = 0
    for b in range(b_):
        for t in range(sq):
            ref = expanded_rows(s.indices[b, t, 0], 300, t, sq, 3, 1,
                                lambda j: s.kv[b, j, 0], s.kv[b, 0, 0])
            assert np.array_equal(got[b, t], ref), f"sparse dense token ({b}, {t})"
            keys = orc.sparse_key_set(s.indices[b, t, 0], sq, 300, t, 3)
            nsel += len(keys)
    assert nsel > 0


SPARSE_PAGED_CASES = [
    # name, lens, sq, topk, block size, page, mode
    ("block1_page16", [100, 37], 4, 48, 1, 16, 3),
    ("block4_page32", [200, 64], 3, 20, 4, 32, 3),
    ("block64_page64", [1000, 130], 2, 8, 64, 64, 0),
]


@pytest.mark.parametrize("case", SPARSE_PAGED_CASES, ids=[c[0] for c in SPARSE_PAGED_CASES])
def test_gather_sparse_paged(case):
    name, lens, sq, topk, bs, page, mode = case
    log("case gather sparse", name)
    w = inputs.sparse_paged(8700 + len(name), lens, sq, topk, bs, page, hq=16, sparse_mode=mode,
                            spare_pages=2)
    # an index whose block runs past the sequence end, and a padding entry
    w.indices[0, 0, 0, :2] = [(int(lens[0]) - 1) // bs, -1]
    got = host_bits(B.attn_debug_gather_sparse(dev(w.kv_cache), dev(w.indices), mode,
                                               dev(w.block_table), dev(w.seqlens_kv), bs))
    torch.cuda.synchronize()
    for b, lk in enumerate(lens):
        rows = orc.gather_paged(w.kv_cache, w.block_table, b, int(lk), page)[:, 0]
        for t in range(sq):
            ref = expanded_rows(w.indices[b, t, 0], int(lk), t, sq, mode, bs,
                                lambda j: rows[j], w.kv_cache[0, 0, 0])
            assert np.array_equal(got[b, t], ref), f"{name}: token ({b}, {t})"
