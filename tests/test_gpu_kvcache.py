"""GPU parity of attn_fwd_varlen_kvcache (queries over a paged cache of earlier
tokens followed by the current K/V rows) against the float64 oracle, through
the C ABI."""
import numpy as np
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from tests.gpu_util import TOL_O_BF16, compare, dev, log

pytestmark = pytest.mark.gpu

NAN_BF16 = np.uint16(0x7FC0)


def run_kvcache(w, k_cache=None, v_cache=None, block_table=None):
    lq = np.diff(w.cu_seqlens_q)
    return B.attn_fwd_varlen_kvcache(
        dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k),
        dev(w.k_cache if k_cache is None else k_cache),
        dev(w.v_cache if v_cache is None else v_cache),
        dev(w.block_table if block_table is None else block_table), dev(w.cache_seqlens),
        max(1, int(lq.max())), w.scale, w.causal, w.window,
        None if w.sinks is None else dev(w.sinks))


def oracle_kvcache(w, seqs=None):
    return orc.attention_varlen_kvcache(
        w.f32("q"), w.f32("k"), w.f32("v"), w.cu_seqlens_q, w.cu_seqlens_k,
        inputs.bits_to_f32(w.k_cache), inputs.bits_to_f32(w.v_cache), w.block_table,
        w.cache_seqlens, w.page_size, w.scale, w.causal, w.window, w.sinks, seqs)


KV_CASES = [
    # name, lens_q, lens_new, lens_cache, hq, hkv, d, page, causal, window, sinks
    # cache ends inside a 16-row block and inside a 32-key tile; an empty cache
    ("straddle_d128", [37, 200, 64], [37, 200, 64], [100, 333, 0], 8, 2, 128, 64, True,
     (-1, -1), False),
    # tiles wholly in the cache, then wholly current
    ("aligned_d128", [64, 5], [64, 5], [512, 1024], 4, 2, 128, 64, True, (-1, -1), False),
    # 64-key tiles over four 16-row pages
    ("page16_d64_gqa8", [50, 130, 3], [50, 130, 3], [77, 250, 16], 8, 1, 64, 16, True,
     (-1, -1), False),
    ("page32_d64_window", [90, 40], [90, 40], [300, 45], 4, 2, 64, 32, True, (100, -1), False),
    ("page16_d128_noncausal_window", [70, 33], [70, 33], [190, 64], 4, 4, 128, 16, False,
     (50, 20), False),
    ("empty_cache_d128", [17, 130], [17, 130], [0, 0], 4, 2, 128, 64, True, (-1, -1), False),
    # queries whose keys are all cached (no current rows), decode-like
    ("cache_only_keys", [4, 1], [0, 0], [300, 65], 8, 2, 128, 32, False, (-1, -1), False),
    ("cache_only_keys_causal_d64", [40, 3], [0, 0], [129, 200], 4, 2, 64, 16, True, (-1, -1),
     False),
    ("sinks_causal_d128", [150, 3], [150, 3], [81, 500], 8, 2, 128, 64, True, (-1, -1), True),
    ("empty_sequence", [30, 0, 70], [30, 0, 70], [20, 50, 0], 4, 2, 128, 16, True, (-1, -1),
     False),
    # more queries than keys of the sequence: the first rows see nothing
    ("q_gt_k_empty_rows", [90, 10], [40, 10], [10, 0], 4, 2, 128, 16, True, (-1, -1), False),
]


@pytest.mark.parametrize("case", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_varlen_kvcache(case):
    name, lq, ln, lc, hq, hkv, d, page, causal, window, sinks = case
    log("case", name)
    w = inputs.varlen_kvcache(5000 + len(name), lq, ln, lc, hq=hq, hkv=hkv, d=d, page=page,
                              causal=causal, window=window, with_sinks=sinks, spare_pages=2)
    o, lse = run_kvcache(w)
    torch.cuda.synchronize()
    ro, rl = oracle_kvcache(w)
    compare(name, o, lse, ro, rl, TOL_O_BF16)


def test_kvcache_poisoned_pool():
    """NaN in the pool pages no sequence references and in every cache row
    past a sequence's cache length inside its last page: a read of any of
    them would turn the output NaN."""
    lq, lc, page, extra = [48, 100, 7], [70, 129, 16], 32, 3
    w = inputs.varlen_kvcache(5101, lq, lq, lc, hq=8, hkv=2, d=128, page=page, causal=True)
    log("case kvcache_poisoned_pool")

    def poison(c):
        c = np.concatenate([np.full((extra,) + c.shape[1:], NAN_BF16, np.uint16), c])
        for b, n in enumerate(lc):
            if n % page:
                c[int(w.block_table[b, (n - 1) // page]) + extra, n % page:] = NAN_BF16
        return c

    bt = np.where(w.block_table >= 0, w.block_table + extra, -1).astype(np.int32)
    o, lse = run_kvcache(w, poison(w.k_cache), poison(w.v_cache), bt)
    torch.cuda.synchronize()
    ro, rl = oracle_kvcache(w)
    compare("kvcache_poisoned_pool", o, lse, ro, rl, TOL_O_BF16)


def test_kvcache_empty_cache_matches_varlen():
    """With every cache empty the keys are the current rows alone: the result
    equals attn_fwd_varlen's on the same inputs, bit for bit (the same tiles in
    the same order)."""
    lq = [33, 257, 64]
    for d in (64, 128):
        w = inputs.varlen_kvcache(5200 + d, lq, lq, [0, 0, 0], hq=8, hkv=2, d=d, page=16)
        log("case kvcache_empty_cache_matches_varlen d", d)
        o1, l1 = run_kvcache(w)
        o2, l2 = B.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q),
                                   dev(w.cu_seqlens_k), max(lq), max(lq), w.scale, True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_kvcache_chunked_prefill_large():
    """A chunk of 1024 new tokens per sequence after caches of 4096 and 7001
    tokens, Hq=32, Hkv=8, D=128, page 64, causal: every output element."""
    w = inputs.varlen_kvcache(5300, [1024, 1024], [1024, 1024], [4096, 7001], hq=32, hkv=8,
                              d=128, page=64, causal=True)
    log("case kvcache_chunked_prefill_large")
    o, lse = run_kvcache(w)
    torch.cuda.synchronize()
    ro, rl = oracle_kvcache(w)
    compare("kvcache_chunked_prefill_large", o, lse, ro, rl, TOL_O_BF16)


def test_kvcache_deterministic():
    w = inputs.varlen_kvcache(5400, [100, 300], [100, 300], [77, 1000], hq=8, hkv=2, d=128,
                              page=16)
    o1, l1 = run_kvcache(w)
    o2, l2 = run_kvcache(w)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_kvcache_chunked_workload():
    """The benchmarked chunked-prefill workload (seed 1006: 8 chunks of 1024
    tokens after caches of U[1024, 8192] tokens, page 64, Hq=32, Hkv=8,
    D=128, causal), in the launch configuration bench.py times; sequences 0
    and 4 compared element by element."""
    w = inputs.chunked_prefill()
    log("case kvcache_chunked_workload caches", w.cache_seqlens.tolist())
    o, lse = run_kvcache(w)
    torch.cuda.synchronize()
    ro, rl = oracle_kvcache(w, seqs=[0, 4])
    compare("kvcache_chunked_workload", o, lse, ro, rl, TOL_O_BF16)


MASK_CASES = [
    # name, lens_q, lens_cache, hq, hkv, d, page, causal, mask_heads, neg_inf_fraction
    ("mask_heads_d128", [37, 200, 64], [100, 333, 0], 8, 2, 128, 64, True, 8, 0.0),
    ("mask_shared_neginf_d128", [150, 3], [81, 500], 8, 2, 128, 16, True, 1, 0.2),
    ("mask_d64_noncausal", [50, 130], [77, 250], 8, 1, 64, 16, False, 8, 0.1),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_kvcache_additive_mask(case):
    """Additive bf16 mask on the scaled scores, N(0, 2^2) values with a share
    of -inf entries, over keys of the cache and the current rows."""
    name, lq, lc, hq, hkv, d, page, causal, mh, frac = case
    log("case", name)
    w = inputs.varlen_kvcache(5500 + len(name), lq, lq, lc, hq=hq, hkv=hkv, d=d, page=page,
                              causal=causal)
    tq = int(sum(lq))
    ld = ((max(a + b for a, b in zip(lq, lc)) + 63) // 64) * 64 + 64
    rng = np.random.default_rng(5600 + len(name))
    m = (2.0 * rng.standard_normal((mh, tq, ld))).astype(np.float32)
    m[rng.random(m.shape) < frac] = -np.inf
    mbits = inputs.bf16_bits(m)
    mvals = inputs.bits_to_f32(mbits).astype(np.float64)
    o, lse = B.attn_fwd_varlen_kvcache(
        dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k), dev(w.k_cache),
        dev(w.v_cache), dev(w.block_table), dev(w.cache_seqlens), max(lq), w.scale, causal,
        mask=dev(mbits))
    torch.cuda.synchronize()
    ro, rl = orc.attention_varlen_kvcache(
        w.f32("q"), w.f32("k"), w.f32("v"), w.cu_seqlens_q, w.cu_seqlens_k,
        inputs.bits_to_f32(w.k_cache), inputs.bits_to_f32(w.v_cache), w.block_table,
        w.cache_seqlens, w.page_size, w.scale, causal, mask=mvals)
    compare(name, o, lse, ro, rl, TOL_O_BF16)


def test_kvcache_mask_rows_fully_masked():
    """Rows whose mask is -inf on every key are empty (O = 0, LSE = -inf);
    the other rows are unaffected."""
    lq, lc = [40, 70], [30, 100]
    w = inputs.varlen_kvcache(5700, lq, lq, lc, hq=4, hkv=2, d=128, page=16, causal=True)
    tq, ld = 110, 192
    m = np.zeros((1, tq, ld), np.float32)
    m[0, ::7] = -np.inf
    mbits = inputs.bf16_bits(m)
    log("case kvcache_mask_rows_fully_masked")
    o, lse = B.attn_fwd_varlen_kvcache(
        dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k), dev(w.k_cache),
        dev(w.v_cache), dev(w.block_table), dev(w.cache_seqlens), max(lq), w.scale, True,
        mask=dev(mbits))
    torch.cuda.synchronize()
    ro, rl = orc.attention_varlen_kvcache(
        w.f32("q"), w.f32("k"), w.f32("v"), w.cu_seqlens_q, w.cu_seqlens_k,
        inputs.bits_to_f32(w.k_cache), inputs.bits_to_f32(w.v_cache), w.block_table,
        w.cache_seqlens, w.page_size, w.scale, True, mask=inputs.bits_to_f32(mbits).astype(float))
    assert np.isneginf(rl[:, ::7]).all()
    compare("kvcache_mask_rows_fully_masked", o, lse, ro, rl, TOL_O_BF16)


def test_kvcache_chunked_mask_workload():
    """The benchmarked masked chunked-prefill workload (seed 1006 with the
    shared N(0,1) bf16 mask), in the launch configuration bench.py times;
    sequences 0 and 4 compared element by element."""
    w = inputs.chunked_prefill()
    lq = np.diff(w.cu_seqlens_q)
    ld = ((int((lq + w.cache_seqlens).max()) + 63) // 64) * 64
    mbits = inputs.chunked_mask(int(lq.sum()), ld)
    log("case kvcache_chunked_mask_workload")
    o, lse = B.attn_fwd_varlen_kvcache(
        dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k), dev(w.k_cache),
        dev(w.v_cache), dev(w.block_table), dev(w.cache_seqlens), int(lq.max()), w.scale, True,
        mask=dev(mbits))
    torch.cuda.synchronize()
    ro, rl = orc.attention_varlen_kvcache(
        w.f32("q"), w.f32("k"), w.f32("v"), w.cu_seqlens_q, w.cu_seqlens_k,
        inputs.bits_to_f32(w.k_cache), inputs.bits_to_f32(w.v_cache), w.block_table,
        w.cache_seqlens, w.page_size, w.scale, True, seqs=[0, 4], mask=inputs.bits_to_f32(mbits))
    compare("kvcache_chunked_mask_workload", o, lse, ro, rl, TOL_O_BF16)


QV_CASES = [
    # name, lens_q, lens_new, lens_cache, hq, hkv, page, causal, window, sinks, only_qv
    ("qv_straddle", [37, 200, 64], [37, 200, 64], [100, 333, 0], 8, 2, 64, True, (-1, -1),
     False, False),
    ("qv_page16_window", [70, 33], [70, 33], [190, 64], 4, 4, 16, False, (50, 20), False,
     False),
    ("qv_cache_only_keys", [4, 1], [0, 0], [300, 65], 8, 2, 32, False, (-1, -1), False, False),
    ("qv_sinks_aligned", [64, 5], [64, 5], [512, 1024], 4, 2, 64, True, (-1, -1), True, False),
    ("only_qv_straddle", [37, 200, 64], [37, 200, 64], [100, 333, 0], 8, 2, 64, True,
     (-1, -1), False, True),
    ("only_qv_page16_empty_seq", [30, 0, 70], [30, 0, 70], [20, 50, 0], 4, 2, 16, True,
     (-1, -1), False, True),
]


@pytest.mark.parametrize("case", QV_CASES, ids=[c[0] for c in QV_CASES])
def test_varlen_kvcache_qv(case):
    """attn_fwd_varlen_kvcache_qv: scores q.k + qv.v (or qv.v alone) over the
    cached and current rows, against the float64 oracle."""
    name, lq, ln, lc, hq, hkv, page, causal, window, sinks, only_qv = case
    log("case", name)
    w = inputs.varlen_kvcache(5200 + len(name), lq, ln, lc, hq=hq, hkv=hkv, d=128, page=page,
                              causal=causal, window=window, with_sinks=sinks, spare_pages=2,
                              with_qv=True)
    o, lse = B.attn_fwd_varlen_kvcache_qv(
        None if only_qv else dev(w.q), dev(w.qv), None if only_qv else dev(w.k), dev(w.v),
        dev(w.cu_seqlens_q), dev(w.cu_seqlens_k), None if only_qv else dev(w.k_cache),
        dev(w.v_cache), dev(w.block_table), dev(w.cache_seqlens),
        max(1, int(np.diff(w.cu_seqlens_q).max())), w.scale, w.causal, w.window,
        None if w.sinks is None else dev(w.sinks), only_qv=only_qv)
    torch.cuda.synchronize()
    ro, rl = orc.attention_varlen_kvcache(
        None if only_qv else w.f32("q"), None if only_qv else w.f32("k"), w.f32("v"),
        w.cu_seqlens_q, w.cu_seqlens_k,
        None if only_qv else inputs.bits_to_f32(w.k_cache), inputs.bits_to_f32(w.v_cache),
        w.block_table, w.cache_seqlens, w.page_size, w.scale, w.causal, w.window, w.sinks,
        qv=w.f32("qv"), only_qv=only_qv)
    compare(name, o, lse, ro, rl, TOL_O_BF16)
