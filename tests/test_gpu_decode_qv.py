"""GPU parity of the paged decode with a second query qv scored against the
value rows (attn_decode_paged_qv, then attn_combine), bf16 and FP8, with and
without the QK path (only_qv), against the float64 oracle through the C ABI.

Tolerance: the qv . v scores come from the same bf16 MFMAs (on exactly
widened codes for FP8) summed in fp32, so the decode bars apply: max-abs
2e-2 on O (times v_descale for FP8), 1e-3 on LSE."""
import numpy as np
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from oracle import fp8 as ofp8
from tests.gpu_util import TOL_O_BF16, compare, dev, log

pytestmark = pytest.mark.gpu


def run(w, only_qv=False, fmt=None, max_splits=16, waves=4, min_blocks=4, drop_qk=False):
    ds = [None] * 3 if fmt is None else \
        [None if x is None else dev(x) for x in (w.q_descale, w.k_descale, w.v_descale)]
    q = None if drop_qk else dev(w.q)
    kc = None if drop_qk else dev(w.k_cache)
    return B.paged_decode_qv(q, dev(w.qv), kc, dev(w.v_cache), dev(w.block_table),
                             dev(w.cache_seqlens), w.scale, fmt, *ds, causal=w.causal,
                             only_qv=only_qv, max_splits=max_splits, waves=waves,
                             min_blocks=min_blocks)


def oracle(w, only_qv=False, fmt=None, batches=None):
    if fmt is None:
        f = inputs.bits_to_f32
        return orc.attention_paged(None if only_qv else f(w.q),
                                   None if only_qv else f(w.k_cache), f(w.v_cache),
                                   w.block_table, w.cache_seqlens, w.page_size, w.scale,
                                   w.causal, batches=batches, qv=f(w.qv), only_qv=only_qv)
    return ofp8.attention_paged_fp8(None if only_qv else w.q, None if only_qv else w.k_cache,
                                    w.v_cache, fmt, w.q_descale, w.k_descale, w.v_descale,
                                    w.block_table, w.cache_seqlens, w.page_size, w.scale,
                                    w.causal, batches=batches, qv8=w.qv, only_qv=only_qv)


CASES = [
    # name, fmt, lens, sq, hq, hkv, page, causal, only_qv, max_splits, waves, min_blocks
    ("bf16_ragged", None, [1, 63, 64, 65, 700, 2049], 1, 32, 8, 64, False, False, 16, 4, 4),
    ("bf16_only_qv", None, [1, 63, 64, 65, 700, 2049], 1, 32, 8, 64, False, True, 16, 4, 4),
    ("bf16_causal_sq3_page16", None, [90, 400, 3], 3, 16, 4, 16, True, False, 8, 16, 1),
    ("bf16_only_qv_many_splits", None, [5000, 130, 4097], 1, 8, 2, 16, False, True, 16, 64, 1),
    ("e4m3_ragged", "e4m3", [1, 63, 64, 65, 700, 2049], 1, 32, 8, 64, False, False, 16, 4, 4),
    ("e5m2_causal_sq3", "e5m2", [90, 400, 3], 3, 16, 4, 16, True, False, 8, 16, 1),
    ("e4m3_only_qv", "e4m3", [300, 1200, 17], 1, 8, 2, 64, False, True, 16, 8, 2),
    ("e5m2_only_qv_gqa16", "e5m2", [333, 1000], 2, 16, 1, 64, True, True, 16, 8, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_qv(case):
    name, fmt, lens, sq, hq, hkv, page, causal, only, ms, waves, mb = case
    log("case decode_qv", name)
    if fmt is None:
        w = inputs.paged(9500 + len(name), lens, sq=sq, hq=hq, hkv=hkv, page=page,
                         causal=causal, with_qv=True)
        tol = TOL_O_BF16
    else:
        w = inputs.paged_fp8(9500 + len(name), lens, fmt, sq=sq, hq=hq, hkv=hkv, page=page,
                             causal=causal, with_qv=True)
        tol = TOL_O_BF16 * float(w.v_descale.max())
    o, lse, _ = run(w, only, fmt, ms, waves, mb, drop_qk=only)
    torch.cuda.synchronize()
    ro, rl = oracle(w, only, fmt)
    compare(name, o, lse, ro, rl, tol)


def test_decode_qv_zero_is_plain_decode():
    """qv = 0 adds nothing: the output equals attn_decode_paged's on the same
    plan up to the last bits (the same MFMA chain continued with zeros)."""
    w = inputs.paged(9600, [700, 2049, 64], sq=1, hq=32, hkv=8, page=64, with_qv=True)
    w.qv = np.zeros_like(w.qv)
    log("case decode_qv_zero")
    o1, l1, _ = run(w)
    o2, l2, _ = B.paged_decode(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                               dev(w.cache_seqlens), w.scale, max_splits=16, waves=4,
                               min_blocks=4)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_qv_workload():
    """The paged-decode workload (seed 1003: 64 sequences U[1024, 32768],
    page 64, Hq=32, Hkv=8, D=128, bf16) with a qv of its own (seed 1010), in
    the launch configuration bench.py times; sequences 0, 17 and 63 compared
    element by element, with and without the QK path (plans (16, 8, 2) and
    (16, 16, 2))."""
    w = inputs.paged_decode()
    w.qv = inputs.paged_decode_qv(w)
    for only in (False, True):
        log("case decode_qv_workload only_qv", only)
        o, lse, _ = run(w, only, None, 16, 16 if only else 8, 2, drop_qk=only)
        torch.cuda.synchronize()
        ro, rl = oracle(w, only, None, batches=[0, 17, 63])
        compare(f"decode_qv_workload_only{int(only)}", o, lse, ro, rl, TOL_O_BF16)
