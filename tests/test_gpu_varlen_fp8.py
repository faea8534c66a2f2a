"""GPU parity of attn_fwd_varlen_fp8 (packed varlen attention on FP8 Q/K/V
with per-(sequence, KV head) descales) against the float64 oracle on the
decoded codes, through the C ABI.

Tolerance: Q.K^T of the codes is exact in products and summed in float32 and
the rest is the bfloat16 path's arithmetic (P and O rounded to bfloat16), so
the bfloat16 bars apply with O scaled by its V descale (up to 4 here):
max-abs 2e-2 * v_descale on O, 1e-3 on LSE."""
import numpy as np
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import fp8 as ofp8
from tests.gpu_util import TOL_O_BF16, compare, dev, log

pytestmark = pytest.mark.gpu


def run(w, q=None, k=None, v=None, max_q=None):
    lq = np.diff(w.cu_seqlens_q)
    lk = np.diff(w.cu_seqlens_k)
    ds = [None if x is None else dev(x) for x in (w.q_descale, w.k_descale, w.v_descale)]
    return B.attn_fwd_varlen_fp8(
        dev(w.q if q is None else q), dev(w.k if k is None else k), dev(w.v if v is None else v),
        dev(w.cu_seqlens_q), dev(w.cu_seqlens_k), max_q or max(1, int(lq.max())),
        int(lk.max()), w.scale, w.fmt, *ds, causal=w.causal, window=w.window,
        sinks=None if w.sinks is None else dev(w.sinks))


def oracle(w, seqs=None, q=None, k=None, v=None):
    return ofp8.attention_varlen_fp8(w.q if q is None else q, w.k if k is None else k,
                                     w.v if v is None else v, w.fmt, w.q_descale, w.k_descale,
                                     w.v_descale, w.cu_seqlens_q, w.cu_seqlens_k, w.scale,
                                     w.causal, w.window, w.sinks, seqs)


def tol(w):
    return TOL_O_BF16 * (1.0 if w.v_descale is None else float(w.v_descale.max()))


CASES = [
    # name, fmt, lens_q, lens_k, hq, hkv, causal, window, descale, sinks
    ("e4m3_ragged_causal", "e4m3", [1, 17, 130, 300], None, 8, 2, True, (-1, -1), True, False),
    ("e5m2_ragged_causal", "e5m2", [1, 17, 130, 300], None, 8, 2, True, (-1, -1), True, False),
    ("e4m3_noncausal", "e4m3", [5, 64, 129, 257], None, 4, 4, False, (-1, -1), True, False),
    ("e4m3_no_descale_gqa8", "e4m3", [200, 3, 128], None, 8, 1, True, (-1, -1), False, False),
    ("e5m2_bottom_right", "e5m2", [7, 100, 33], [50, 300, 33], 4, 2, True, (-1, -1), True,
     False),
    ("e4m3_q_gt_k_empty_rows", "e4m3", [90, 10], [40, 10], 4, 2, True, (-1, -1), True, False),
    ("e4m3_window_left", "e4m3", [300, 77], None, 4, 2, True, (40, -1), True, False),
    ("e5m2_window_both", "e5m2", [260], None, 4, 4, False, (31, 9), True, False),
    ("e4m3_sinks", "e4m3", [150, 3], None, 8, 2, True, (-1, -1), True, True),
    ("e4m3_empty_sequence", "e4m3", [30, 0, 70], None, 4, 2, True, (-1, -1), True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_fp8(case):
    name, fmt, lq, lk, hq, hkv, causal, window, descale, sinks = case
    log("case varlen_fp8", name)
    w = inputs.varlen_fp8(9000 + len(name), lq, lk, fmt=fmt, hq=hq, hkv=hkv, causal=causal,
                          window=window, descale=descale, with_sinks=sinks)
    o, lse = run(w)
    torch.cuda.synchronize()
    ro, rl = oracle(w)
    compare(name, o, lse, ro, rl, tol(w))


def test_varlen_fp8_extreme_codes():
    """Codes drawn uniformly over every finite code of each format (largest
    magnitudes and subnormals included), descales 1 / max code, so that every
    exponent and the subnormals reach the scores and the output."""
    for fmt in ("e4m3", "e5m2"):
        w = inputs.varlen_fp8(9100, [97, 200], fmt=fmt, hq=4, hkv=2, causal=True)
        rng = np.random.default_rng(9101)
        finite = np.flatnonzero(np.isfinite(ofp8.decode(np.arange(256, dtype=np.uint8), fmt)))
        pick = lambda shape: finite[rng.integers(0, len(finite), size=shape)].astype(np.uint8)
        w.q, w.k, w.v = pick(w.q.shape), pick(w.k.shape), pick(w.v.shape)
        top = float(np.abs(ofp8.decode(finite.astype(np.uint8), fmt)).max())
        for name in ("q_descale", "k_descale", "v_descale"):
            setattr(w, name, np.full_like(getattr(w, name), 1.0 / top))
        log("case varlen_fp8_extreme", fmt)
        o, lse = run(w)
        torch.cuda.synchronize()
        ro, rl = oracle(w)
        compare(f"varlen_fp8_extreme_{fmt}", o, lse, ro, rl, TOL_O_BF16)


def test_varlen_fp8_matches_bf16_path():
    """With unit descales the FP8 path equals attn_fwd_varlen on the codes
    widened to bfloat16 (exact) up to the summation order of Q.K^T: both
    round P and O to bfloat16, so the outputs agree far inside the oracle
    bar."""
    w = inputs.varlen_fp8(9200, [333, 64, 1000], fmt="e4m3", hq=8, hkv=2, causal=True,
                          descale=False)
    log("case varlen_fp8_matches_bf16")
    o8, l8 = run(w)
    wide = lambda x: torch.from_numpy(x).view(torch.float8_e4m3fn).to(torch.bfloat16).cuda()
    lq = np.diff(w.cu_seqlens_q)
    ob, lb = B.attn_fwd_varlen(wide(w.q), wide(w.k), wide(w.v), dev(w.cu_seqlens_q),
                               dev(w.cu_seqlens_k), int(lq.max()), int(lq.max()), w.scale, True)
    torch.cuda.synchronize()
    d_o = float((o8.float() - ob.float()).abs().max())
    d_l = float((l8 - lb).abs().max())
    log(f"fp8 vs bf16 path: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= 1e-2 and d_l <= 1e-4


NAN_E4M3 = np.uint8(0x7F)


def test_varlen_fp8_poisoned_neighbours():
    """NaN codes in the other KV head's columns and in key rows of the other
    sequences: a kernel that reads outside its (sequence, KV head) slice
    produces NaN."""
    w = inputs.varlen_fp8(9300, [70, 150], fmt="e4m3", hq=4, hkv=2, causal=True)
    log("case varlen_fp8_poisoned")
    k, v = w.k.copy(), w.v.copy()
    # head 1 of sequence 0 and head 0 of sequence 1 are poisoned; queries of
    # the other head of each sequence must stay clean
    c = w.cu_seqlens_k
    k[c[0]:c[1], 1] = NAN_E4M3
    v[c[0]:c[1], 1] = NAN_E4M3
    k[c[1]:c[2], 0] = NAN_E4M3
    v[c[1]:c[2], 0] = NAN_E4M3
    o, lse = run(w, k=k, v=v)
    torch.cuda.synchronize()
    ro, rl = oracle(w, k=k, v=v)
    cq = w.cu_seqlens_q
    sel = np.zeros(ro.shape, bool)
    sel[cq[0]:cq[1], 0:2] = True        # sequence 0, query heads of KV head 0
    sel[cq[1]:cq[2], 2:4] = True        # sequence 1, query heads of KV head 1
    lsel = np.transpose(sel[:, :, 0])
    rl = np.where(lsel, rl, np.nan)
    compare("varlen_fp8_poisoned", o, lse, ro, rl, tol(w), mask=sel)


def test_varlen_fp8_prefill_workload():
    """The FP8 varlen prefill workload (seed 1009: 8 sequences U[512, 4096],
    Hq=32, Hkv=8, D=128, causal, e4m3 with descales) in the launch
    configuration bench.py times; sequences 1 and 5 compared element by
    element."""
    w = inputs.varlen_prefill_fp8()
    log("case varlen_fp8_prefill_workload")
    o, lse = run(w)
    torch.cuda.synchronize()
    ro, rl = oracle(w, seqs=[1, 5])
    compare("varlen_fp8_prefill_workload", o, lse, ro, rl, tol(w))
