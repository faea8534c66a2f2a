"""Hypothesis-drawn small shapes, GPU against the float64 oracle through the C
ABI: varlen prefill, paged decode (bf16 and FP8) with split plans from one
split per sequence to many single-page splits.

Each draw covers the axes the fixed cases take one at a time: head dim 64 or
128, GQA ratios 1-8, lengths that are not multiples of the page (and zero),
several query tokens per sequence with bottom-right causal masks that leave
rows or whole splits empty, windows, and sinks of either sign and of large
magnitude. Draws are derandomized (the same examples every run) and each is
logged before its GPU call."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from oracle import fp8 as ofp8
from tests.gpu_util import TOL_O_BF16, compare, dev, log

pytestmark = pytest.mark.gpu

FUZZ = settings(max_examples=30, deadline=None, derandomize=True, database=None,
                suppress_health_check=list(HealthCheck))


@st.composite
def heads(draw):
    hkv = draw(st.sampled_from([1, 2, 4]))
    grp = draw(st.integers(1, 8))
    return hkv * grp, hkv


@st.composite
def sinks_scale(draw):
    """None (no sinks) or the factor applied to N(0,1) sinks: about 1, or 30
    so that the sink term dominates a row or vanishes beside it."""
    return draw(st.sampled_from([None, 1.0, 30.0]))


@st.composite
def varlen_case(draw):
    d = draw(st.sampled_from([64, 128]))
    hq, hkv = draw(heads())
    n = draw(st.integers(1, 4))
    lq = draw(st.lists(st.integers(0, 300), min_size=n, max_size=n))
    lq[0] = max(lq[0], 1)
    lk = list(lq) if draw(st.booleans()) else draw(st.lists(st.integers(0, 400), min_size=n,
                                                             max_size=n))
    lk[0] = max(lk[0], 1)
    causal = draw(st.booleans())
    wl = draw(st.sampled_from([-1, -1, 0, 17, 64]))
    wr = draw(st.sampled_from([-1, -1, 0, 5, 40])) if not causal else -1
    return dict(d=d, hq=hq, hkv=hkv, lq=lq, lk=list(lk), causal=causal, window=(wl, wr),
                sinks=draw(sinks_scale()), seed=draw(st.integers(0, 2**31 - 1)))


@given(varlen_case())
@FUZZ
def test_fuzz_varlen(c):
    log("case fuzz_varlen", c)
    w = inputs.varlen(c["seed"], c["lq"], c["lk"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                      causal=c["causal"], window=c["window"], with_sinks=c["sinks"] is not None)
    if c["sinks"] is not None:
        w.sinks = (w.sinks * c["sinks"]).astype(np.float32)
    o, lse = B.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_seqlens_q),
                               dev(w.cu_seqlens_k), max(c["lq"]), max(c["lk"]), w.scale,
                               w.causal, w.window, None if w.sinks is None else dev(w.sinks))
    torch.cuda.synchronize()
    ro, rl = orc.attention_varlen(w.f32("q"), w.f32("k"), w.f32("v"), w.cu_seqlens_q,
                                  w.cu_seqlens_k, w.scale, w.causal, w.window, w.sinks)
    compare("fuzz_varlen", o, lse, ro, rl, TOL_O_BF16)


@st.composite
def plan_params(draw):
    """(max_splits, waves, min_blocks): from one split per sequence to one
    page per split."""
    return (draw(st.sampled_from([1, 3, 16])), draw(st.sampled_from([1, 8, 64])),
            draw(st.sampled_from([1, 2])))


@st.composite
def decode_case(draw):
    hq, hkv = draw(heads())
    page = draw(st.sampled_from([16, 32, 64]))
    n = draw(st.integers(1, 4))
    lens = draw(st.lists(st.integers(0, 700), min_size=n, max_size=n))
    lens[0] = max(lens[0], 1)
    return dict(d=draw(st.sampled_from([64, 128])), hq=hq, hkv=hkv, page=page, lens=lens,
                sq=draw(st.integers(1, 3)), causal=draw(st.booleans()),
                sinks=draw(sinks_scale()), plan=draw(plan_params()),
                seed=draw(st.integers(0, 2**31 - 1)))


@given(decode_case())
@FUZZ
def test_fuzz_paged_decode(c):
    log("case fuzz_paged_decode", c)
    w = inputs.paged(c["seed"], c["lens"], sq=c["sq"], hq=c["hq"], hkv=c["hkv"], d=c["d"],
                     page=c["page"], causal=c["causal"], with_sinks=c["sinks"] is not None)
    if c["sinks"] is not None:
        w.sinks = (w.sinks * c["sinks"]).astype(np.float32)
    o, lse, _ = B.paged_decode(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                               dev(w.cache_seqlens), w.scale, w.causal,
                               None if w.sinks is None else dev(w.sinks), *c["plan"])
    torch.cuda.synchronize()
    q, kc, vc = (inputs.bits_to_f32(x) for x in (w.q, w.k_cache, w.v_cache))
    ro, rl = orc.attention_paged(q, kc, vc, w.block_table, w.cache_seqlens, w.page_size, w.scale,
                                 w.causal, w.sinks)
    compare("fuzz_paged_decode", o, lse, ro, rl, TOL_O_BF16)


@st.composite
def fp8_case(draw):
    hq, hkv = draw(heads())
    n = draw(st.integers(1, 4))
    lens = draw(st.lists(st.integers(0, 700), min_size=n, max_size=n))
    lens[0] = max(lens[0], 1)
    return dict(fmt=draw(st.sampled_from(["e4m3", "e5m2"])), hq=hq, hkv=hkv,
                page=draw(st.sampled_from([16, 32, 64])),
                lens=lens,
                sq=draw(st.integers(1, 3)), causal=draw(st.booleans()),
                descale=draw(st.booleans()), plan=draw(plan_params()),
                seed=draw(st.integers(0, 2**31 - 1)))


@given(fp8_case())
@FUZZ
def test_fuzz_paged_decode_fp8(c):
    log("case fuzz_paged_decode_fp8", c)
    w = inputs.paged_fp8(c["seed"], c["lens"], c["fmt"], sq=c["sq"], hq=c["hq"], hkv=c["hkv"],
                         page=c["page"], causal=c["causal"], descale=c["descale"])
    ds = [None if x is None else dev(x) for x in (w.q_descale, w.k_descale, w.v_descale)]
    o, lse, _ = B.paged_decode_fp8(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                   dev(w.cache_seqlens), w.scale, w.fmt, *ds, causal=w.causal,
                                   max_splits=c["plan"][0], waves=c["plan"][1],
                                   min_blocks=c["plan"][2])
    torch.cuda.synchronize()
    ro, rl = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, w.fmt, w.q_descale,
                                      w.k_descale, w.v_descale, w.block_table, w.cache_seqlens,
                                      w.page_size, w.scale, w.causal)
    tol = TOL_O_BF16 * (1.0 if w.v_descale is None else float(w.v_descale.max()))
    compare("fuzz_paged_decode_fp8", o, lse, ro, rl, tol)
