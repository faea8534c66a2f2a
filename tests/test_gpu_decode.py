"""GPU parity of the split planner, the paged gather, split-KV decode (GQA
and MLA shapes) and the combine, through the C ABI."""
import numpy as np
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from tests.gpu_util import assert_plan_equal, TOL_O_BF16, compare, dev, host, log

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------- planner
PLAN_CASES = [
    # lens, page, upb, num_cu, waves, max_splits, min_blocks
    ("decode_lens", None, 64, 8, 256, 4, 16, 4),
    ("mla_lens", None, 64, 4, 256, 2, 16, 4),
    ("with_zeros", [0, 1, 64, 65, 0, 40000, 12], 64, 1, 4, 1, 3, 2),
    ("many_seqs", list(range(0, 5000 * 97, 97)), 16, 3, 256, 8, 16, 1),
    # 3560 splits in 475 groups (up to 15 splits of one length per sequence)
    ("many_splits_few_groups",
     [int(x) for x in np.random.default_rng(9).integers(1, 200000, 240)], 16, 1, 256, 64, 16, 1),
    # more than 1024 groups with at most 4096 splits: the bitonic network
    ("bitonic_one_split_each", [3000 + (i % 7) * 16 for i in range(1500)], 16, 1, 256, 2, 4, 64),
    ("bitonic_two_splits_each", [1000 + (i % 5) * 40 for i in range(800)], 16, 1, 256, 4, 2, 40),
    # equal lengths across sequences, lengths that fill their last page exactly
    ("ties_and_full_pages", [4096] * 100 + [4095, 1, 0, 4097, 64, 128], 64, 2, 256, 16, 16, 1),
]


@pytest.mark.parametrize("case", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_plan_bit_exact(case):
    name, lens, page, upb, ncu, waves, ms, mb = case
    if lens is None:
        w = inputs.paged_decode() if name == "decode_lens" else inputs.mla_decode()
        lens = w.cache_seqlens
    lens = np.asarray(lens, dtype=np.int32)
    log("case plan", name, len(lens))
    plan = B.attn_plan_splits(dev(lens), page, upb, ncu, waves, ms, mb)
    ref = orc.plan_splits(lens, page, upb, ncu, waves, ms, mb)
    assert_plan_equal(host(plan), ref, len(lens), ms)


# ---------------------------------------------------------------------- GQA
def run_decode(w, max_splits=16, waves=4, min_blocks=4):
    return B.paged_decode(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                          dev(w.cache_seqlens), w.scale, w.causal,
                          None if w.sinks is None else dev(w.sinks), max_splits=max_splits,
                          waves=waves, min_blocks=min_blocks)


def oracle_decode(w, batches=None):
    q, kc, vc = (inputs.bits_to_f32(x) for x in (w.q, w.k_cache, w.v_cache))
    return orc.attention_paged(q, kc, vc, w.block_table, w.cache_seqlens, w.page_size, w.scale,
                               w.causal, w.sinks, batches=batches)


DECODE_CASES = [
    # name, lens, sq, hq, hkv, page, causal, sinks, max_splits, waves, min_blocks
    ("ragged_pages", [1, 63, 64, 65, 700, 2049], 1, 32, 8, 64, False, False, 16, 4, 4),
    ("many_splits", [5000, 130, 4097], 1, 8, 2, 16, False, False, 16, 64, 1),
    ("one_split", [300, 1200], 1, 8, 8, 64, False, False, 1, 4, 4),
    ("causal_sq3", [90, 400, 3], 3, 16, 4, 16, True, False, 8, 16, 1),
    ("sinks", [1000, 17], 2, 8, 2, 32, False, True, 4, 8, 1),
    ("gqa16_rows32", [333, 1000], 2, 16, 1, 64, True, False, 16, 8, 2),
]

# head dim 64: name, lens, sq, hq, hkv, page, causal, max_splits, waves, min_blocks
DECODE_D64_CASES = [
    ("d64_ragged", [1, 63, 64, 65, 700, 2049], 1, 32, 8, 64, False, 16, 4, 4),
    ("d64_causal_sq3_page16", [90, 400, 3], 3, 16, 4, 16, True, 8, 16, 1),
    ("d64_many_splits", [5000, 130, 4097], 1, 8, 2, 16, False, 16, 64, 1),
]


@pytest.mark.parametrize("case", DECODE_D64_CASES, ids=[c[0] for c in DECODE_D64_CASES])
def test_decode_gqa_d64(case):
    name, lens, sq, hq, hkv, page, causal, ms, waves, mb = case
    log("case decode", name)
    w = inputs.paged(6400 + len(name), lens, sq=sq, hq=hq, hkv=hkv, d=64, page=page,
                     causal=causal)
    o, lse, _ = run_decode(w, ms, waves, mb)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w)
    compare(name, o, lse, ro, rl, TOL_O_BF16)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_gqa(case):
    name, lens, sq, hq, hkv, page, causal, sinks, ms, waves, mb = case
    log("case decode", name)
    w = inputs.paged(5000 + len(name), lens, sq=sq, hq=hq, hkv=hkv, d=128, page=page,
                     causal=causal, with_sinks=sinks)
    o, lse, plan = run_decode(w, ms, waves, mb)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w)
    compare(name, o, lse, ro, rl, TOL_O_BF16)
    ref_plan = orc.plan_splits(w.cache_seqlens, page, hkv * ((sq * hq // hkv + 15) // 16),
                               B.attn_device_info(0), waves, ms, mb)
    assert_plan_equal(host(plan), ref_plan, len(lens), ms)


DECODE_MASK_CASES = [
    # name, lens, sq, hq, hkv, d, page, causal, mask_heads, neg_inf_fraction, plan
    ("mask_heads_d128", [1, 63, 700, 2049], 1, 32, 8, 128, 64, False, 32, 0.0, (16, 4, 4)),
    ("mask_shared_neginf_causal_sq3", [90, 400, 3], 3, 16, 4, 128, 16, True, 1, 0.2, (8, 16, 1)),
    ("mask_d64_gqa8_many_splits", [5000, 130, 17], 2, 16, 2, 64, 32, True, 16, 0.1,
     (16, 64, 1)),
]


@pytest.mark.parametrize("case", DECODE_MASK_CASES, ids=[c[0] for c in DECODE_MASK_CASES])
def test_decode_additive_mask(case):
    """attn_decode_paged_mask through plan, split decode and combine: an
    additive bf16 mask (N(0, 2^2) with a share of -inf entries) per head or
    shared, with ragged lengths, page sizes and plans of many short splits."""
    name, lens, sq, hq, hkv, d, page, causal, mh, frac, (ms, waves, mb) = case
    log("case decode_mask", name)
    w = inputs.paged(5300 + len(name), lens, sq=sq, hq=hq, hkv=hkv, d=d, page=page,
                     causal=causal)
    ld = ((max(lens) + 63) // 64) * 64
    rng = np.random.default_rng(5400 + len(name))
    m = (2.0 * rng.standard_normal((len(lens), mh, sq, ld))).astype(np.float32)
    m[rng.random(m.shape) < frac] = -np.inf
    mbits = inputs.bf16_bits(m)
    o, lse, _ = B.paged_decode(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                               dev(w.cache_seqlens), w.scale, w.causal, None, max_splits=ms,
                               waves=waves, min_blocks=mb, mask=dev(mbits))
    torch.cuda.synchronize()
    q, kc, vc = (inputs.bits_to_f32(x) for x in (w.q, w.k_cache, w.v_cache))
    ro, rl = orc.attention_paged(q, kc, vc, w.block_table, w.cache_seqlens, w.page_size, w.scale,
                                 w.causal, mask=inputs.bits_to_f32(mbits).astype(np.float64))
    compare(name, o, lse, ro, rl, TOL_O_BF16)


NAN_BF16 = np.uint16(0x7FC0)


def poison_pool(w, extra):
    """Copies of the caches with `extra` NaN pages placed in front of the
    pool (no block_table entry names them) and NaN in every row past a
    sequence's length inside its last page. A read of any row outside
    [0, len) that reached the softmax or P.V would make the output NaN."""
    def one(c):
        c = np.concatenate([np.full((extra,) + c.shape[1:], NAN_BF16, np.uint16), c])
        for b, L in enumerate(w.cache_seqlens):
            L = int(L)
            if L % w.page_size:
                last = int(w.block_table[b, (L - 1) // w.page_size]) + extra
                c[last, L % w.page_size:] = NAN_BF16
        return c
    bt = np.where(w.block_table >= 0, w.block_table + extra, -1).astype(np.int32)
    vc = None if w.v_cache is None else one(w.v_cache)
    return inputs.Paged(w.q, one(w.k_cache), vc, bt, w.cache_seqlens, w.page_size, w.dv,
                        w.scale, w.causal)


def test_decode_gqa_unreferenced_pages_poisoned():
    """Unreferenced pool pages and the rows past each sequence's length are
    NaN (see poison_pool)."""
    lens = [100, 64, 7]
    w = inputs.paged(91, lens, sq=1, hq=8, hkv=2, d=128, page=16)
    w2 = poison_pool(w, 5)
    o, lse, _ = run_decode(w2)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w)
    compare("poisoned_pool", o, lse, ro, rl, TOL_O_BF16)


def test_decode_gqa_full():
    """Full workload: batch 64, lengths U[1024, 32768], page 64, Hq=32, Hkv=8,
    D=128, with the plan the benchmark times (binding.GQA_DECODE_PLAN); every
    sequence compared element by element, and the plan bit for bit."""
    w = inputs.paged_decode()
    log("case decode_gqa_full seed", inputs.SEED_PAGED_DECODE, "plan", B.GQA_DECODE_PLAN)
    o, lse, plan = run_decode(w, *B.GQA_DECODE_PLAN)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(w)
    compare("decode_gqa_full", o, lse, ro, rl, TOL_O_BF16)
    ms, waves, mb = B.GQA_DECODE_PLAN
    ref_plan = orc.plan_splits(w.cache_seqlens, 64, 8, B.attn_device_info(0), waves, ms, mb)
    assert_plan_equal(host(plan), ref_plan, len(w.cache_seqlens), ms)


# ----------------------------------------------------------------------- MLA
def run_mla(w, max_splits=16, waves=2, min_blocks=4):
    return B.mla_decode(dev(w.q), dev(w.k_cache), dev(w.block_table), dev(w.cache_seqlens),
                        w.scale, w.causal, max_splits=max_splits, waves=waves,
                        min_blocks=min_blocks)


def oracle_mla(w, batches=None):
    q, kc = inputs.bits_to_f32(w.q), inputs.bits_to_f32(w.k_cache)
    return orc.mla_decode_paged(q, kc, w.block_table, w.cache_seqlens, w.page_size, w.scale,
                                w.causal, 512, batches)


MLA_CASES = [
    ("mla_small", [100, 1, 700], 2, 16, 64, False, 16, 2, 1),
    ("mla_causal_sq4", [65, 300], 4, 32, 16, True, 8, 8, 1),
    ("mla_hq128", [2000, 513], 1, 128, 64, False, 16, 2, 2),
    # 192 rows: two row tiles, the second half empty; causal, 16-row pages
    ("mla_causal_2tiles", [37, 1000, 129], 3, 64, 16, True, 8, 3, 1),
    # many short splits on 32-row pages, sequence shorter than one tile
    ("mla_many_splits", [4000, 31, 2048], 2, 128, 32, False, 16, 8, 1),
]


@pytest.mark.parametrize("case", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_mla_decode(case):
    name, lens, sq, hq, page, causal, ms, waves, mb = case
    log("case", name)
    w = inputs.paged(6000 + len(name), lens, sq=sq, hq=hq, hkv=1, d=576, dv=512, page=page,
                     shared_kv=True, causal=causal)
    o, lse, _ = run_mla(w, ms, waves, mb)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(w)
    compare(name, o, lse, ro, rl, TOL_O_BF16)


def test_mla_decode_poisoned():
    """MLA over a pool with NaN outside every sequence's rows (see poison_pool);
    lengths end mid-tile and mid-page."""
    w = inputs.paged(6100, [100, 47, 300], sq=2, hq=64, hkv=1, d=576, dv=512, page=16,
                     shared_kv=True)
    w2 = poison_pool(w, 3)
    o, lse, _ = run_mla(w2, 8, 4, 1)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(w)
    compare("mla_poisoned", o, lse, ro, rl, TOL_O_BF16)


def test_mla_decode_full():
    """Full workload: batch 64, 2 query tokens, Hq=128, one 576-wide KV head,
    V = first 512 entries, page 64, lengths U[2048, 16384], with the plan the
    benchmark times (binding.MLA_DECODE_PLAN); every sequence compared element
    by element, and the plan bit for bit."""
    w = inputs.mla_decode()
    log("case mla_decode_full seed", inputs.SEED_MLA_DECODE, "plan", B.MLA_DECODE_PLAN)
    o, lse, plan = run_mla(w, *B.MLA_DECODE_PLAN)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(w)
    compare("mla_decode_full", o, lse, ro, rl, TOL_O_BF16)
    ms, waves, mb = B.MLA_DECODE_PLAN
    ref_plan = orc.plan_splits(w.cache_seqlens, 64, 2, B.attn_device_info(0), waves, ms, mb)
    assert_plan_equal(host(plan), ref_plan, len(w.cache_seqlens), ms)


def test_mla_mate_example():
    """The MATE minimal MLA example on the GPU: q (1, 32, 8, 576), k_cache
    (4, 16, 2, 576) (two KV heads, four query heads each), block_table zeros
    (1, 4), page 16, cache_seqlens [32], head_dim_v 512. Every logical page
    is physical page 0, so keys 16..31 repeat keys 0..15: besides matching the
    oracle, O equals attention over page 0's 16 keys and LSE is theirs + ln 2."""
    w = inputs.mla_mate_example()
    log("case mla_mate_example")
    o, lse, _ = run_mla(w, 16, 8, 1)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(w)
    compare("mla_mate_example", o, lse, ro, rl, TOL_O_BF16)
    q, kc = inputs.bits_to_f32(w.q), inputs.bits_to_f32(w.k_cache)
    k16 = kc[0][None]
    o16, l16 = orc.attention_dense(q, k16, k16[..., :512], w.scale)
    compare("mla_mate_example_16_keys", o, lse, o16, l16 + np.log(2.0), TOL_O_BF16)


# MLA rows with several KV heads (attn_decode_paged, d = 576, dv = 512) and
# head counts that are not multiples of 16
MLA_GQA_CASES = [
    # name, lens, sq, hq, hkv, page, causal, max_splits, waves, min_blocks
    ("hkv2_hq8_sq32", [32, 300], 32, 8, 2, 16, False, 16, 8, 1),
    ("hkv4_hq20_sq3_causal", [50, 1000, 7], 3, 20, 4, 32, True, 8, 16, 1),
    ("hkv1_hq24_sq2", [100, 513], 2, 24, 1, 64, False, 16, 4, 2),
    ("hkv2_hq256_sq1", [2000, 64], 1, 256, 2, 64, False, 8, 3, 2),
]


@pytest.mark.parametrize("case", MLA_GQA_CASES, ids=[c[0] for c in MLA_GQA_CASES])
def test_mla_decode_hkv(case):
    name, lens, sq, hq, hkv, page, causal, ms, waves, mb = case
    log("case", name)
    w = inputs.paged(6200 + len(name), lens, sq=sq, hq=hq, hkv=hkv, d=576, dv=512, page=page,
                     shared_kv=True, causal=causal)
    o, lse, _ = run_mla(w, ms, waves, mb)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(w)
    compare(name, o, lse, ro, rl, TOL_O_BF16)


def test_decode_peaky_q():
    """The paged-decode and MLA workloads with Q scaled by 4 (exact in bf16):
    sharper softmax rows, so an output error cannot hide behind the small |O|
    of rows averaging thousands of keys; four sequences of each compared
    element by element."""
    w = inputs.paged_decode()
    w.q = inputs.bf16_bits(inputs.bits_to_f32(w.q) * 4)
    log("case decode_peaky")
    o, lse, _ = run_decode(w, *B.GQA_DECODE_PLAN)
    torch.cuda.synchronize()
    pick = [0, 21, 42, 63]
    ro, rl = oracle_decode(w, batches=pick)
    mask = np.zeros(ro.shape, bool)
    mask[pick] = True
    compare("decode_peaky", o, lse, ro, rl, TOL_O_BF16, mask=mask)
    m = inputs.mla_decode()
    m.q = inputs.bf16_bits(inputs.bits_to_f32(m.q) * 4)
    log("case mla_peaky")
    o, lse, _ = run_mla(m, *B.MLA_DECODE_PLAN)
    torch.cuda.synchronize()
    pick = [0, 31, 63]
    ro, rl = oracle_mla(m, batches=pick)
    mask = np.zeros(ro.shape, bool)
    mask[pick] = True
    compare("mla_peaky", o, lse, ro, rl, TOL_O_BF16, mask=mask)
