"""Pins for the float64 oracle, checked against what the pages and mathematics
fix: hand-derived closed forms (tests/golden), invariants, special cases that
reduce to a library routine, and brute force on tiny inputs. A final test
plants typical mistakes in the oracle and checks that the pins catch each one.
CPU only."""
import json
import math
import os

import numpy as np
import pytest

from attention_attn_fwd_02_amd import inputs
from oracle import attention as orc
from oracle import brute
from oracle import fp8 as ofp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- closed forms
def check_golden():
    with open(GOLDEN) as f:
        cases = json.load(f)
    for c in cases:
        if c["kind"] == "rows":
            o, lse = orc.attend_rows(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                     c["scale"], None, c.get("sink"))
        elif c["kind"] == "dense":
            o, lse = orc.attention_dense(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                         c["scale"], c["causal"], tuple(c["window"]))
        elif c["kind"] == "combine":
            op = np.array(c["o_partial"])[:, :, :]          # (2 splits, 1 row, 2)
            lp = np.array(c["lse_partial"])                  # (2, 1)
            o, lse = orc.combine(op, lp, [0, 2], 1, 1, 1, 2)
            np.testing.assert_allclose(o.ravel(), c["o"], rtol=0, atol=1e-14, err_msg=c["name"])
            np.testing.assert_allclose(lse.ravel(), [c["lse"]], rtol=0, atol=1e-14)
            o, lse = orc.combine(op, lp, [0, 2], 1, 1, 1, 2, sinks=[c["sink"]])
            np.testing.assert_allclose(o.ravel(), c["o_sink"], rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse.ravel(), [c["lse"]], rtol=0, atol=1e-14)
            continue
        elif c["kind"] == "sparse":
            sk = c["sk"]
            q = np.zeros((1, c["sq"], 1, 2))
            kv = np.zeros((1, sk, 1, 2))
            kv[0, :, 0, 0] = np.arange(sk)        # value (first entry) = key index
            idx = np.array(c["indices"], dtype=np.int32).reshape(1, 1, 1, -1)
            o, lse = orc.mla_sparse(q, kv, idx, 1.0, c["mode"], None, dv=1)
            np.testing.assert_allclose(o.ravel(), [c["o"]], rtol=0, atol=1e-14, err_msg=c["name"])
            np.testing.assert_allclose(lse.ravel(), [c["lse"]], rtol=0, atol=1e-14)
            continue
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-13, err_msg=c["name"])


def test_golden_closed_forms():
    check_golden()


# ------------------------------------------------------------------ invariants
def check_rows_sum_to_one():
    """With V = identity the output row is the probability row itself."""
    rng = _rng(1)
    n = 9
    q, k = rng.standard_normal((5, 4)), rng.standard_normal((n, 4))
    vis = orc.visible_band(5, n, True, 2, -1)
    o, _ = orc.attend_rows(q, k, np.eye(n), 0.7, vis)
    np.testing.assert_allclose(o.sum(axis=1), 1.0, atol=1e-12)
    assert (o >= 0).all() and (o[~vis] == 0).all()


def test_rows_sum_to_one():
    check_rows_sum_to_one()


def check_lse_identity():
    rng = _rng(2)
    q, k, v = rng.standard_normal((6, 5)), rng.standard_normal((11, 5)), rng.standard_normal((11, 3))
    vis = orc.visible_band(6, 11, True)
    _, lse = orc.attend_rows(q, k, v, 0.4, vis)
    for i in range(6):
        s = [0.4 * math.fsum(q[i] * k[j]) for j in range(11) if vis[i, j]]
        mx = max(s)
        ref = math.log(math.fsum(math.exp(x - mx) for x in s)) + mx
        assert abs(lse[i] - ref) <= 1e-12
        assert mx - 1e-12 <= lse[i] <= mx + math.log(len(s)) + 1e-12


def test_lse_identity():
    check_lse_identity()


def check_identical_keys():
    """All keys equal: O is the mean of the values, LSE = S + log|J|."""
    rng = _rng(3)
    q = rng.standard_normal((4, 8))
    k = np.tile(rng.standard_normal((1, 8)), (7, 1))
    v = rng.standard_normal((7, 5))
    o, lse = orc.attend_rows(q, k, v, 0.3, None)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (4, 1)), atol=1e-13)
    np.testing.assert_allclose(lse, 0.3 * (q @ k[0]) + math.log(7), atol=1e-13)


def test_identical_keys():
    check_identical_keys()


def check_single_key():
    rng = _rng(4)
    q, k, v = rng.standard_normal((3, 6)), rng.standard_normal((1, 6)), rng.standard_normal((1, 4))
    o, lse = orc.attend_rows(q, k, v, 1.3, None)
    np.testing.assert_allclose(o, np.tile(v, (3, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, 1.3 * (q @ k[0]), atol=1e-14)


def test_single_key():
    check_single_key()


def check_sink():
    """O_sink = O * sigmoid(LSE - sink); sink -> -inf gives O, sink -> +inf gives 0."""
    rng = _rng(5)
    q, k, v = rng.standard_normal((5, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 3))
    vis = orc.visible_band(5, 9, True)
    o, lse = orc.attend_rows(q, k, v, 0.8, vis)
    for sink in (-2.0, 0.3, 1.7):
        os_, ls = orc.attend_rows(q, k, v, 0.8, vis, sink)
        np.testing.assert_allclose(os_, o / (1 + np.exp(sink - lse))[:, None], atol=1e-13)
        np.testing.assert_allclose(ls, lse, atol=0)
    np.testing.assert_allclose(orc.attend_rows(q, k, v, 0.8, vis, -1e30)[0], o, atol=1e-14)
    np.testing.assert_allclose(orc.attend_rows(q, k, v, 0.8, vis, 1e30)[0], 0.0, atol=1e-14)


def test_sink():
    check_sink()


def test_empty_rows():
    q, k, v = np.ones((2, 3)), np.ones((0, 3)), np.ones((0, 2))
    o, lse = orc.attend_rows(q, k, v, 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()
    vis = np.zeros((2, 4), bool)
    o, lse = orc.attend_rows(q, np.ones((4, 3)), np.ones((4, 2)), 1.0, vis, 0.5)
    assert (o == 0).all() and np.isneginf(lse).all()


# ----------------------------------------------------------- split and combine
def _random_plan(rng, lens, max_splits):
    """A hand-made plan with arbitrary cut points (including single-key and
    empty-key splits), independent of the planner rule."""
    ptr, tri = [0], []
    for b, n in enumerate(lens):
        ns = int(rng.integers(1, max_splits + 1))
        cuts = np.sort(rng.integers(0, n + 1, size=ns - 1)) if n else np.zeros(ns - 1, int)
        edges = [0, *cuts.tolist(), n]
        for s in range(ns):
            tri.append((b, edges[s], edges[s + 1]))
        ptr.append(ptr[-1] + ns)
    plan = np.zeros(orc.plan_words(len(lens), max_splits), np.int32)
    plan[0], plan[1] = len(tri), 0
    plan[2:3 + len(lens)] = ptr
    plan[3 + len(lens):3 + len(lens) + 3 * len(tri)] = np.array(tri).ravel()
    return plan


def check_split_combine():
    rng = _rng(6)
    for causal, with_sink in ((False, False), (True, True)):
        lens = [1, 5, 37, 64]
        p = inputs.paged(11, lens, sq=2, hq=4, hkv=2, d=8, page=4, causal=causal,
                         with_sinks=with_sink)
        q, kc, vc = (inputs.bits_to_f32(x) for x in (p.q, p.k_cache, p.v_cache))
        ref_o, ref_l = orc.attention_paged(q, kc, vc, p.block_table, p.cache_seqlens, 4, p.scale,
                                           causal, p.sinks)
        for _ in range(3):
            plan = _random_plan(rng, lens, 6)
            op, lp = orc.attention_paged_split(q, kc, vc, p.block_table, p.cache_seqlens, 4,
                                               p.scale, plan, 6, causal)
            ptr, _ = orc.plan_unpack(plan, len(lens))
            o, l = orc.combine(op, lp, ptr, len(lens), 2, 4, 6, p.sinks)
            np.testing.assert_allclose(o, ref_o, atol=1e-12)
            np.testing.assert_allclose(l, ref_l, atol=1e-12)


def test_split_combine():
    check_split_combine()


# ------------------------------------------------------------- GQA and varlen
def check_gqa_equals_mha():
    d = inputs.varlen(7, [5, 9], hq=6, hkv=2, d=8, causal=True)
    q, k, v = d.f32("q"), d.f32("k"), d.f32("v")
    o, lse = orc.attention_varlen(q, k, v, d.cu_seqlens_q, d.cu_seqlens_k, d.scale, True)
    o2, lse2 = orc.attention_varlen(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1),
                                    d.cu_seqlens_q, d.cu_seqlens_k, d.scale, True)
    np.testing.assert_allclose(o, o2, atol=0)
    np.testing.assert_allclose(lse, lse2, atol=0)


def test_gqa_equals_mha():
    check_gqa_equals_mha()


def check_varlen_equals_dense():
    lq, lk = [3, 8, 1], [6, 8, 4]
    d = inputs.varlen(8, lq, lk, hq=4, hkv=2, d=8, causal=True, window=(3, -1))
    q, k, v = d.f32("q"), d.f32("k"), d.f32("v")
    o, lse = orc.attention_varlen(q, k, v, d.cu_seqlens_q, d.cu_seqlens_k, d.scale, True, (3, -1))
    for b in range(3):
        a0, a1 = d.cu_seqlens_q[b], d.cu_seqlens_q[b + 1]
        c0, c1 = d.cu_seqlens_k[b], d.cu_seqlens_k[b + 1]
        ob, lb = orc.attention_dense(q[None, a0:a1], k[None, c0:c1], v[None, c0:c1], d.scale,
                                     True, (3, -1))
        np.testing.assert_allclose(o[a0:a1], ob[0], atol=0)
        np.testing.assert_allclose(lse[:, a0:a1], lb[0], atol=0)


def test_varlen_equals_dense():
    check_varlen_equals_dense()


# ------------------------------------------------------------------ paged KV
def check_paged_equals_contiguous():
    p = inputs.paged(9, [13, 40, 1], sq=3, hq=4, hkv=2, d=8, page=8, causal=True)
    q, kc, vc = (inputs.bits_to_f32(x) for x in (p.q, p.k_cache, p.v_cache))
    o, lse = orc.attention_paged(q, kc, vc, p.block_table, p.cache_seqlens, 8, p.scale, True)
    for b, n in enumerate(p.cache_seqlens):
        # contiguous copy made by explicit loops, not by the oracle's gather
        kk = np.stack([kc[p.block_table[b, j // 8], j % 8] for j in range(n)])
        vv = np.stack([vc[p.block_table[b, j // 8], j % 8] for j in range(n)])
        ob, lb = orc.attention_dense(q[b:b + 1], kk[None], vv[None], p.scale, True)
        np.testing.assert_allclose(o[b], ob[0], atol=0)
        np.testing.assert_allclose(lse[b], lb[0], atol=0)
    # page-pool permutation invariance
    rng = _rng(10)
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    table = np.where(p.block_table >= 0, inv[np.maximum(p.block_table, 0)], -1)
    o2, l2 = orc.attention_paged(q, kc[perm], vc[perm], table, p.cache_seqlens, 8, p.scale, True)
    np.testing.assert_allclose(o2, o, atol=0)
    np.testing.assert_allclose(l2, lse, atol=0)


def test_paged_equals_contiguous():
    check_paged_equals_contiguous()


# ------------------------------------------------- cache + current K/V (split-KV)
def _kvcache_case(seed, lq, ln, lc, hq=4, hkv=2, d=4, page=4):
    """Tiny varlen problem: per sequence lq[b] queries, ln[b] current K/V rows
    and lc[b] cached rows in a shuffled page pool (float values)."""
    rng = _rng(seed)
    bsz = len(lq)
    q = rng.standard_normal((sum(lq), hq, d))
    k = rng.standard_normal((sum(ln), hkv, d))
    v = rng.standard_normal((sum(ln), hkv, d))
    npg = [(n + page - 1) // page for n in lc]
    pool = sum(npg) + 2
    kc = rng.standard_normal((pool, page, hkv, d))
    vc = rng.standard_normal((pool, page, hkv, d))
    perm = rng.permutation(pool)
    table = np.full((bsz, max(max(npg), 1)), -1, np.int64)
    at = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[at:at + n]
        at += n
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(ln)])
    return q, k, v, cq, ck, kc, vc, table, np.asarray(lc), page


def check_kvcache_brute_force():
    """Brute force with its own key list: cache rows read slot by slot, then
    the current rows, bottom-right causal over the whole key sequence."""
    q, k, v, cq, ck, kc, vc, table, lc, page = _kvcache_case(41, [3, 1, 4], [2, 0, 4], [5, 3, 0])
    o, lse = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.7, True)
    grp = q.shape[1] // k.shape[1]
    for b in range(len(lc)):
        nq, nn, nc = cq[b + 1] - cq[b], ck[b + 1] - ck[b], int(lc[b])
        for h in range(q.shape[1]):
            g = h // grp
            keys = [list(kc[table[b, j // page], j % page, g]) for j in range(nc)]
            vals = [list(vc[table[b, j // page], j % page, g]) for j in range(nc)]
            keys += [list(k[ck[b] + j, g]) for j in range(nn)]
            vals += [list(v[ck[b] + j, g]) for j in range(nn)]
            lk = nc + nn
            qs = [list(q[cq[b] + t, h]) for t in range(nq)]
            ob, lb = brute.rows(qs, keys, vals, 0.7, visible=lambda t, j: j <= t + lk - nq)
            for t in range(nq):
                if math.isinf(lb[t]):
                    assert np.isneginf(lse[h, cq[b] + t]) and not o[cq[b] + t, h].any()
                    continue
                assert abs(lse[h, cq[b] + t] - lb[t]) <= 1e-12
                np.testing.assert_allclose(o[cq[b] + t, h], ob[t], atol=1e-12)


def check_kvcache_special_cases():
    # an empty cache is plain varlen attention over the current rows
    q, k, v, cq, ck, kc, vc, table, lc, page = _kvcache_case(42, [4, 2], [4, 5], [0, 0])
    o, lse = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.5, True)
    o2, l2 = orc.attention_varlen(q, k, v, cq, ck, 0.5, True)
    np.testing.assert_allclose(o, o2, atol=0)
    np.testing.assert_allclose(lse, l2, atol=0)
    # chunked prefill: a sequence's first rows cached (slot by slot), the rest
    # current, queries = the last rows; equals attention over the whole
    # contiguous sequence with those queries (bottom-right causal)
    rng = _rng(43)
    total, lq, page, hq, hkv, d = 11, 4, 4, 2, 1, 4
    kf = rng.standard_normal((total, hkv, d))
    vf = rng.standard_normal((total, hkv, d))
    qf = rng.standard_normal((lq, hq, d))
    lcache = total - lq
    npg = (lcache + page - 1) // page
    kc = np.zeros((npg + 1, page, hkv, d))
    vc = np.zeros((npg + 1, page, hkv, d))
    table = np.array([[npg - i for i in range(npg)]])   # pages in reverse pool order
    for j in range(lcache):
        kc[table[0, j // page], j % page] = kf[j]
        vc[table[0, j // page], j % page] = vf[j]
    o, lse = orc.attention_varlen_kvcache(qf, kf[lcache:], vf[lcache:], np.array([0, lq]),
                                          np.array([0, lq]), kc, vc, table,
                                          np.array([lcache]), page, 0.6, True)
    o2, l2 = orc.attention_varlen(qf, kf, vf, np.array([0, lq]), np.array([0, total]), 0.6, True)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, l2, atol=1e-14)


def check_additive_mask():
    """Additive mask [MOJO input_mask_fn]: zeros change nothing; a constant c
    on every key of a row leaves O and adds c to LSE (softmax is shift
    invariant); -inf entries equal removing those keys; a finite mask agrees
    with brute force on exp(scale q.k + mask)."""
    q, k, v, cq, ck, kc, vc, table, lc, page = _kvcache_case(44, [4, 3], [4, 3], [5, 2])
    tq, hq = q.shape[0], q.shape[1]
    ld = 12
    base = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True)
    z = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True,
                                     mask=np.zeros((1, tq, ld)))
    np.testing.assert_allclose(z[0], base[0], atol=0)
    c = np.linspace(-1.5, 0.75, hq)[:, None, None] * np.ones((hq, tq, ld))
    sh = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True,
                                      mask=c)
    np.testing.assert_allclose(sh[0], base[0], atol=1e-13)
    np.testing.assert_allclose(sh[1], base[1] + c[:, :, 0], atol=1e-13)
    # a random mask with -inf on key 0 of every row, against brute force that
    # drops key 0 and adds the mask to each remaining score
    rng = _rng(45)
    m = rng.standard_normal((hq, tq, ld))
    m[:, :, 0] = -np.inf
    o, lse = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True,
                                          mask=m)
    grp = hq // k.shape[1]
    for b in range(len(lc)):
        nq, nn, nc = cq[b + 1] - cq[b], ck[b + 1] - ck[b], int(lc[b])
        for h in range(hq):
            g = h // grp
            keys = [list(kc[table[b, j // page], j % page, g]) for j in range(nc)]
            vals = [list(vc[table[b, j // page], j % page, g]) for j in range(nc)]
            keys += [list(k[ck[b] + j, g]) for j in range(nn)]
            vals += [list(v[ck[b] + j, g]) for j in range(nn)]
            lk = nc + nn
            for t in range(nq):
                r = cq[b] + t
                w = [math.exp(0.6 * sum(a * bb for a, bb in zip(q[r, h], keys[j])) + m[h, r, j])
                     if (j <= t + lk - nq and j > 0) else 0.0 for j in range(lk)]
                tot = math.fsum(w)
                if tot == 0.0:
                    assert np.isneginf(lse[h, r])
                    continue
                assert abs(lse[h, r] - math.log(tot)) <= 1e-12
                ref = [math.fsum(w[j] * vals[j][e] for j in range(lk)) / tot
                       for e in range(v.shape[2])]
                np.testing.assert_allclose(o[r, h], ref, rtol=0, atol=1e-12)


def test_additive_mask():
    check_additive_mask()


def check_kvcache_qv():
    """qv over a cache plus current rows [MATE FMHA notes: qv; MOJO cache +
    current K/V]. With K = 0 (cached and current) and qv = q the scores are
    scale q.v, so the result is the plain cache-plus-current attention with V
    in the role of K; only_qv with qv equals that attention with qv as the
    query and V as the keys; with no cached rows it is attention_varlen with
    the same qv; and qv = 0 leaves the plain result."""
    q, k, v, cq, ck, kc, vc, table, lc, page = _kvcache_case(61, [4, 3, 2], [3, 4, 0], [5, 2, 6])
    plain_vk = orc.attention_varlen_kvcache(q, v, v, cq, ck, vc, vc, table, lc, page, 0.6, True)
    got = orc.attention_varlen_kvcache(q, np.zeros_like(k), v, cq, ck, np.zeros_like(kc), vc,
                                       table, lc, page, 0.6, True, qv=q)
    np.testing.assert_allclose(got[0], plain_vk[0], atol=1e-13)
    np.testing.assert_allclose(got[1], plain_vk[1], atol=1e-13)
    qv = _rng(62).standard_normal(q.shape)
    only = orc.attention_varlen_kvcache(None, None, v, cq, ck, None, vc, table, lc, page, 0.6,
                                        True, qv=qv, only_qv=True)
    ref = orc.attention_varlen_kvcache(qv, v, v, cq, ck, vc, vc, table, lc, page, 0.6, True)
    np.testing.assert_allclose(only[0], ref[0], atol=1e-13)
    np.testing.assert_allclose(only[1], ref[1], atol=1e-13)
    none = np.zeros(len(lc), np.int64)
    a = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, none, page, 0.6, True, qv=qv)
    b = orc.attention_varlen(q, k, v, cq, ck, 0.6, True, qv=qv)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13, equal_nan=True)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13, equal_nan=True)
    z = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True,
                                     qv=np.zeros_like(q))
    base = orc.attention_varlen_kvcache(q, k, v, cq, ck, kc, vc, table, lc, page, 0.6, True)
    np.testing.assert_allclose(z[0], base[0], atol=1e-13)
    # a planted mistake (the qv term dropped) fails the first identity
    bad = orc.attention_varlen_kvcache(q, np.zeros_like(k), v, cq, ck, np.zeros_like(kc), vc,
                                       table, lc, page, 0.6, True)
    assert not np.allclose(bad[0], plain_vk[0], atol=1e-6)


def test_kvcache_qv():
    check_kvcache_qv()


def check_paged_mask():
    """Additive mask on the paged decode [MOJO input_mask_fn]: zeros change
    nothing; a constant c per (sequence, head) leaves O and adds c to LSE; a
    shared plane equals the same plane repeated per head; a random mask with
    -inf entries agrees with brute force over the rows gathered by explicit
    page/slot loops; and split partials combined equal the unsplit result."""
    p = inputs.paged(46, [13, 40, 1], sq=3, hq=4, hkv=2, d=8, page=8, causal=True)
    q, kc, vc = (inputs.bits_to_f32(x) for x in (p.q, p.k_cache, p.v_cache))
    bsz, sq, hq = q.shape[0], q.shape[1], q.shape[2]
    ld = 48
    args = (q, kc, vc, p.block_table, p.cache_seqlens, 8, p.scale, True)
    base = orc.attention_paged(*args)
    z = orc.attention_paged(*args, mask=np.zeros((bsz, 1, sq, ld)))
    np.testing.assert_allclose(z[0], base[0], atol=0)
    np.testing.assert_allclose(z[1], base[1], atol=0)
    c = np.linspace(-1.25, 2.0, bsz * hq).reshape(bsz, hq)
    sh = orc.attention_paged(*args, mask=c[:, :, None, None] * np.ones((bsz, hq, sq, ld)))
    np.testing.assert_allclose(sh[0], base[0], atol=1e-13)
    fin = np.isfinite(base[1])
    np.testing.assert_allclose(sh[1][fin], (base[1] + c[:, :, None])[fin], atol=1e-13)
    rng = _rng(47)
    one = rng.standard_normal((bsz, 1, sq, ld))
    a1 = orc.attention_paged(*args, mask=one)
    a2 = orc.attention_paged(*args, mask=np.repeat(one, hq, axis=1))
    np.testing.assert_allclose(a1[0], a2[0], atol=0)
    np.testing.assert_allclose(a1[1], a2[1], atol=0)
    m = rng.standard_normal((bsz, hq, sq, ld))
    m[rng.random(m.shape) < 0.2] = -np.inf
    o, lse = orc.attention_paged(*args, mask=m)
    grp = hq // kc.shape[2]
    for b in range(bsz):
        n = int(p.cache_seqlens[b])
        for h in range(hq):
            g = h // grp
            # Python floats throughout (float32 scalars would keep float32 products)
            keys = [kc[p.block_table[b, j // 8], j % 8, g].tolist() for j in range(n)]
            vals = [vc[p.block_table[b, j // 8], j % 8, g].tolist() for j in range(n)]
            for t in range(sq):
                qt = q[b, t, h].tolist()
                w = [math.exp(p.scale * math.fsum(x * y for x, y in zip(qt, keys[j]))
                              + m[b, h, t, j])
                     if j <= t + n - sq and np.isfinite(m[b, h, t, j]) else 0.0
                     for j in range(n)]
                tot = math.fsum(w)
                if tot == 0.0:
                    assert np.isneginf(lse[b, h, t])
                    continue
                assert abs(lse[b, h, t] - math.log(tot)) <= 1e-12
                ref = [math.fsum(w[j] * vals[j][e] for j in range(n)) / tot
                       for e in range(vc.shape[3])]
                np.testing.assert_allclose(o[b, t, h], ref, rtol=0, atol=1e-12)
    # split partials combined equal the unsplit masked decode
    plan = orc.plan_splits(p.cache_seqlens, 8, 2, 4, 8, 4, 1)
    op, lp = orc.attention_paged_split(q, kc, vc, p.block_table, p.cache_seqlens, 8, p.scale,
                                       plan, 4, True, mask=m)
    ptr, _ = orc.plan_unpack(plan, bsz)
    oc, lc = orc.combine(op, lp, ptr, bsz, sq, hq, 4)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(lc, lse, atol=1e-12)


def test_paged_mask():
    check_paged_mask()


def test_kvcache_brute_force():
    check_kvcache_brute_force()


def test_kvcache_special_cases():
    check_kvcache_special_cases()


# ------------------------------------------------------------------ FP8 inputs
def check_fp8_decode_library():
    """Every code of both formats against torch's float8 dtypes (a library
    conversion): equal values, NaN exactly where torch has NaN."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        ref = torch.from_numpy(codes).view(dt).to(torch.float64).numpy()
        got = ofp8.decode(codes, fmt)
        assert np.array_equal(np.isnan(ref), np.isnan(got)), fmt
        fin = ~np.isnan(ref)
        assert np.array_equal(ref[fin], got[fin]), fmt
        assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin])), fmt


def check_fp8_decode_values():
    """Codes whose values follow from the format definitions by hand."""
    known = {"e4m3": {0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
                      0x08: 2.0 ** -6, 0x3C: 1.5, 0x00: 0.0},
             "e5m2": {0x3C: 1.0, 0xBC: -1.0, 0x7B: 57344.0, 0x7C: math.inf, 0xFC: -math.inf,
                      0x01: 2.0 ** -16, 0x04: 2.0 ** -14, 0x3E: 1.5}}
    for fmt, table in known.items():
        for code, val in table.items():
            assert ofp8.decode(np.array([code], np.uint8), fmt)[0] == val, (fmt, hex(code))
    assert np.isnan(ofp8.decode(np.array([0x7F, 0xFF], np.uint8), "e4m3")).all()
    assert np.isnan(ofp8.decode(np.array([0x7D, 0x7F], np.uint8), "e5m2")).all()
    assert np.signbit(ofp8.decode(np.array([0x80], np.uint8), "e4m3")[0])


def _fp8_case(seed, fmt, descale=True):
    return inputs.paged_fp8(seed, [5, 3], fmt, sq=2, hq=4, hkv=2, d=4, page=4, causal=True,
                            descale=descale)


def check_fp8_attention_brute():
    """Brute force on values dequantized by an independent path (torch's
    float8 conversion times the descale of (batch, h // (Hq/Hkv)))."""
    import torch
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        w = _fp8_case(61, fmt)
        o, lse = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, fmt, w.q_descale,
                                          w.k_descale, w.v_descale, w.block_table,
                                          w.cache_seqlens, w.page_size, w.scale, True)
        deq = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(dt).to(torch.float64).numpy()
        bsz, sq, hq, _ = w.q.shape
        grp = hq // w.k_cache.shape[2]
        for b in range(bsz):
            n = int(w.cache_seqlens[b])
            rows = [(w.block_table[b, j // w.page_size], j % w.page_size) for j in range(n)]
            for h in range(hq):
                g = h // grp
                qs = [list(deq(w.q[b, t, h]) * float(w.q_descale[b, g])) for t in range(sq)]
                ks = [list(deq(w.k_cache[p, s, g]) * float(w.k_descale[b, g])) for p, s in rows]
                vs = [list(deq(w.v_cache[p, s, g]) * float(w.v_descale[b, g])) for p, s in rows]
                ob, lb = brute.rows(qs, ks, vs, w.scale, visible=lambda t, j: j <= t + n - sq)
                for t in range(sq):
                    assert abs(lse[b, h, t] - lb[t]) <= 1e-12
                    np.testing.assert_allclose(o[b, t, h], ob[t], rtol=0, atol=1e-12)


def check_fp8_descale_identities():
    """Only the product of the Q and K descales enters the scores; the V
    descale scales O and leaves LSE unchanged."""
    w = _fp8_case(62, "e4m3")
    args = (w.block_table, w.cache_seqlens, w.page_size, w.scale, True)
    o, lse = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, "e4m3", w.q_descale,
                                      w.k_descale, w.v_descale, *args)
    o2, l2 = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, "e4m3", w.q_descale * 2,
                                      w.k_descale / 2, w.v_descale.astype(np.float64) * 3,
                                      *args)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o2, o * 3, rtol=1e-12, atol=1e-12)
    # unit descales are the plain paged decode of the decoded codes
    o1, l1 = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, "e4m3", None, None, None, *args)
    o3, l3 = orc.attention_paged(ofp8.decode(w.q, "e4m3"), ofp8.decode(w.k_cache, "e4m3"),
                                 ofp8.decode(w.v_cache, "e4m3"), *args)
    np.testing.assert_allclose(o1, o3, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l3, rtol=0, atol=1e-14)


def check_fp8_varlen():
    """Varlen FP8: brute force on values dequantized by torch's float8
    conversion and the (sequence, h // (Hq/Hkv)) descales; unit descales are
    plain varlen attention on the decoded codes."""
    import torch
    w = inputs.varlen_fp8(63, [3, 5], [4, 5], "e5m2", hq=4, hkv=2, d=4, causal=True)
    o, lse = ofp8.attention_varlen_fp8(w.q, w.k, w.v, "e5m2", w.q_descale, w.k_descale,
                                       w.v_descale, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True)
    deq = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e5m2).to(
        torch.float64).numpy()
    cq, ck = w.cu_seqlens_q, w.cu_seqlens_k
    for b in range(2):
        nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for h in range(4):
            g = h // 2
            qs = [list(deq(w.q[cq[b] + t, h]) * float(w.q_descale[b, g])) for t in range(nq)]
            ks = [list(deq(w.k[ck[b] + j, g]) * float(w.k_descale[b, g])) for j in range(nk)]
            vs = [list(deq(w.v[ck[b] + j, g]) * float(w.v_descale[b, g])) for j in range(nk)]
            ob, lb = brute.rows(qs, ks, vs, w.scale, visible=lambda t, j: j <= t + nk - nq)
            for t in range(nq):
                assert abs(lse[h, cq[b] + t] - lb[t]) <= 1e-12
                np.testing.assert_allclose(o[cq[b] + t, h], ob[t], rtol=0, atol=1e-12)
    o1, l1 = ofp8.attention_varlen_fp8(w.q, w.k, w.v, "e5m2", None, None, None, cq, ck,
                                       w.scale, True)
    o2, l2 = orc.attention_varlen(ofp8.decode(w.q, "e5m2"), ofp8.decode(w.k, "e5m2"),
                                  ofp8.decode(w.v, "e5m2"), cq, ck, w.scale, True)
    np.testing.assert_allclose(o1, o2, atol=0)
    np.testing.assert_allclose(l1, l2, atol=0)


def check_fp8_qv():
    """FP8 qv: brute force on torch-dequantized codes (qv with the query
    descale, scored against the descaled V rows), with and without the QK
    path; unit descales equal the real-valued oracle on the decoded codes."""
    import torch
    w = inputs.paged_fp8(64, [6, 11], "e4m3", sq=2, hq=4, hkv=2, d=4, page=4, causal=True,
                         with_qv=True)
    deq = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    for only in (False, True):
        o, lse = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, "e4m3", w.q_descale,
                                          w.k_descale, w.v_descale, w.block_table,
                                          w.cache_seqlens, w.page_size, w.scale, True,
                                          qv8=w.qv, only_qv=only)
        for b, lk in enumerate(w.cache_seqlens):
            rows = [orc.gather_paged(c, w.block_table, b, int(lk), w.page_size)
                    for c in (w.k_cache, w.v_cache)]
            for h in range(4):
                g = h // 2
                qd, kd, vd = (float(x[b, g]) for x in (w.q_descale, w.k_descale, w.v_descale))
                qs = [list(deq(w.q[b, t, h]) * qd) for t in range(2)]
                qvs = [list(deq(w.qv[b, t, h]) * qd) for t in range(2)]
                ks = [list(deq(r) * kd) for r in rows[0][:, g]]
                vs = [list(deq(r) * vd) for r in rows[1][:, g]]
                ob, lb = brute.rows(None if only else qs, ks, vs, w.scale,
                                    visible=lambda t, j, lk=int(lk): j <= t + lk - 2, qv=qvs)
                for t in range(2):
                    assert abs(lse[b, h, t] - lb[t]) <= 1e-12
                    np.testing.assert_allclose(o[b, t, h], ob[t], rtol=0, atol=1e-12)
    # unit descales: the real-valued oracle on the decoded codes
    dec = lambda x: ofp8.decode(x, "e4m3")
    o1, l1 = ofp8.attention_paged_fp8(w.q, w.k_cache, w.v_cache, "e4m3", None, None, None,
                                      w.block_table, w.cache_seqlens, w.page_size, w.scale, True,
                                      qv8=w.qv)
    o2, l2 = orc.attention_paged(dec(w.q), dec(w.k_cache), dec(w.v_cache), w.block_table,
                                 w.cache_seqlens, w.page_size, w.scale, True, qv=dec(w.qv))
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_fp8_qv():
    check_fp8_qv()


def test_fp8_varlen():
    check_fp8_varlen()


def test_fp8_decode_library():
    check_fp8_decode_library()


def test_fp8_decode_values():
    check_fp8_decode_values()


def test_fp8_attention_brute():
    check_fp8_attention_brute()


def test_fp8_descale_identities():
    check_fp8_descale_identities()


FP8_PINS = [check_fp8_decode_library, check_fp8_decode_values, check_fp8_attention_brute,
            check_fp8_descale_identities, check_fp8_varlen, check_fp8_qv]


def _fp8_mutants():
    base_decode = ofp8.decode
    base_attn = ofp8.attention_paged_fp8

    def decode_bias_off(bits, fmt):
        return base_decode(bits, fmt) * (2.0 if fmt == "e4m3" else 1.0)

    def decode_no_inf(bits, fmt):
        v = base_decode(bits, fmt)
        return np.where(np.isinf(v), np.nan, v)

    def q_descale_by_query_head(q8, k8, v8, fmt, q_descale, k_descale, v_descale, *rest, **kw):
        qd = None if q_descale is None else np.asarray(q_descale)[:, ::-1]
        return base_attn(q8, k8, v8, fmt, qd, k_descale, v_descale, *rest, **kw)

    def v_descale_on_k(q8, k8, v8, fmt, q_descale, k_descale, v_descale, *rest, **kw):
        return base_attn(q8, k8, v8, fmt, q_descale, v_descale, k_descale, *rest, **kw)

    base_varlen = ofp8.attention_varlen_fp8

    def varlen_q_descale_by_query_head(q8, k8, v8, fmt, q_descale, k_descale, v_descale,
                                       *rest, **kw):
        qd = None if q_descale is None else np.asarray(q_descale)[:, ::-1]
        return base_varlen(q8, k8, v8, fmt, qd, k_descale, v_descale, *rest, **kw)

    def qv_and_q_crossed(q8, k8, v8, fmt, q_descale, k_descale, v_descale, *rest, qv8=None,
                         only_qv=False, **kw):
        # q scored against V and qv against K
        if qv8 is None or only_qv:
            return base_attn(q8, k8, v8, fmt, q_descale, k_descale, v_descale, *rest, qv8=qv8,
                             only_qv=only_qv, **kw)
        return base_attn(qv8, k8, v8, fmt, q_descale, k_descale, v_descale, *rest, qv8=q8, **kw)

    return [("decode", decode_bias_off), ("decode", decode_no_inf),
            ("attention_paged_fp8", q_descale_by_query_head),
            ("attention_paged_fp8", v_descale_on_k),
            ("attention_varlen_fp8", varlen_q_descale_by_query_head),
            ("attention_paged_fp8", qv_and_q_crossed)]


@pytest.mark.parametrize("i", range(6))
def test_fp8_pins_catch_planted_mistakes(monkeypatch, i):
    name, fn = _fp8_mutants()[i]
    monkeypatch.setattr(ofp8, name, fn)
    caught = []
    for pin in FP8_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {fn.__name__} of {name} passed every pin"


def check_qv():
    """qv ([MATE] FMHA notes; reading: a second query scored against the V
    rows of the same KV head, added to q . k before the scale). Brute force
    with and without the QK path (only_qv), and identities: qv = 0 is plain
    decode; with V = K, only_qv is plain decode with q := qv and qv = a q
    scales the scores by (1 + a); q = 0 equals only_qv."""
    w = inputs.paged(65, [7, 13], sq=2, hq=4, hkv=2, d=4, page=4, causal=True, with_qv=True)
    f = lambda x: inputs.bits_to_f32(x).astype(np.float64)
    q, kc, vc, qv = f(w.q), f(w.k_cache), f(w.v_cache), f(w.qv)
    args = (w.block_table, w.cache_seqlens, w.page_size, w.scale, True)
    for only in (False, True):
        o, lse = orc.attention_paged(None if only else q, None if only else kc, vc, *args,
                                     qv=qv, only_qv=only)
        for b, lk in enumerate(w.cache_seqlens):
            ks = orc.gather_paged(kc, w.block_table, b, int(lk), w.page_size)
            vs = orc.gather_paged(vc, w.block_table, b, int(lk), w.page_size)
            for h in range(4):
                g = h // 2
                ob, lb = brute.rows(None if only else [list(r) for r in q[b, :, h]],
                                    [list(r) for r in ks[:, g]], [list(r) for r in vs[:, g]],
                                    w.scale, visible=lambda t, j, lk=int(lk): j <= t + lk - 2,
                                    qv=[list(r) for r in qv[b, :, h]])
                for t in range(2):
                    assert abs(lse[b, h, t] - lb[t]) <= 1e-12
                    np.testing.assert_allclose(o[b, t, h], ob[t], rtol=0, atol=1e-12)
    o0, l0 = orc.attention_paged(q, kc, vc, *args)
    o1, l1 = orc.attention_paged(q, kc, vc, *args, qv=np.zeros_like(qv))
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, atol=1e-13)
    o2, l2 = orc.attention_paged(None, None, kc, *args, qv=qv, only_qv=True)
    o3, l3 = orc.attention_paged(qv, kc, kc, *args)
    np.testing.assert_allclose(o2, o3, atol=1e-13)
    np.testing.assert_allclose(l2, l3, atol=1e-13)
    a = 0.75
    o4, l4 = orc.attention_paged(q, kc, kc, *args, qv=a * q)
    o5, l5 = orc.attention_paged(q, kc, kc, w.block_table, w.cache_seqlens, w.page_size,
                                 w.scale * (1 + a), True)
    np.testing.assert_allclose(o4, o5, atol=1e-12)
    np.testing.assert_allclose(l4, l5, atol=1e-12)
    o6, l6 = orc.attention_paged(np.zeros_like(q), kc, vc, *args, qv=qv)
    o7, l7 = orc.attention_paged(None, None, vc, *args, qv=qv, only_qv=True)
    np.testing.assert_allclose(o6, o7, atol=1e-13)
    np.testing.assert_allclose(l6, l7, atol=1e-13)


def test_qv():
    check_qv()


def check_qv_varlen():
    """qv on packed varlen sequences (bottom-right causal, Lq != Lk): brute
    force per sequence and head with and without the QK path; the FP8 form on
    torch-dequantized codes (qv with the Q descale)."""
    import torch
    w = inputs.varlen(66, [3, 6], [5, 6], hq=4, hkv=2, d=4, causal=True, with_qv=True)
    q, k, v, qv = (w.f32(n).astype(np.float64) for n in ("q", "k", "v", "qv"))
    cq, ck = w.cu_seqlens_q, w.cu_seqlens_k
    for only in (False, True):
        o, lse = orc.attention_varlen(None if only else q, None if only else k, v, cq, ck,
                                      w.scale, True, qv=qv, only_qv=only)
        for b in range(2):
            nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
            for h in range(4):
                g = h // 2
                ob, lb = brute.rows(None if only else [list(r) for r in q[cq[b]:cq[b + 1], h]],
                                    [list(r) for r in k[ck[b]:ck[b + 1], g]],
                                    [list(r) for r in v[ck[b]:ck[b + 1], g]], w.scale,
                                    visible=lambda t, j: j <= t + nk - nq,
                                    qv=[list(r) for r in qv[cq[b]:cq[b + 1], h]])
                for t in range(nq):
                    assert abs(lse[h, cq[b] + t] - lb[t]) <= 1e-12
                    np.testing.assert_allclose(o[cq[b] + t, h], ob[t], rtol=0, atol=1e-12)
    w8 = inputs.varlen_fp8(67, [3, 6], [5, 6], fmt="e5m2", hq=4, hkv=2, d=4, with_qv=True)
    deq = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e5m2).to(
        torch.float64).numpy()
    cq, ck = w8.cu_seqlens_q, w8.cu_seqlens_k
    for only in (False, True):
        o, lse = ofp8.attention_varlen_fp8(None if only else w8.q, None if only else w8.k,
                                           w8.v, "e5m2", w8.q_descale, w8.k_descale,
                                           w8.v_descale, cq, ck, w8.scale, True, qv8=w8.qv,
                                           only_qv=only)
        for b in range(2):
            nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
            for h in range(4):
                g = h // 2
                qd, kd, vd = (float(x[b, g]) for x in (w8.q_descale, w8.k_descale, w8.v_descale))
                ob, lb = brute.rows(
                    None if only else [list(deq(r) * qd) for r in w8.q[cq[b]:cq[b + 1], h]],
                    [list(deq(r) * kd) for r in w8.k[ck[b]:ck[b + 1], g]],
                    [list(deq(r) * vd) for r in w8.v[ck[b]:ck[b + 1], g]], w8.scale,
                    visible=lambda t, j: j <= t + nk - nq,
                    qv=[list(deq(r) * qd) for r in w8.qv[cq[b]:cq[b + 1], h]])
                for t in range(nq):
                    assert abs(lse[h, cq[b] + t] - lb[t]) <= 1e-12
                    np.testing.assert_allclose(o[cq[b] + t, h], ob[t], rtol=0, atol=1e-12)


def test_qv_varlen():
    check_qv_varlen()


def test_mate_mla_example_shape():
    """MATE minimal MLA example: q (1,32,8,576), k_cache (4,16,2,576),
    block_table zeros (1,4), cache_seqlens [32], head_dim_v 512. Every logical
    page maps to physical page 0, so keys 16..31 repeat keys 0..15: O equals
    attention over those 16 keys and LSE is larger by log 2."""
    rng = _rng(12)
    q = rng.standard_normal((1, 32, 8, 576))
    kc = rng.standard_normal((4, 16, 2, 576))
    table = np.zeros((1, 4), np.int32)
    scale = 1 / math.sqrt(576)
    o, lse = orc.mla_decode_paged(q, kc, table, [32], 16, scale)
    k16 = kc[0][None]                     # (1, 16, 2, 576)
    o16, l16 = orc.attention_dense(q, k16, k16[..., :512], scale)
    np.testing.assert_allclose(o, o16, atol=1e-13)
    np.testing.assert_allclose(lse, l16 + math.log(2), atol=1e-13)


def check_gather():
    rng = _rng(13)
    cache = rng.integers(0, 65535, size=(7, 4, 2, 3)).astype(np.uint16)
    table = np.array([[5, 0, 3, -1], [6, 1, 2, 4]], np.int32)
    rows = orc.gather_paged(cache, table, 1, 14, 4)
    for j in range(14):
        assert np.array_equal(rows[j], cache[table[1, j // 4], j % 4])


def test_gather():
    check_gather()


# ------------------------------------------------------------------------ MLA
def test_mla_equals_generic():
    p = inputs.paged(14, [20, 7], sq=2, hq=4, hkv=1, d=24, dv=16, page=8, shared_kv=True)
    q, kc = inputs.bits_to_f32(p.q), inputs.bits_to_f32(p.k_cache)
    o, lse = orc.mla_decode_paged(q, kc, p.block_table, p.cache_seqlens, 8, p.scale, dv=16)
    o2, l2 = orc.attention_paged(q, kc, np.ascontiguousarray(kc[..., :16]), p.block_table,
                                 p.cache_seqlens, 8, p.scale)
    np.testing.assert_allclose(o, o2, atol=0)
    np.testing.assert_allclose(lse, l2, atol=0)


# --------------------------------------------------------------------- sparse
def check_sparse():
    """Indices = whole causal prefix (shorter than topk) equals dense
    bottom-right causal; index order is irrelevant; -1 slots are ignored."""
    s = inputs.sparse_mla(15, batch=2, sq=5, sk=12, hq=4, d=24, dv=16, topk=16)
    q, kv = inputs.bits_to_f32(s.q), inputs.bits_to_f32(s.kv)
    o, lse = orc.mla_sparse(q, kv, s.indices, s.scale, 3, s.sinks, dv=16)
    od, ld = orc.attention_dense(q, kv, np.ascontiguousarray(kv[..., :16]), s.scale, True,
                                 sinks=s.sinks)
    np.testing.assert_allclose(o, od, atol=1e-13)
    np.testing.assert_allclose(lse, ld, atol=1e-13)
    rng = _rng(16)
    idx2 = s.indices.copy()
    for b in range(2):
        for t in range(5):
            idx2[b, t, 0] = rng.permutation(idx2[b, t, 0])
    o2, l2 = orc.mla_sparse(q, kv, idx2, s.scale, 3, s.sinks, dv=16)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    # mode 0 with indices beyond the causal limit: those keys now count
    idx3 = np.full_like(s.indices, -1)
    idx3[..., 0] = 11
    o3, _ = orc.mla_sparse(q, kv, idx3, s.scale, 0, None, dv=16)
    np.testing.assert_allclose(o3[:, :, :, :], np.broadcast_to(kv[:, 11:12, :, :16], o3.shape),
                               atol=0)
    o4, l4 = orc.mla_sparse(q, kv, idx3, s.scale, 3, None, dv=16)
    assert (o4[:, :4] == 0).all() and np.isneginf(l4[:, :, :4]).all()  # t < 4 cannot see key 11


def test_sparse():
    check_sparse()


def check_sparse_paged():
    """Block-sparse MLA over a paged cache [SFA PA_BSND, sparse_block_size]:
    selecting every block of the causal prefix equals dense bottom-right
    causal attention over the contiguous rows (blocks past the prefix hold
    keys the mask drops); one block index m selects exactly keys m*s ..
    m*s + s - 1; with block size 1 and the cache laid out contiguously it is
    the dense-layout sparse path."""
    lens, sq, d, dv, page, bs = [13, 9], 4, 24, 16, 4, 4
    w = inputs.sparse_paged(71, lens, sq, topk=8, block_size=bs, page=page, hq=4, d=d, dv=dv)
    q, kc = inputs.bits_to_f32(w.q), inputs.bits_to_f32(w.kv_cache)
    o, lse = orc.mla_sparse_paged(q, kc, w.block_table, w.seqlens_kv, page, w.indices, w.scale,
                                  3, w.sinks, bs, dv=dv)
    for b, lk in enumerate(lens):
        rows = orc.gather_paged(kc, w.block_table, b, lk, page)     # (lk, 1, d)
        od, ld = orc.attention_dense(q[b:b + 1], rows[None], np.ascontiguousarray(
            rows[None, ..., :dv]), w.scale, True, sinks=w.sinks)
        np.testing.assert_allclose(o[b], od[0], atol=1e-13)
        np.testing.assert_allclose(lse[b], ld[0], atol=1e-13)
    # a single block index m: keys m*bs .. m*bs+bs-1 (mode 0, block inside the sequence)
    idx1 = np.full_like(w.indices, -1)
    idx1[..., 0] = 1
    o1, l1 = orc.mla_sparse_paged(q, kc, w.block_table, w.seqlens_kv, page, idx1, w.scale, 0,
                                  None, bs, dv=dv)
    for b, lk in enumerate(lens):
        rows = orc.gather_paged(kc, w.block_table, b, lk, page)[bs:2 * bs, 0]
        for t in range(sq):
            ob, lb = orc.attend_rows(q[b, t], rows, rows[:, :dv], w.scale)
            np.testing.assert_allclose(o1[b, t], ob, atol=1e-13)
            np.testing.assert_allclose(l1[b, :, t], lb, atol=1e-13)
    # block size 1, pages in order: the dense-layout sparse path
    s = inputs.sparse_mla(72, batch=1, sq=5, sk=12, hq=4, d=d, dv=dv, topk=6)
    kv = inputs.bits_to_f32(s.kv)
    cache = kv[0].reshape(3, 4, 1, d)
    table = np.array([[0, 1, 2]], np.int32)
    qs = inputs.bits_to_f32(s.q)
    o2, l2 = orc.mla_sparse_paged(qs, cache, table, [12], 4, s.indices, s.scale, 3, s.sinks, 1,
                                  dv=dv)
    o3, l3 = orc.mla_sparse(qs, kv, s.indices, s.scale, 3, s.sinks, dv=dv)
    np.testing.assert_allclose(o2, o3, atol=0)
    np.testing.assert_allclose(l2, l3, atol=0)


def test_sparse_paged():
    check_sparse_paged()


# ----------------------------------------------------------- library routine
def test_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    d = inputs.varlen(17, [33], hq=4, hkv=4, d=16, causal=True, dtype="f32")
    q, k, v = (torch.from_numpy(d.f32(n).astype(np.float64)).permute(1, 0, 2)[None]
               for n in ("q", "k", "v"))
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal,
                                                               scale=d.scale)
        o, _ = orc.attention_varlen(d.f32("q"), d.f32("k"), d.f32("v"), d.cu_seqlens_q,
                                    d.cu_seqlens_k, d.scale, causal)
        np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


# ---------------------------------------------------------------- brute force
def check_brute_force():
    rng = _rng(18)
    for causal, window, sink in ((False, (-1, -1), False), (True, (-1, -1), True),
                                 (False, (2, 1), False), (True, (1, -1), True)):
        bsz, sq, sk, hq, hkv, dd, dv = 2, 5, 7, 4, 2, 3, 2
        q = rng.standard_normal((bsz, sq, hq, dd))
        k = rng.standard_normal((bsz, sk, hkv, dd))
        v = rng.standard_normal((bsz, sk, hkv, dv))
        sinks = rng.standard_normal(hq) if sink else None
        o, lse = orc.attention_dense(q, k, v, 0.9, causal, window, sinks)
        ob, lb = brute.dense(q, k, v, 0.9, causal, window, sinks)
        np.testing.assert_allclose(o, np.array(ob, dtype=float), atol=1e-12)
        np.testing.assert_allclose(lse, np.array(lb, dtype=float), atol=1e-12)


def test_brute_force():
    check_brute_force()


# -------------------------------------------------------------------- planner
def _check_plan(plan, lens, page, max_splits):
    bsz = len(lens)
    ptr, tri = orc.plan_unpack(plan, bsz)
    assert ptr[0] == 0 and ptr[-1] == plan[0] == len(tri)
    assert len(plan) == 3 + bsz + 4 * bsz * max_splits
    # work order: a permutation of the splits, lengths non-increasing, ties
    # in split order (identity above PLAN_SORT_MAX splits)
    order = orc.plan_order(plan, bsz, max_splits)
    assert sorted(order.tolist()) == list(range(len(tri)))
    if len(tri) <= orc.PLAN_SORT_MAX:
        ln = tri[order, 2] - tri[order, 1]
        assert (ln[:-1] >= ln[1:]).all()
        eq = ln[:-1] == ln[1:]
        assert (order[:-1][eq] < order[1:][eq]).all()
    else:
        assert (order == np.arange(len(tri))).all()
    for b, n in enumerate(lens):
        ns = ptr[b + 1] - ptr[b]
        assert 0 <= ns <= max_splits
        assert (ns == 0) == (n <= 0)
        seg = tri[ptr[b]:ptr[b + 1]]
        assert (seg[:, 0] == b).all()
        if ns:
            assert seg[0, 1] == 0 and seg[-1, 2] == n                       # cover
            assert (seg[1:, 1] == seg[:-1, 2]).all()                         # contiguous
            assert (seg[:, 2] > seg[:, 1]).all()                             # non-empty
            assert (seg[:, 1] % page == 0).all()                             # page aligned


def test_planner_properties():
    rng = _rng(19)
    for _ in range(200):
        bsz = int(rng.integers(1, 40))
        page = int(rng.choice([16, 64]))
        lens = rng.integers(0, 40000, size=bsz)
        ms = int(rng.integers(1, 17))
        plan = orc.plan_splits(lens, page, int(rng.integers(1, 9)), 256, int(rng.integers(1, 8)),
                               ms, int(rng.integers(1, 9)))
        _check_plan(plan, lens, page, ms)


def test_planner_rule_example():
    """Hand-worked instance of the rule: lens [1000, 64, 0], page 64,
    units_per_block 2, 4 CUs x 1 wave, max 3 splits, min 2 blocks:
    nblk = [16, 1, 0], total = 34, bps = max(2, ceil(34/4)) = 9,
    ns0 = min(3, ceil(16/9)) = 2, pps0 = 8 -> splits [0,512) [512,1000);
    ns1 = 1 -> [0,64); ns2 = 0."""
    plan = orc.plan_splits([1000, 64, 0], 64, 2, 4, 1, 3, 2)
    assert plan[:2 + 4 + 9].tolist() == [3, 9, 0, 2, 3, 3,
                                              0, 0, 512, 0, 512, 1000, 1, 0, 64]
    assert orc.plan_order(plan, 3, 3).tolist() == [0, 1, 2]   # lengths 512, 488, 64


def test_planner_order_example():
    """Hand-worked work order: lens [70, 1000], page 64, units_per_block 2,
    4 CUs x 1 wave, max 3 splits, min 2 blocks: nblk = [2, 16], total = 36,
    bps = 9; sequence 0: one split [0,70); sequence 1: ns = 2, pps = 8,
    splits [0,512) [512,1000). Split lengths 70, 512, 488 in plan order, so
    the longest-first order is 1, 2, 0; the order section starts after the
    3 * 2 * 3 triple words."""
    plan = orc.plan_splits([70, 1000], 64, 2, 4, 1, 3, 2)
    assert plan[:2 + 3 + 9].tolist() == [3, 9, 0, 1, 3, 0, 0, 70, 1, 0, 512, 1, 512, 1000]
    assert plan[3 + 2 + 18:3 + 2 + 18 + 3].tolist() == [1, 2, 0]
    assert (plan[3 + 2 + 18 + 3:] == 0).all() and len(plan) == 3 + 2 + 24


def test_planner_order_identity_above_limit():
    """More than PLAN_SORT_MAX splits: the work order is the plan order."""
    lens = [1000 + 64 * (i % 7) for i in range(300)]
    plan = orc.plan_splits(lens, 16, 1, 100000, 1, 16, 1)   # 14-16 splits per sequence
    assert int(plan[0]) > orc.PLAN_SORT_MAX
    _check_plan(plan, lens, 16, 16)


# --------------------------------------------------------------- mutation test
def _mutants():
    base_rows = orc.attend_rows
    base_vis = orc.visible_band
    base_combine = orc.combine
    base_gather = orc.gather_paged

    def no_scale(q, k, v, scale, visible=None, sink=None, bias=None):
        return base_rows(q, k, v, 1.0, visible, sink, bias)

    def sink_dropped(q, k, v, scale, visible=None, sink=None, bias=None):
        return base_rows(q, k, v, scale, visible, None, bias)

    def lse_without_max(q, k, v, scale, visible=None, sink=None, bias=None):
        o, lse = base_rows(q, k, v, scale, visible, sink, bias)
        qq, kk = np.asarray(q, float), np.asarray(k, float)
        if kk.shape[0] == 0:
            return o, lse
        s = scale * (qq @ kk.T)
        if visible is not None:
            s = np.where(visible, s, -np.inf)
        return o, lse - s.max(axis=1)

    def transposed_kv(q, k, v, scale, visible=None, sink=None, bias=None):
        k = np.asarray(k)
        v = np.asarray(v)
        return base_rows(q, k[::-1], v, scale, visible, sink, bias)

    def causal_top_left(lq, lk, causal, window_left=-1, window_right=-1, q_pos=None, k_pos=None):
        return base_vis(lk, lk, causal, window_left, window_right,
                        q_pos=np.arange(lq) if q_pos is None else q_pos, k_pos=k_pos)[:lq]

    def window_sides_swapped(lq, lk, causal, window_left=-1, window_right=-1, q_pos=None,
                             k_pos=None):
        return base_vis(lq, lk, causal, window_right, window_left, q_pos, k_pos)

    def combine_unweighted(o_partial, lse_partial, split_ptr, batch, seqlen_q, hq, max_splits,
                           sinks=None):
        return base_combine(o_partial, np.zeros_like(lse_partial), split_ptr, batch, seqlen_q, hq,
                            max_splits, sinks)

    def gather_swapped(cache, block_table, b, n, page_size):
        j = np.arange(n)
        return cache[np.asarray(block_table)[b, j % page_size % block_table.shape[1]],
                     j // page_size % cache.shape[1]]

    base_kvc = orc.attention_varlen_kvcache

    def kvcache_order_swapped(q, k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache,
                              block_table, cache_seqlens, page_size, scale, causal=False,
                              window=(-1, -1), sinks=None, seqs=None, mask=None):
        # current rows placed before the cached ones
        bsz = len(cu_seqlens_q) - 1
        ks, vs, cu = [], [], [0]
        for b in range(bsz):
            lc = int(cache_seqlens[b])
            kb = np.concatenate([k[cu_seqlens_k[b]:cu_seqlens_k[b + 1]],
                                 orc.gather_paged(k_cache, block_table, b, lc, page_size)])
            vb = np.concatenate([v[cu_seqlens_k[b]:cu_seqlens_k[b + 1]],
                                 orc.gather_paged(v_cache, block_table, b, lc, page_size)])
            ks.append(kb)
            vs.append(vb)
            cu.append(cu[-1] + len(kb))
        return orc.attention_varlen(q, np.concatenate(ks), np.concatenate(vs), cu_seqlens_q,
                                    np.asarray(cu), scale, causal, window, sinks, seqs, mask)

    del base_kvc

    def bias_scaled(q, k, v, scale, visible=None, sink=None, bias=None):
        # the mask added before the scale: scale * (q k + mask)
        if bias is not None:
            bias = np.asarray(bias, dtype=np.float64) * scale
        return base_rows(q, k, v, scale, visible, sink, bias)

    def block_keys_unscaled(indices_row, seqlen_q, seqlen_k, t, sparse_mode, block_size):
        idx = np.asarray(indices_row, dtype=np.int64)
        idx = idx[idx >= 0]
        keys = (idx[:, None] + np.arange(block_size)[None, :]).ravel()
        keep = keys < seqlen_k
        if sparse_mode == 3:
            keep &= keys <= t + (seqlen_k - seqlen_q)
        return keys[keep]

    base_paged = orc.attention_paged

    def paged_mask_shifted(*args, mask=None, **kw):
        # the decode mask read one key column late
        if mask is not None:
            mask = np.roll(np.asarray(mask, np.float64), -1, axis=3)
        return base_paged(*args, mask=mask, **kw)

    def qv_against_k(q, k_cache, v_cache, *rest, qv=None, only_qv=False, **kw):
        # qv scored against the key rows: q . k + qv . k = (q + qv) . k
        if qv is None:
            return base_paged(q, k_cache, v_cache, *rest, **kw)
        if only_qv:
            return base_paged(qv, k_cache if k_cache is not None else v_cache, v_cache, *rest,
                              **kw)
        return base_paged(q + qv, k_cache, v_cache, *rest, **kw)

    def qv_unscaled(q, k_cache, v_cache, block_table, cache_seqlens, page_size, scale, *rest,
                    qv=None, only_qv=False, **kw):
        # the softmax scale applied to q . k only
        if qv is not None:
            qv = np.asarray(qv, np.float64) / scale
        return base_paged(q, k_cache, v_cache, block_table, cache_seqlens, page_size, scale,
                          *rest, qv=qv, only_qv=only_qv, **kw)

    base_varlen = orc.attention_varlen

    def varlen_qv_against_k(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                            window=(-1, -1), sinks=None, seqs=None, mask=None, qv=None,
                            only_qv=False):
        if qv is None:
            return base_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal, window,
                               sinks, seqs, mask)
        # qv scored against the key rows: q . k + qv . k = (q + qv) . k
        if only_qv:
            return base_varlen(qv, v if k is None else k, v, cu_seqlens_q, cu_seqlens_k, scale,
                               causal, window, sinks, seqs, mask)
        return base_varlen(q + qv, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal, window,
                           sinks, seqs, mask)

    return [("attention_paged", paged_mask_shifted), ("attention_varlen", varlen_qv_against_k),
            ("attention_paged", qv_against_k), ("attention_paged", qv_unscaled),
            ("sparse_block_keys", block_keys_unscaled), ("attend_rows", bias_scaled),
            ("attend_rows", no_scale), ("attend_rows", sink_dropped),
            ("attend_rows", lse_without_max), ("attend_rows", transposed_kv),
            ("visible_band", causal_top_left), ("visible_band", window_sides_swapped),
            ("combine", combine_unweighted), ("gather_paged", gather_swapped),
            ("attention_varlen_kvcache", kvcache_order_swapped)]


PINS = [check_golden, check_rows_sum_to_one, check_lse_identity, check_identical_keys,
        check_single_key, check_sink, check_split_combine, check_gqa_equals_mha,
        check_varlen_equals_dense, check_paged_equals_contiguous, check_gather, check_sparse,
        check_brute_force, check_kvcache_brute_force, check_kvcache_special_cases,
        check_sparse_paged, check_additive_mask, check_qv, check_qv_varlen, check_paged_mask]


@pytest.mark.parametrize("i", range(15))
def test_pins_catch_planted_mistakes(monkeypatch, i):
    name, fn = _mutants()[i]
    monkeypatch.setattr(orc, name, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {fn.__name__} of {name} passed every pin"


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_kvcache_is_fp8_varlen_over_the_concatenation(fmt):
    # Cache-plus-current attention on FP8 codes is the FP8 varlen attention
    # over the keys [cached rows of b in page-table order ; current rows of b],
    # with the descales of sequence b on both parts. The concatenation is
    # written here by explicit page/slot indexing; distinct per-sequence
    # descales and a permuted page table catch a descale taken per page or a
    # swapped cache/current order.
    from attention_attn_fwd_02_amd import inputs as I
    from oracle import fp8 as F
    w = I.varlen_kvcache_fp8(77, [20, 45, 9], [20, 45, 0], [70, 0, 33], fmt, hq=4, hkv=2,
                             d=128, page=16, causal=True, with_sinks=True)
    kc, vc, cu = [], [], [0]
    for b in range(3):
        rows_k, rows_v = [], []
        for j in range(int(w.cache_seqlens[b])):
            pg = w.block_table[b, j // w.page_size]
            rows_k.append(w.k_cache[pg, j % w.page_size])
            rows_v.append(w.v_cache[pg, j % w.page_size])
        for j in range(w.cu_seqlens_k[b], w.cu_seqlens_k[b + 1]):
            rows_k.append(w.k[j])
            rows_v.append(w.v[j])
        kc += rows_k
        vc += rows_v
        cu.append(cu[-1] + len(rows_k))
    k8, v8 = np.stack(kc), np.stack(vc)
    o1, l1 = F.attention_varlen_kvcache_fp8(
        w.q, w.k, w.v, fmt, w.q_descale, w.k_descale, w.v_descale, w.cu_seqlens_q,
        w.cu_seqlens_k, w.k_cache, w.v_cache, w.block_table, w.cache_seqlens, w.page_size,
        w.scale, True, sinks=w.sinks)
    o2, l2 = F.attention_varlen_fp8(w.q, k8, v8, fmt, w.q_descale, w.k_descale, w.v_descale,
                                    w.cu_seqlens_q, np.asarray(cu), w.scale, True,
                                    sinks=w.sinks)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12, equal_nan=True)
    assert np.allclose(l1, l2, rtol=0, atol=1e-12, equal_nan=True)
    assert np.isfinite(l1[:, :w.cu_seqlens_q[2]]).all()
    assert len(np.unique(w.k_descale)) == w.k_descale.size
