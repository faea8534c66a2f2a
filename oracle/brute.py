"""Brute-force attention on tiny shapes, in pure Python with math.fsum.

TEST INFRASTRUCTURE ONLY (imported by tests alone). It is written separately
from oracle.attention on purpose: explicit loops over every (row, key, dim),
exactly summed dot products and denominators, and its own visibility rule, so
that an indexing or masking slip in the vectorised oracle shows up as a
disagreement. Formulas: CANN ops-transformer "flash_attn" page, attention,
sink and softmax_lse equations; bottom-right causal as in the MindSpore
"sparse_flash_attention" rightDownCausal mode.
"""
from __future__ import annotations

import math


def _dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def rows(q, k, v, scale, visible=None, sink=None, qv=None):
    """q: list of M rows, k/v: lists of N rows; visible(i, j) -> bool or None.
    qv: None or M rows of a second query whose dot product with v_j is added
    to q_i . k_j before the scale ([MATE] FMHA notes: optional qv input); q
    may then be None (the QK term is skipped, only_qv).
    Returns (o, lse) as Python lists."""
    out, lses = [], []
    dv = len(v[0]) if len(v) else 0
    m_rows = len(q) if q is not None else len(qv)
    for i in range(m_rows):
        s = []
        for j in range(len(v)):
            if visible is None or visible(i, j):
                terms = []
                if q is not None:
                    terms.append(_dot(q[i], k[j]))
                if qv is not None:
                    terms.append(_dot(qv[i], v[j]))
                s.append((scale * math.fsum(terms), j))
        if not s:
            out.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        mx = max(x for x, _ in s)
        den = math.fsum(math.exp(x - mx) for x, _ in s)
        lses.append(math.log(den) + mx)
        ref = mx if sink is None else max(mx, float(sink if not hasattr(sink, "__len__") else sink[i]))
        w = [(math.exp(x - ref), j) for x, j in s]
        tot = math.fsum(a for a, _ in w)
        if sink is not None:
            sg = float(sink if not hasattr(sink, "__len__") else sink[i])
            tot = math.fsum([tot, math.exp(sg - ref)])
        out.append([math.fsum(a * float(v[j][d]) for a, j in w) / tot for d in range(dv)])
    return out, lses


def dense(q, k, v, scale, causal=False, window=(-1, -1), sinks=None):
    """q [B][Sq][Hq][D], k [B][Sk][Hkv][D], v [B][Sk][Hkv][Dv] nested lists or
    arrays. Returns o [B][Sq][Hq][Dv] and lse [B][Hq][Sq] as nested lists."""
    bsz, sq, hq = len(q), len(q[0]), len(q[0][0])
    sk, hkv = len(k[0]), len(k[0][0])
    grp = hq // hkv
    wl, wr = window

    def vis(i, j):
        d = i + sk - sq
        if causal and j > d:
            return False
        if wl >= 0 and j < d - wl:
            return False
        if wr >= 0 and j > d + wr:
            return False
        return True

    o = [[[None] * hq for _ in range(sq)] for _ in range(bsz)]
    lse = [[[None] * sq for _ in range(hq)] for _ in range(bsz)]
    for b in range(bsz):
        for h in range(hq):
            kh = h // grp
            qs = [q[b][t][h] for t in range(sq)]
            ks = [k[b][j][kh] for j in range(sk)]
            vs = [v[b][j][kh] for j in range(sk)]
            ob, lb = rows(qs, ks, vs, scale, vis, None if sinks is None else sinks[h])
            for t in range(sq):
                o[b][t][h] = ob[t]
                lse[b][h][t] = lb[t]
    return o, lse
