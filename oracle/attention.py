"""Float64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path
(no kernels, headers, helpers or constants) and imports nothing from it.

Every function is the plain definition written out in float64 numpy: for each
query row, the visible key set is formed explicitly, the full score row is
materialised, and softmax, log-sum-exp and the weighted sum of values follow
the formulas on the pages. There is no tiling, no online rescaling and no
reordering beyond what numpy's matmul does inside one dot product.

Sources (the reference pages):
  [CANN] hiascend CANN ops-transformer "flash_attn" page: the attention formula
         (计算公式), the sink formulas, the softmax_lse formula and the output
         description of softmax_lse (shapes (B,Q_N,Q_S) and (Q_N,Q_T) for TND).
  [SFA]  MindSpore "mindspore.ops.sparse_flash_attention" page: the formula with
         selected keys K~/V~, the GQA grouping (N2, N1/N2), sparse_indices
         shape, sparse_mode 3 = rightDownCausal, the MLA-absorb concat of the
         nope and rope parts along D.
  [MATE] MATE "Attention" API page (FMHA and MLA sections): varlen, KV-cache
         with block_table and cache_seqlens, combine of partial outputs and LSE,
         the minimal dense MLA example.
  [LB]   MindSpore Lite "lite_boost.layers.flash_attention" page: causal and
         window_size=(-1,-1) arguments, softmax_scale default 1/sqrt(D).
  [MOJO] Modular "flash_attention_split_kv" page: attention of the current
         queries over the previous KV cache followed by the current K/V,
         passed separately instead of concatenated.

Readings where the pages are silent (each is listed in the design notes):
  * causal is bottom-right aligned: key j is visible to query t iff
    j <= t + (Lk - Lq)                                   (SFA rightDownCausal)
  * window (left, right) is an inclusive band around that diagonal, -1 means
    unbounded.
  * a row with no visible key gives O = 0 and LSE = -inf.
  * LSE excludes the sink (the softmax_lse formula uses max(S) only).
  * the sink is a logit in the scaled-score domain, one per query head.
  * query head h uses KV head h // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Row definition
# --------------------------------------------------------------------------
def attend_rows(q, k, v, scale, visible=None, sink=None, bias=None):
    """Attention of M query rows against N key rows.

    q (M, D), k (N, D), v (N, Dv): float arrays (widened to float64).
    visible (M, N) bool, True where key j may be seen by row i; None = all.
    sink: scalar or (M,) array of sink logits, or None.
    bias: (M, N) additive mask added to the scaled scores, or None; a -inf
    entry removes that key from the row              [MOJO input_mask_fn]

    S = scale * q k^T (+ bias)                         [CANN formula; SFA formula]
    m = max_j S, lse = log sum_j exp(S - m) + m        [CANN softmax_lse formula]
    no sink:   O = sum_j exp(S_j - m) v_j / sum_j exp(S_j - m)
    with sink: m' = max(sink, m),
               O = sum_j exp(S_j - m') v_j / (sum_j exp(S_j - m') + exp(sink - m'))
                                                       [CANN sink formulas]
    Rows with no visible key: O = 0, lse = -inf.
    Returns o (M, Dv) float64, lse (M,) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_rows, dv = q.shape[0], v.shape[1]
    o = np.zeros((m_rows, dv))
    lse = np.full(m_rows, NEG_INF)
    if m_rows == 0 or k.shape[0] == 0:
        return o, lse
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    if visible is not None:
        s = np.where(visible, s, NEG_INF)
    m = s.max(axis=1)
    live = np.isfinite(m)
    if not live.any():
        return o, lse
    s, m = s[live], m[live]
    e = np.exp(s - m[:, None])              # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    lse[live] = np.log(l) + m
    if sink is None:
        o[live] = (e @ v) / l[:, None]
    else:
        sk = np.broadcast_to(np.asarray(sink, dtype=np.float64), (m_rows,))[live]
        mp = np.maximum(sk, m)
        ep = np.exp(s - mp[:, None])
        o[live] = (ep @ v) / (ep.sum(axis=1) + np.exp(sk - mp))[:, None]
    return o, lse


def visible_band(lq, lk, causal, window_left=-1, window_right=-1, q_pos=None, k_pos=None):
    """Visibility of keys k_pos (default 0..lk-1) to queries q_pos (default
    0..lq-1) of one sequence, with bottom-right causal alignment: the diagonal
    of query t is key t + (lk - lq). window (left, right) bounds the band on
    each side of it, -1 = unbounded; causal is the same as right = 0."""
    t = np.arange(lq) if q_pos is None else np.asarray(q_pos)
    j = np.arange(lk) if k_pos is None else np.asarray(k_pos)
    diag = (t + (lk - lq))[:, None]
    vis = np.broadcast_to((j[None, :] >= 0) & (j[None, :] < lk), (len(t), len(j))).copy()
    if causal:
        vis &= j[None, :] <= diag
    if window_left >= 0:
        vis &= j[None, :] >= diag - window_left
    if window_right >= 0:
        vis &= j[None, :] <= diag + window_right
    return vis


def _group(hq, hkv):
    if hkv <= 0 or hq % hkv:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return hq // hkv


# --------------------------------------------------------------------------
# Packed variable-length attention (prefill)
# --------------------------------------------------------------------------
def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                     window=(-1, -1), sinks=None, seqs=None, mask=None, qv=None,
                     only_qv=False):
    """Packed varlen attention.                [MATE FMHA flash_attn_varlen_func]

    q (Tq, Hq, D), k (Tk, Hkv, D), v (Tk, Hkv, Dv); cu_seqlens_* (B+1) prefix
    sums with a leading 0. Sequence b owns query rows cu_q[b]:cu_q[b+1] and key
    rows cu_k[b]:cu_k[b+1]. Query head h reads KV head h // (Hq/Hkv)
    [SFA (N2, N1/N2) grouping]. sinks: (Hq,) or None. seqs: optional subset of
    sequences to evaluate (other rows are left NaN). mask: optional additive
    mask (Hm, Tq, L) with Hm = 1 (all heads) or Hq: query row r of sequence b
    adds mask[h or 0, r, j] to its scaled score with key j of the sequence
    [MOJO flash_attention_split_kv input_mask_fn].

    qv (Tq, Hq, Dv): a second query scored against the value rows, as in
    attention_paged: score scale * (q . k_j + qv . v_j), or scale * qv . v_j
    with only_qv (q and k may then be None) [MATE FMHA notes: optional qv].

    Returns O (Tq, Hq, Dv) float64 and LSE (Hq, Tq) float64 [CANN: TND LSE is
    (Q_N, Q_T)].
    """
    if only_qv and qv is None:
        raise ValueError("only_qv needs qv")
    tq, hq, _ = (qv if only_qv else q).shape
    hkv, dv = v.shape[1], v.shape[2]
    g = _group(hq, hkv)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    o = np.full((tq, hq, dv), np.nan)
    lse = np.full((hq, tq), np.nan)
    wl, wr = window
    for b in (range(len(cq) - 1) if seqs is None else seqs):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        lq, lk = int(q1 - q0), int(k1 - k0)
        vis = visible_band(lq, lk, causal, wl, wr)
        for h in range(hq):
            kh = h // g
            sink = None if sinks is None else float(sinks[h])
            bias = None if mask is None else mask[h if mask.shape[0] > 1 else 0, q0:q1, :lk]
            vj = v[k0:k1, kh]
            if qv is None:
                qh, kj = q[q0:q1, h], k[k0:k1, kh]
            elif only_qv:
                qh, kj = qv[q0:q1, h], vj
            else:
                qh = np.concatenate([q[q0:q1, h], qv[q0:q1, h]], axis=-1)
                kj = np.concatenate([k[k0:k1, kh], vj], axis=-1)
            ob, lb = attend_rows(qh, kj, vj, scale, vis, sink, bias)
            o[q0:q1, h] = ob
            lse[h, q0:q1] = lb
    return o, lse


def attention_dense(q, k, v, scale, causal=False, window=(-1, -1), sinks=None):
    """Batched dense attention, q (B,Sq,Hq,D), k (B,Sk,Hkv,D), v (B,Sk,Hkv,Dv).
    Returns O (B,Sq,Hq,Dv) and LSE (B,Hq,Sq) [CANN: LSE shape (B, Q_N, Q_S)]."""
    bsz, sq, hq, _ = q.shape
    sk = k.shape[1]
    cu_q = np.arange(bsz + 1) * sq
    cu_k = np.arange(bsz + 1) * sk
    o, lse = attention_varlen(q.reshape(bsz * sq, hq, -1), k.reshape(bsz * sk, k.shape[2], -1),
                              v.reshape(bsz * sk, v.shape[2], -1), cu_q, cu_k, scale, causal,
                              window, sinks)
    return (o.reshape(bsz, sq, hq, -1),
            lse.reshape(hq, bsz, sq).transpose(1, 0, 2))


# --------------------------------------------------------------------------
# Paged KV cache
# --------------------------------------------------------------------------
def gather_paged(cache, block_table, b, n, page_size):
    """Logical rows 0..n-1 of sequence b: row j lives in physical page
    block_table[b, j // page_size] at slot j % page_size.
    [MATE flash_attn_with_kvcache: k_cache (pages, page, Hkv, D) + block_table]"""
    j = np.arange(n)
    return cache[np.asarray(block_table)[b, j // page_size], j % page_size]


def attention_paged(q, k_cache, v_cache, block_table, cache_seqlens, page_size, scale,
                    causal=False, sinks=None, dv=None, batches=None, key_range=None, qv=None,
                    only_qv=False, mask=None):
    """Decode against a paged cache.         [MATE flash_attn_with_kvcache / MLA]

    q (B, Sq, Hq, D); k_cache (P, page, Hkv, D); v_cache (P, page, Hkv, Dv), or
    None when K and V share the cache, in which case the value of a key is the
    first dv entries of its row [CANN: shared-KV interface; SFA: nope || rope].
    Sequence b sees keys 0..cache_seqlens[b]-1 (the cache already holds the
    current tokens). Causal is bottom-right: query token t sees j <= t + L - Sq.

    qv (B, Sq, Hq, Dv): a second query scored against the value rows of the
    same KV head [MATE FMHA notes: optional qv input; only_qv skips the QK
    score path, q and k_cache may then be None]. The score of key j is
    scale * (q . k_j + qv . v_j), or scale * (qv . v_j) with only_qv; it is
    evaluated as one dot product of the concatenated rows [q | qv] and
    [k_j | v_j].

    key_range: optional (b -> (start, end)) restricting the keys to
    [start, end) of the full sequence (split mode); masks stay relative to the
    full length.

    mask: optional additive mask (B, Hm, Sq, L), Hm = 1 (all heads) or Hq, L
    at least every cache_seqlens[b]: query token t of sequence b and head h
    adds mask[b, h or 0, t, j] to its scaled score with key j
    [MOJO flash_attention_split_kv input_mask_fn: additive mask values];
    -inf removes the key. Returns O (B, Sq, Hq, Dv) and LSE (B, Hq, Sq).
    """
    if only_qv and qv is None:
        raise ValueError("only_qv needs qv")
    src = qv if only_qv else q
    bsz, sq, hq, _ = src.shape
    hkv = (v_cache if only_qv else k_cache).shape[2]
    g = _group(hq, hkv)
    if v_cache is None:
        dv = dv if dv is not None else k_cache.shape[3]
    else:
        dv = v_cache.shape[3]
    o = np.full((bsz, sq, hq, dv), np.nan)
    lse = np.full((bsz, hq, sq), np.nan)
    for b in (range(bsz) if batches is None else batches):
        lk = int(cache_seqlens[b])
        j0, j1 = (0, lk) if key_range is None else key_range(b)
        vr = None if v_cache is None else \
            gather_paged(v_cache, block_table, b, lk, page_size)[j0:j1]
        kr = None if only_qv else gather_paged(k_cache, block_table, b, lk, page_size)[j0:j1]
        if vr is None:
            vr = kr[..., :dv]
        vis = visible_band(sq, lk, causal, k_pos=np.arange(j0, j1))
        for h in range(hq):
            kh = h // g
            sink = None if sinks is None else float(sinks[h])
            if qv is None:
                qh, kj = q[b, :, h], kr[:, kh]
            elif only_qv:
                qh, kj = qv[b, :, h], vr[:, kh]
            else:
                qh = np.concatenate([q[b, :, h], qv[b, :, h]], axis=-1)
                kj = np.concatenate([kr[:, kh], vr[:, kh]], axis=-1)
            bias = None if mask is None else \
                np.asarray(mask[b, h if mask.shape[1] > 1 else 0, :, j0:j1], np.float64)
            ob, lb = attend_rows(qh, kj, vr[:, kh], scale, vis, sink, bias)
            o[b, :, h] = ob
            lse[b, h] = lb
    return o, lse


# --------------------------------------------------------------------------
# Split planner, split-KV partials and the LSE-weighted combine
# --------------------------------------------------------------------------
def attention_varlen_kvcache(q, k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache,
                             block_table, cache_seqlens, page_size, scale, causal=False,
                             window=(-1, -1), sinks=None, seqs=None, mask=None, qv=None,
                             only_qv=False):
    """Packed queries over a paged cache of earlier tokens plus the current
    K/V rows.                                   [MOJO flash_attention_split_kv]

    q (Tq, Hq, D); k, v (Tk, Hkv, D|Dv) hold the current tokens (sequence b
    owns rows cu_seqlens_k[b]:cu_seqlens_k[b+1]); k_cache / v_cache
    (P, page, Hkv, D|Dv) with block_table hold the cache_seqlens[b] earlier
    tokens [MATE flash_attn_with_kvcache paging]. The key sequence of b is the
    cache rows 0..Lc-1 followed by the current rows, Lk = Lc + Ln; masks are
    those of attention_varlen over that sequence (bottom-right causal); mask
    columns are key positions of that sequence (cache rows first).
    qv / only_qv: the second query scored against the value rows (cached and
    current), as in attention_varlen [MATE FMHA notes: optional qv]; with
    only_qv, k and k_cache are not read.
    Written as its definition: the concatenated K/V, then attention_varlen.
    Returns O (Tq, Hq, Dv) and LSE (Hq, Tq).
    """
    bsz = len(cu_seqlens_q) - 1
    ks, vs, cu = [], [], [0]
    for b in range(bsz):
        lc = int(cache_seqlens[b])
        vb = np.concatenate([gather_paged(v_cache, block_table, b, lc, page_size),
                             v[cu_seqlens_k[b]:cu_seqlens_k[b + 1]]])
        if only_qv:
            ks.append(vb)
            vs.append(vb)
            cu.append(cu[-1] + len(vb))
            continue
        kb = np.concatenate([gather_paged(k_cache, block_table, b, lc, page_size),
                             k[cu_seqlens_k[b]:cu_seqlens_k[b + 1]]])
        ks.append(kb)
        vs.append(vb)
        cu.append(cu[-1] + len(kb))
    return attention_varlen(q, np.concatenate(ks), np.concatenate(vs), cu_seqlens_q,
                            np.asarray(cu, np.int64), scale, causal, window, sinks, seqs, mask,
                            qv=qv, only_qv=only_qv)


# Plans of at most this many splits carry a longest-first work order; larger
# ones keep the splits in batch order.
PLAN_SORT_MAX = 4096


def plan_words(batch, max_splits):
    """int32 words of a plan buffer: header (2), split_ptr (B+1), up to
    B*max_splits (batch, kv_start, kv_end) triples, then B*max_splits words of
    work order."""
    return 3 + batch + 4 * batch * max_splits


def _cdiv(a, b):
    return -(-a // b)


def plan_splits(cache_seqlens, page_size, units_per_block, num_cu, waves, max_splits,
                min_blocks):
    """Split plan for split-KV decode.

    The pages name a metadata step that precomputes the work split before the
    main call [MATE get_scheduler_metadata / get_mla_metadata; CANN
    flash_attn_metadata] but give no rule, so the rule is ours, integer only:
      nblk_b = ceil(len_b / page)                 (0 when len_b <= 0)
      total  = sum_b nblk_b * units_per_block
      bps    = max(min_blocks, ceil(total / (num_cu * waves)))
      ns_b   = min(max_splits, max(1, ceil(nblk_b / bps)))
      pps_b  = ceil(nblk_b / ns_b);  ns_b = ceil(nblk_b / pps_b)
      split s of b covers tokens [s*pps_b*page, min((s+1)*pps_b*page, len_b))
    Empty sequences get no split.
    Work order (the order in which decode workgroups take the splits): by
    length kv_end - kv_start, longest first, ties in split order (the
    longest-processing-time rule of list scheduling); the identity when
    there are more than PLAN_SORT_MAX splits.

    Returns the int32 plan: [total_splits, bps, split_ptr[0..B],
    (batch, kv_start, kv_end) per split in batch order, padded to
    B*max_splits triples, then the work order (split indices) padded to
    B*max_splits words]; the buffer is plan_words(B, max_splits) long and
    padding words are 0.
    """
    lens = [max(0, int(x)) for x in cache_seqlens]
    bsz = len(lens)
    nblk = [_cdiv(n, page_size) for n in lens]
    total = sum(nblk) * units_per_block
    bps = max(min_blocks, _cdiv(total, num_cu * waves))
    triples, ptr = [], [0]
    for b, nb in enumerate(nblk):
        if nb == 0:
            ns = 0
        else:
            ns = min(max_splits, max(1, _cdiv(nb, bps)))
            pps = _cdiv(nb, ns)
            ns = _cdiv(nb, pps)
            for s in range(ns):
                triples.append((b, s * pps * page_size, min((s + 1) * pps * page_size, lens[b])))
        ptr.append(ptr[-1] + ns)
    plan = np.zeros(plan_words(bsz, max_splits), dtype=np.int32)
    plan[0] = len(triples)
    plan[1] = bps
    plan[2:3 + bsz] = ptr
    if triples:
        plan[3 + bsz:3 + bsz + 3 * len(triples)] = np.asarray(triples, dtype=np.int32).ravel()
    n = len(triples)
    if n <= PLAN_SORT_MAX:
        order = sorted(range(n), key=lambda i: (-(triples[i][2] - triples[i][1]), i))
    else:
        order = list(range(n))
    base = 3 + bsz + 3 * bsz * max_splits
    plan[base:base + n] = order
    return plan


def plan_order(plan, batch, max_splits):
    """The work order (split indices, length total_splits) of a plan buffer."""
    base = 3 + batch + 3 * batch * max_splits
    return np.asarray(plan[base:base + int(plan[0])])


def plan_unpack(plan, batch):
    """(split_ptr (B+1), triples (total, 3)) from a plan buffer."""
    plan = np.asarray(plan)
    total = int(plan[0])
    ptr = plan[2:3 + batch].astype(np.int64)
    tri = plan[3 + batch:3 + batch + 3 * total].reshape(total, 3).astype(np.int64)
    return ptr, tri


def attention_paged_split(q, k_cache, v_cache, block_table, cache_seqlens, page_size, scale,
                          plan, max_splits, causal=False, dv=None, mask=None):
    """Per-split partial results [MATE: partial outputs and LSE buffers].

    Split s of sequence b is plain attention restricted to its key range; its
    output is normalised within the split. Returns o_partial
    (B*max_splits, Sq*Hq, Dv) and lse_partial (B*max_splits, Sq*Hq), slot
    b*max_splits + s, row t*Hq + h. Unused slots are NaN. mask: as in
    attention_paged (columns are key positions of the whole sequence).
    """
    bsz, sq, hq, _ = q.shape
    ptr, tri = plan_unpack(plan, bsz)
    dv = (dv if dv is not None else k_cache.shape[3]) if v_cache is None else v_cache.shape[3]
    op = np.full((bsz * max_splits, sq * hq, dv), np.nan)
    lp = np.full((bsz * max_splits, sq * hq), np.nan)
    for b in range(bsz):
        for s in range(int(ptr[b + 1] - ptr[b])):
            tb, j0, j1 = tri[ptr[b] + s]
            assert tb == b
            o, lse = attention_paged(q, k_cache, v_cache, block_table, cache_seqlens, page_size,
                                     scale, causal, None, dv, batches=[b],
                                     key_range=lambda _b, a=int(j0), e=int(j1): (a, e),
                                     mask=mask)
            op[b * max_splits + s] = o[b].reshape(sq * hq, dv)
            lp[b * max_splits + s] = lse[b].transpose(1, 0).reshape(sq * hq)
    return op, lp


def combine(o_partial, lse_partial, split_ptr, batch, seqlen_q, hq, max_splits, sinks=None):
    """LSE-weighted merge of per-split results [MATE flash_attn_combine;
    CANN softmax_lse definition].

    For one output row with split results (O_s, LSE_s):
      M = max_s LSE_s;  w_s = exp(LSE_s - M);  LSE = M + log sum_s w_s
      O = sum_s w_s O_s / sum_s w_s
    With a sink sigma of the row's head: M* = max(M, sigma),
      O = sum_s exp(LSE_s - M*) O_s / (sum_s exp(LSE_s - M*) + exp(sigma - M*)),
    and LSE stays sink-free. No split, or all LSE_s = -inf: O = 0, LSE = -inf.
    Returns O (B, Sq, Hq, Dv) and LSE (B, Hq, Sq).
    """
    dv = o_partial.shape[2]
    o = np.zeros((batch, seqlen_q, hq, dv))
    lse = np.full((batch, hq, seqlen_q), NEG_INF)
    ptr = np.asarray(split_ptr, dtype=np.int64)
    for b in range(batch):
        ns = int(ptr[b + 1] - ptr[b])
        if ns == 0:
            continue
        slots = b * max_splits + np.arange(ns)
        for t in range(seqlen_q):
            for h in range(hq):
                r = t * hq + h
                ls = np.asarray(lse_partial[slots, r], dtype=np.float64)
                os_ = np.asarray(o_partial[slots, r], dtype=np.float64)
                mx = ls.max()
                if not np.isfinite(mx):
                    continue
                w = np.exp(ls - mx)
                lse[b, h, t] = mx + np.log(w.sum())
                if sinks is None:
                    o[b, t, h] = (w @ os_) / w.sum()
                else:
                    sg = float(sinks[h])
                    ms = max(mx, sg)
                    ws = np.exp(ls - ms)
                    o[b, t, h] = (ws @ os_) / (ws.sum() + np.exp(sg - ms))
    return o, lse


# --------------------------------------------------------------------------
# MLA (absorbed) decode and top-k sparse MLA
# --------------------------------------------------------------------------
def mla_decode_paged(q, kv_cache, block_table, cache_seqlens, page_size, scale, causal=False,
                     dv=512, batches=None):
    """MLA-absorbed decode [MATE flash_mla_with_kvcache example: q (B,Sq,Hq,576),
    k_cache (P,page,Hkv,576), head_dim_v=512]: one cached row per token holds
    the 512-wide latent followed by the 64-wide rope part [SFA MLA-absorb
    concat]; the key is the whole row and the value is its first dv entries.
    Returns O (B, Sq, Hq, dv), LSE (B, Hq, Sq)."""
    return attention_paged(q, kv_cache, None, block_table, cache_seqlens, page_size, scale,
                           causal, None, dv, batches)


def sparse_key_set(indices_row, seqlen_q, seqlen_k, t, sparse_mode):
    """Keys selected for query token t [SFA sparse_indices; sparse_mode 0 = all,
    3 = rightDownCausal]: entries outside [0, Sk) (including the -1 padding)
    are skipped, mode 3 also skips keys after t + (Sk - Sq); duplicates count
    as often as they appear and the order does not matter."""
    idx = np.asarray(indices_row, dtype=np.int64)
    keep = (idx >= 0) & (idx < seqlen_k)
    if sparse_mode == 3:
        keep &= idx <= t + (seqlen_k - seqlen_q)
    return idx[keep]


def sparse_block_keys(indices_row, seqlen_q, seqlen_k, t, sparse_mode, block_size):
    """Keys selected for query token t when each index names a block of
    block_size consecutive keys [SFA sparse_indices with sparse_block_size,
    PA_BSND]: index i >= 0 selects keys i*block_size .. i*block_size +
    block_size - 1; keys at or past seqlen_k, and in mode 3 after
    t + (seqlen_k - seqlen_q), are dropped; duplicates count each time."""
    idx = np.asarray(indices_row, dtype=np.int64)
    idx = idx[idx >= 0]
    keys = (idx[:, None] * block_size + np.arange(block_size)[None, :]).ravel()
    keep = keys < seqlen_k
    if sparse_mode == 3:
        keep &= keys <= t + (seqlen_k - seqlen_q)
    return keys[keep]


def mla_sparse_paged(q, kv_cache, block_table, seqlens_kv, page_size, sparse_indices, scale,
                     sparse_mode=3, sinks=None, sparse_block_size=1, dv=512, tokens=None):
    """Sparse MLA over a paged latent cache [SFA layout_kv PA_BSND: key
    (block_num, block_size, 1, D) with block_table, actual_seq_lengths_kv;
    sparse_block_size]. Sequence b has seqlens_kv[b] keys, key j at page
    block_table[b, j // page_size], slot j % page_size; its selected keys are
    sparse_block_keys(...); the rest as mla_sparse.
    Returns O (B, Sq, Hq, dv), LSE (B, Hq, Sq), or per listed (b, t) token."""
    bsz, sq, hq, _ = q.shape
    if tokens is None:
        o = np.zeros((bsz, sq, hq, dv))
        lse = np.zeros((bsz, hq, sq))
        todo = [(b, t) for b in range(bsz) for t in range(sq)]
    else:
        o = np.zeros((len(tokens), hq, dv))
        lse = np.zeros((len(tokens), hq))
        todo = tokens
    for i, (b, t) in enumerate(todo):
        lk = int(seqlens_kv[b])
        keys = sparse_block_keys(sparse_indices[b, t, 0], sq, lk, t, sparse_mode,
                                 sparse_block_size)
        rows = gather_paged(kv_cache, block_table, b, lk, page_size)[keys, 0]
        ob, lb = attend_rows(q[b, t], rows, rows[:, :dv], scale, None, sinks)
        if tokens is None:
            o[b, t] = ob
            lse[b, :, t] = lb
        else:
            o[i] = ob
            lse[i] = lb
    return o, lse


def mla_sparse(q, kv, sparse_indices, scale, sparse_mode=3, sinks=None, dv=512, tokens=None):
    """Top-k sparse MLA with optional per-head sinks [SFA formula with the
    selected K~ = V~ rows; CANN sink formulas].

    q (B, Sq, Hq, D), kv (B, Sk, 1, D), sparse_indices (B, Sq, 1, topk) int32.
    All query heads of a token share its index list (N2 = 1).
    Returns O (B, Sq, Hq, dv), LSE (B, Hq, Sq); when tokens (a list of (b, t))
    is given, only those are evaluated and O (n, Hq, dv), LSE (n, Hq) are
    returned in the order of the list.
    """
    bsz, sq, hq, _ = q.shape
    sk = kv.shape[1]
    if tokens is None:
        o = np.zeros((bsz, sq, hq, dv))
        lse = np.zeros((bsz, hq, sq))
        todo = [(b, t) for b in range(bsz) for t in range(sq)]
    else:
        o = np.zeros((len(tokens), hq, dv))
        lse = np.zeros((len(tokens), hq))
        todo = tokens
    for i, (b, t) in enumerate(todo):
        keys = sparse_key_set(sparse_indices[b, t, 0], sq, sk, t, sparse_mode)
        rows = kv[b, keys, 0]
        ob, lb = attend_rows(q[b, t], rows, rows[:, :dv], scale, None, sinks)
        if tokens is None:
            o[b, t] = ob
            lse[b, :, t] = lb
        else:
            o[i] = ob
            lse[i] = lb
    return o, lse
