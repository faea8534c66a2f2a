"""FP8 inputs for the float64 oracle: the two 8-bit float formats and
attention over descaled FP8 Q / K / V.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares nothing with the HIP path.

Source: [MATE] "Attention" API page, FMHA forward dtype notes. The varlen and
KV-cache forward paths take float8_e4m3fn and float8_e5m2 inputs; optional
float32 q_descale, k_descale and v_descale tensors of shape
(batch_size, num_heads_kv) scale them; FP8 inputs give bfloat16 outputs. The
real value of an element is its FP8 value times the descale of its (batch,
KV head); for Q that is the KV head its query head reads (the grouping
(N2, N1/N2) of the MindSpore sparse_flash_attention page), which is the plain
reading of a query descale indexed by num_heads_kv.

The formats themselves are the OCP 8-bit floating-point formats the dtype
names refer to (sign, exponent, mantissa bits; value
(-1)^s 2^(e-bias) (1 + m/2^M) for e > 0 and (-1)^s 2^(1-bias) m/2^M for e = 0):
  e4m3fn: 4 exponent bits (bias 7), 3 mantissa bits, no infinities, S.1111.111
          is NaN, largest finite 448;
  e5m2:   5 exponent bits (bias 15), 2 mantissa bits, exponent 31 is infinity
          (mantissa 0) or NaN, largest finite 57344.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import _group, attend_rows, attention_varlen, gather_paged, visible_band

FORMATS = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}   # exponent bits, mantissa bits, bias


def decode(bits, fmt):
    """float64 values of uint8 FP8 codes, from the bit-field definition."""
    ebits, mbits, bias = FORMATS[fmt]
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> mbits) & ((1 << ebits) - 1)
    m = b & ((1 << mbits) - 1)
    normal = sign * np.ldexp(1.0 + m / float(1 << mbits), (e - bias).astype(np.int64))
    sub = sign * np.ldexp(m / float(1 << mbits), 1 - bias)
    val = np.where(e == 0, sub, normal)
    top = (1 << ebits) - 1
    if fmt == "e4m3":
        val = np.where((e == top) & (m == (1 << mbits) - 1), np.nan, val)
    else:
        val = np.where((e == top) & (m == 0), sign * np.inf, val)
        val = np.where((e == top) & (m != 0), np.nan, val)
    return val


def attention_paged_fp8(q8, k8, v8, fmt, q_descale, k_descale, v_descale, block_table,
                        cache_seqlens, page_size, scale, causal=False, sinks=None,
                        batches=None, qv8=None, only_qv=False):
    """Decode against a paged FP8 cache.          [MATE FMHA FP8 dtype notes]

    q8 (B, Sq, Hq, D), k8 (P, page, Hkv, D), v8 (P, page, Hkv, Dv) uint8 codes
    of format fmt ("e4m3" or "e5m2"); descales float (B, Hkv) or None (= 1).
    The real inputs are decode(x8) * descale[b, kv head]; the attention is
    then the paged decode of the plain definition (sequence b sees keys
    0..cache_seqlens[b]-1, bottom-right causal). Returns O (B, Sq, Hq, Dv)
    and LSE (B, Hq, Sq).

    qv8 (B, Sq, Hq, Dv): FP8 codes of the second query; its real value uses
    q_descale as q does (the notes: q_descale applies to both query tensors).
    The score is scale * (q . k_j + qv . v_j) on the real values, or
    scale * (qv . v_j) with only_qv (q8 and k8 may then be None).
    """
    if only_qv and qv8 is None:
        raise ValueError("only_qv needs qv8")
    bsz, sq, hq, _ = (qv8 if only_qv else q8).shape
    hkv = v8.shape[2]
    g = _group(hq, hkv)
    dv = v8.shape[3]
    one = np.ones((bsz, hkv))
    qd = one if q_descale is None else np.asarray(q_descale, np.float64)
    kd = one if k_descale is None else np.asarray(k_descale, np.float64)
    vd = one if v_descale is None else np.asarray(v_descale, np.float64)
    o = np.full((bsz, sq, hq, dv), np.nan)
    lse = np.full((bsz, hq, sq), np.nan)
    for b in (range(bsz) if batches is None else batches):
        lk = int(cache_seqlens[b])
        kr = None if only_qv else decode(gather_paged(k8, block_table, b, lk, page_size), fmt)
        vr = decode(gather_paged(v8, block_table, b, lk, page_size), fmt)
        vis = visible_band(sq, lk, causal)
        for h in range(hq):
            kh = h // g
            vh = vr[:, kh] * vd[b, kh]
            if only_qv:
                qh, kj = decode(qv8[b, :, h], fmt) * qd[b, kh], vh
            else:
                qh, kj = decode(q8[b, :, h], fmt) * qd[b, kh], kr[:, kh] * kd[b, kh]
                if qv8 is not None:
                    qh = np.concatenate([qh, decode(qv8[b, :, h], fmt) * qd[b, kh]], axis=-1)
                    kj = np.concatenate([kj, vh], axis=-1)
            sink = None if sinks is None else float(sinks[h])
            ob, lb = attend_rows(qh, kj, vh, scale, vis, sink)
            o[b, :, h] = ob
            lse[b, h] = lb
    return o, lse


def attention_varlen_fp8(q8, k8, v8, fmt, q_descale, k_descale, v_descale, cu_seqlens_q,
                         cu_seqlens_k, scale, causal=False, window=(-1, -1), sinks=None,
                         seqs=None, qv8=None, only_qv=False):
    """Packed varlen attention on FP8 codes.  [MATE FMHA FP8 dtype notes;
    flash_attn_varlen_func]

    q8 (Tq, Hq, D), k8 (Tk, Hkv, D), v8 (Tk, Hkv, Dv) uint8 codes of fmt;
    descales float (B, Hkv) or None (= 1). The rows of sequence b are
    decode(x8) * descale[b, kv head] (query head h: its KV head h // (Hq/Hkv));
    then attention_varlen. qv8 (Tq, Hq, Dv): codes of the second query, with
    the Q descales (only_qv: q8 and k8 may be None). Returns O (Tq, Hq, Dv),
    LSE (Hq, Tq)."""
    if only_qv and qv8 is None:
        raise ValueError("only_qv needs qv8")
    tq, hq, _ = (qv8 if only_qv else q8).shape
    hkv = v8.shape[1]
    g = _group(hq, hkv)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    bsz = len(cq) - 1
    one = np.ones((bsz, hkv))
    qd = one if q_descale is None else np.asarray(q_descale, np.float64)
    kd = one if k_descale is None else np.asarray(k_descale, np.float64)
    vd = one if v_descale is None else np.asarray(v_descale, np.float64)
    q = None if only_qv else decode(q8, fmt)
    k = None if only_qv else decode(k8, fmt)
    v = decode(v8, fmt)
    qv = None if qv8 is None else decode(qv8, fmt)
    for b in range(bsz):
        qrow = np.repeat(qd[b], g)[None, :, None]
        if not only_qv:
            q[cq[b]:cq[b + 1]] *= qrow
            k[ck[b]:ck[b + 1]] *= kd[b][None, :, None]
        if qv is not None:
            qv[cq[b]:cq[b + 1]] *= qrow
        v[ck[b]:ck[b + 1]] *= vd[b][None, :, None]
    return attention_varlen(q, k, v, cq, ck, scale, causal, window, sinks, seqs, qv=qv,
                            only_qv=only_qv)


def attention_varlen_kvcache_fp8(q8, k8, v8, fmt, q_descale, k_descale, v_descale,
                                 cu_seqlens_q, cu_seqlens_k, k8_cache, v8_cache, block_table,
                                 cache_seqlens, page_size, scale, causal=False, window=(-1, -1),
                                 sinks=None, seqs=None):
    """Queries over a paged FP8 cache of earlier tokens plus the current FP8
    K/V rows.           [MATE FMHA FP8 dtype notes; MOJO flash_attention_split_kv]

    q8 (Tq, Hq, D), k8 / v8 (Tk, Hkv, D) current rows and k8_cache / v8_cache
    (P, page, Hkv, D) uint8 codes of fmt; descales float (B, Hkv) or None (= 1).
    The keys of sequence b are its cache_seqlens[b] cached rows (through
    block_table) followed by its current rows; each of them, cached or
    current, is decode(code) * descale[b, kv head] (the descale belongs to the
    sequence, not to the page). Then attention_varlen over those keys.
    Returns O (Tq, Hq, Dv), LSE (Hq, Tq)."""
    tq, hq, _ = q8.shape
    hkv = v8_cache.shape[2]
    g = _group(hq, hkv)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    bsz = len(cq) - 1
    one = np.ones((bsz, hkv))
    qd = one if q_descale is None else np.asarray(q_descale, np.float64)
    kd = one if k_descale is None else np.asarray(k_descale, np.float64)
    vd = one if v_descale is None else np.asarray(v_descale, np.float64)
    q = decode(q8, fmt)
    ks, vs, cu = [], [], [0]
    for b in range(bsz):
        q[cq[b]:cq[b + 1]] *= np.repeat(qd[b], g)[None, :, None]
        lc = int(cache_seqlens[b])
        kb = np.concatenate([decode(gather_paged(k8_cache, block_table, b, lc, page_size), fmt),
                             decode(k8[ck[b]:ck[b + 1]], fmt)])
        vb = np.concatenate([decode(gather_paged(v8_cache, block_table, b, lc, page_size), fmt),
                             decode(v8[ck[b]:ck[b + 1]], fmt)])
        ks.append(kb * kd[b][None, :, None])
        vs.append(vb * vd[b][None, :, None])
        cu.append(cu[-1] + len(kb))
    return attention_varlen(q, np.concatenate(ks), np.concatenate(vs), cq,
                            np.asarray(cu, np.int64), scale, causal, window, sinks, seqs)
