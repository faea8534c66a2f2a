"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the float64 oracle and the HIP path are fed from it,
and it imports neither of them (numpy only, so it also runs where torch is
absent).

Values that the GPU reads as bfloat16 are drawn as float32 N(0,1) and rounded to
bfloat16 with round-to-nearest-even. They are returned twice: as the raw uint16
bit patterns (what the device tensor holds) and, on request, as float32 arrays
holding exactly the same values (bf16 -> fp32 is exact), which the oracle widens
to float64.

Draw order inside one workload is fixed: lengths, then Q, then K, then V (or the
shared cache), then the page permutation, then sparse indices, then sinks.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np

# One seed per workload of the benchmark set.
SEED_TINY_DENSE = 1001
SEED_VARLEN_PREFILL = 1002
SEED_PAGED_DECODE = 1003
SEED_MLA_DECODE = 1004
SEED_SPARSE_MLA = 1005
SEED_CHUNKED_PREFILL = 1006
SEED_PAGED_DECODE_FP8 = 1007
SEED_SPARSE_PAGED = 1008
SEED_VARLEN_PREFILL_FP8 = 1009
SEED_PAGED_DECODE_QV = 1010
SEED_VARLEN_PREFILL_QV = 1011
SEED_CHUNKED_PREFILL_FP8 = 1012

_CHUNK = 1 << 22  # elements per independently seeded block of a large tensor


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the
    16-bit patterns as uint16. Inputs here are finite normals, so NaN/Inf
    handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bfloat16, returned as uint16 bits.

    One 63-bit key is taken from the workload's generator (so the fixed draw
    order of the workload is kept); the tensor is then filled in C order in
    blocks of _CHUNK elements, block i drawn from its own PCG64 stream seeded
    with SeedSequence([key, i]). Blocks are independent, so they are filled by
    a thread pool and the values do not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    key = int(rng.integers(0, 2**63 - 1))

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, i])))
        u = g.standard_normal(e - s, dtype=np.float32).view(np.uint32)
        u += np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))
        out[s:e] = u >> 16

    nblk = (n + _CHUNK - 1) // _CHUNK
    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _paged_table(rng: np.random.Generator, lens: np.ndarray, page: int):
    """Block table for sequences of the given lengths: one pool holding exactly
    the pages needed, handed out as consecutive chunks of a random permutation.
    Entries past a sequence's last page are -1."""
    nblk = (lens + page - 1) // page
    pool = int(nblk.sum())
    perm = rng.permutation(pool).astype(np.int32)
    width = max(1, int(nblk.max()))
    table = np.full((len(lens), width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, pool


@dataclasses.dataclass
class Dense:
    """Packed variable-length problem: q (Tq,Hq,D), k (Tk,Hkv,D), v (Tk,Hkv,Dv).
    For bfloat16 workloads the arrays hold uint16 bits; for float32 workloads
    they hold float32 values."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    dtype: str  # "bf16" or "f32"
    scale: float
    causal: bool
    window: tuple
    sinks: np.ndarray | None = None
    qv: np.ndarray | None = None     # (Tq,Hq,Dv) second query, same element type, or None

    @property
    def batch(self):
        return len(self.cu_seqlens_q) - 1

    def f32(self, name):
        a = getattr(self, name)
        return bits_to_f32(a) if self.dtype == "bf16" else a


def tiny_dense(seed: int = SEED_TINY_DENSE, s: int = 128, h: int = 4, d: int = 64) -> Dense:
    """B=1, Sq=Sk=s, Hq=Hkv=h, head dim d, float32 N(0,1), non-causal,
    scale 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((s, h, d), dtype=np.float32)
    k = rng.standard_normal((s, h, d), dtype=np.float32)
    v = rng.standard_normal((s, h, d), dtype=np.float32)
    cu = np.array([0, s], dtype=np.int32)
    return Dense(q, k, v, cu, cu.copy(), "f32", 1.0 / np.sqrt(d), False, (-1, -1))


def varlen(seed: int, lens_q, lens_k=None, hq: int = 32, hkv: int = 8, d: int = 128,
           dv: int | None = None, dtype: str = "bf16", causal: bool = True,
           window=(-1, -1), scale: float | None = None, with_sinks: bool = False,
           with_qv: bool = False) -> Dense:
    """Packed varlen problem with explicit per-sequence lengths (qv, when
    asked for, drawn last)."""
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = lens_q if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    w = _varlen_draw(rng, lens_q, lens_k, hq, hkv, d, dv or d, dtype, causal,
                     window, scale, with_sinks)
    if with_qv:
        shape = (int(lens_q.sum()), hq, dv or d)
        w.qv = _normal_bf16(rng, shape) if dtype == "bf16" else \
            rng.standard_normal(shape, dtype=np.float32)
    return w


def _varlen_draw(rng, lens_q, lens_k, hq, hkv, d, dv, dtype, causal, window, scale,
                 with_sinks):
    tq, tk = int(lens_q.sum()), int(lens_k.sum())
    if dtype == "bf16":
        q = _normal_bf16(rng, (tq, hq, d))
        k = _normal_bf16(rng, (tk, hkv, d))
        v = _normal_bf16(rng, (tk, hkv, dv))
    else:
        q = rng.standard_normal((tq, hq, d), dtype=np.float32)
        k = rng.standard_normal((tk, hkv, d), dtype=np.float32)
        v = rng.standard_normal((tk, hkv, dv), dtype=np.float32)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    sinks = rng.standard_normal(hq, dtype=np.float32) if with_sinks else None
    return Dense(q, k, v, cu_q, cu_k, dtype, scale if scale is not None else 1.0 / np.sqrt(d),
                 causal, tuple(window), sinks)


def varlen_prefill(seed: int = SEED_VARLEN_PREFILL, nseq: int = 8, lo: int = 512,
                   hi: int = 4096, hq: int = 32, hkv: int = 8, d: int = 128) -> Dense:
    """Causal GQA prefill: nseq lengths uniform in [lo, hi] packed with
    cu_seqlens, bf16 N(0,1), scale 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, endpoint=True, size=nseq)
    return _varlen_draw(rng, lens, lens, hq, hkv, d, d, "bf16", True, (-1, -1), None, False)


@dataclasses.dataclass
class DenseKV(Dense):
    """A Dense problem whose keys also have an earlier part in a paged cache:
    k_cache (P,page,Hkv,D), v_cache (P,page,Hkv,Dv) bits, block_table
    (B, max_pages) int32 (-1 past a sequence's pages), cache_seqlens (B)."""
    k_cache: np.ndarray = None
    v_cache: np.ndarray = None
    block_table: np.ndarray = None
    cache_seqlens: np.ndarray = None
    page_size: int = 0


def varlen_kvcache(seed: int, lens_q, lens_new, lens_cache, hq: int = 32, hkv: int = 8,
                   d: int = 128, page: int = 64, causal: bool = True, window=(-1, -1),
                   scale: float | None = None, with_sinks: bool = False,
                   spare_pages: int = 0, with_qv: bool = False) -> DenseKV:
    """Chunked prefill: per sequence lens_q queries and lens_new current K/V
    rows (packed as in varlen), after lens_cache earlier rows held in a paged
    bf16 cache. The pool has spare_pages pages that no sequence references.
    Draw order: Q, K, V, K cache, V cache, page permutation, sinks, then qv
    (Tq, Hq, D) when with_qv."""
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_new = np.asarray(lens_new, dtype=np.int64)
    lens_cache = np.asarray(lens_cache, dtype=np.int64)
    tq, tk = int(lens_q.sum()), int(lens_new.sum())
    q = _normal_bf16(rng, (tq, hq, d))
    k = _normal_bf16(rng, (tk, hkv, d))
    v = _normal_bf16(rng, (tk, hkv, d))
    nblk = (lens_cache + page - 1) // page
    pool = max(1, int(nblk.sum()) + spare_pages)
    k_cache = _normal_bf16(rng, (pool, page, hkv, d))
    v_cache = _normal_bf16(rng, (pool, page, hkv, d))
    perm = rng.permutation(pool).astype(np.int32)
    table = np.full((len(lens_cache), max(1, int(nblk.max()))), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    sinks = rng.standard_normal(hq, dtype=np.float32) if with_sinks else None
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_new)]).astype(np.int32)
    w = DenseKV(q, k, v, cu_q, cu_k, "bf16", scale if scale is not None else 1.0 / np.sqrt(d),
                causal, tuple(window), sinks, k_cache=k_cache, v_cache=v_cache,
                block_table=table, cache_seqlens=lens_cache.astype(np.int32), page_size=page)
    if with_qv:
        w.qv = _normal_bf16(rng, (tq, hq, d))
    return w


def chunked_prefill(seed: int = SEED_CHUNKED_PREFILL, nseq: int = 8, chunk: int = 1024,
                    lo: int = 1024, hi: int = 8192, hq: int = 32, hkv: int = 8, d: int = 128,
                    page: int = 64) -> DenseKV:
    """Chunked causal GQA prefill: nseq sequences, each a chunk of `chunk` new
    tokens after a cached prefix of U[lo, hi] tokens in a paged cache."""
    rng = np.random.default_rng(seed)
    lens_cache = rng.integers(lo, hi, endpoint=True, size=nseq)
    lens = np.full(nseq, chunk)
    return varlen_kvcache(int(rng.integers(0, 2**63 - 1)), lens, lens, lens_cache, hq=hq,
                          hkv=hkv, d=d, page=page, causal=True)


def chunked_mask(rows: int, ld: int, seed: int = SEED_CHUNKED_PREFILL) -> np.ndarray:
    """A (1, rows, ld) additive mask of N(0,1) values rounded to bf16 bits."""
    return _normal_bf16(np.random.default_rng(seed + 100), (1, rows, ld))


@dataclasses.dataclass
class Paged:
    """Decode against a paged cache. q (B,Sq,Hq,D) bits; k_cache (P,page,Hkv,D)
    bits; v_cache (P,page,Hkv,Dv) bits, or None when K and V share one cache
    (the value of key j is then its first dv entries)."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray | None
    block_table: np.ndarray
    cache_seqlens: np.ndarray
    page_size: int
    dv: int
    scale: float
    causal: bool
    sinks: np.ndarray | None = None
    qv: np.ndarray | None = None     # (B,Sq,Hq,Dv) bits of the second query, or None

    @property
    def batch(self):
        return self.q.shape[0]


def paged(seed: int, lens, sq: int = 1, hq: int = 32, hkv: int = 8, d: int = 128,
          dv: int | None = None, page: int = 64, shared_kv: bool = False,
          causal: bool = False, scale: float | None = None, with_sinks: bool = False,
          with_qv: bool = False) -> Paged:
    """Draw order: Q, K cache, V cache, page permutation, sinks, then qv."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    w = _paged_draw(rng, lens, sq, hq, hkv, d, dv or d, page, shared_kv, causal,
                    scale, with_sinks)
    if with_qv:
        w.qv = _normal_bf16(rng, (len(lens), sq, hq, dv or d))
    return w


def _paged_draw(rng, lens, sq, hq, hkv, d, dv, page, shared_kv, causal, scale, with_sinks):
    b = len(lens)
    nblk = (lens + page - 1) // page
    pool = max(1, int(nblk.sum()))
    q = _normal_bf16(rng, (b, sq, hq, d))
    k_cache = _normal_bf16(rng, (pool, page, hkv, d))
    v_cache = None if shared_kv else _normal_bf16(rng, (pool, page, hkv, dv))
    table, _ = _paged_table(rng, lens, page)
    sinks = rng.standard_normal(hq, dtype=np.float32) if with_sinks else None
    return Paged(q, k_cache, v_cache, table, lens.astype(np.int32), page, dv,
                 scale if scale is not None else 1.0 / np.sqrt(d), causal, sinks)


# FP8 codes of the OCP formats e4m3fn and e5m2: (mantissa bits, bias,
# largest finite value).
_FP8 = {"e4m3": (3, 7, 448.0), "e5m2": (2, 15, 57344.0)}


def fp8_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Rounds float32 values to the nearest code of an FP8 format (ties to
    even, saturating at the largest finite value) and returns uint8 codes.
    Normal results come from the float32 bit pattern rounded at the format's
    mantissa width with the exponent rebiased; below the least normal value
    the code is the multiple of the least subnormal, rounded half to even."""
    mbits, bias, vmax = _FP8[fmt]
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(vmax))
    u = a.view(np.uint32)
    sh = 23 - mbits
    r = (u + np.uint32((1 << (sh - 1)) - 1) + ((u >> sh) & 1)) >> sh   # exponent | mantissa
    normal = (r.astype(np.int64) - ((127 - bias) << mbits))
    sub = np.rint(a * np.float32(2.0 ** (bias - 1 + mbits))).astype(np.int64)
    code = np.where(a < np.float32(2.0 ** (1 - bias)), sub, normal)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def _normal_fp8(rng: np.random.Generator, shape, fmt: str, mult) -> np.ndarray:
    """N(0,1) float32 draws times a multiplier per row of the last dimension
    (mult(r0, r1) gives those of rows [r0, r1) of the flattened tensor),
    rounded to FP8 codes; blocks of _CHUNK elements drawn as in _normal_bf16
    (one key, one stream per block)."""
    n = int(np.prod(shape))
    d = shape[-1]
    assert _CHUNK % d == 0
    out = np.empty(n, dtype=np.uint8)
    key = int(rng.integers(0, 2**63 - 1))

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, i])))
        x = g.standard_normal(e - s, dtype=np.float32).reshape(-1, d)
        out[s:e] = fp8_bits(x * mult(s // d, e // d)[:, None], fmt).ravel()

    nblk = (n + _CHUNK - 1) // _CHUNK
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1, nblk))) as ex:
        list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


@dataclasses.dataclass
class PagedFP8:
    """Decode against a paged FP8 cache: q (B,Sq,Hq,D), k_cache (P,page,Hkv,D)
    and v_cache (P,page,Hkv,Dv) uint8 codes of format fmt; descales float32
    (B, Hkv) or None."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    fmt: str
    q_descale: np.ndarray | None
    k_descale: np.ndarray | None
    v_descale: np.ndarray | None
    block_table: np.ndarray
    cache_seqlens: np.ndarray
    page_size: int
    scale: float
    causal: bool
    qv: np.ndarray | None = None     # (B,Sq,Hq,Dv) codes of the second query, or None

    @property
    def batch(self):
        return self.q.shape[0]


def paged_fp8(seed: int, lens, fmt: str = "e4m3", sq: int = 1, hq: int = 32, hkv: int = 8,
              d: int = 128, page: int = 64, causal: bool = False, descale: bool = True,
              spare_pages: int = 0, with_qv: bool = False) -> PagedFP8:
    """N(0,1) Q, K, V stored as FP8 codes of x / descale, with descales drawn
    per (batch, KV head) from U[0.25, 4] (or none); a cache page is quantized
    with the descales of the sequence that owns it. Draw order: descales, Q,
    page permutation, K cache, V cache, then qv (quantized with the Q
    descales)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    b = len(lens)
    ds = [rng.uniform(0.25, 4.0, size=(b, hkv)).astype(np.float32) if descale else None
          for _ in range(3)]
    one = np.ones((b, hkv), np.float32)
    qd, kd, vd = (one if x is None else x for x in ds)
    nblk = (lens + page - 1) // page
    pool = max(1, int(nblk.sum()) + spare_pages)
    grp = hq // hkv
    # multiplier of flattened element i of q (B, Sq, Hq, D): 1 / qd[b, h // grp]
    qinv = np.repeat(1.0 / qd, grp, axis=1).astype(np.float32)       # (B, Hq)

    def qmult(r0, r1):                     # rows of q are (b, t, h)
        r = np.arange(r0, r1)
        return qinv[r // (sq * hq), r % hq]

    q8 = _normal_fp8(rng, (b, sq, hq, d), fmt, qmult)
    table, _ = _paged_table(rng, lens, page)
    owner = np.zeros(pool, np.int64)
    for bi, n in enumerate(nblk):
        owner[table[bi, :n]] = bi

    def cmult(inv):                        # rows of a cache are (page, slot, kv head)
        def f(r0, r1):
            r = np.arange(r0, r1)
            return inv[owner[r // (page * hkv)], r % hkv]
        return f

    k8 = _normal_fp8(rng, (pool, page, hkv, d), fmt, cmult((1.0 / kd).astype(np.float32)))
    v8 = _normal_fp8(rng, (pool, page, hkv, d), fmt, cmult((1.0 / vd).astype(np.float32)))
    qv8 = _normal_fp8(rng, (b, sq, hq, d), fmt, qmult) if with_qv else None
    return PagedFP8(q8, k8, v8, fmt, ds[0], ds[1], ds[2], table, lens.astype(np.int32), page,
                    1.0 / np.sqrt(d), causal, qv8)


@dataclasses.dataclass
class DenseFP8:
    """Packed varlen problem with FP8 codes: q (Tq,Hq,D), k (Tk,Hkv,D),
    v (Tk,Hkv,Dv) uint8 of format fmt; descales float32 (B, Hkv) or None."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    fmt: str
    q_descale: np.ndarray | None
    k_descale: np.ndarray | None
    v_descale: np.ndarray | None
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    scale: float
    causal: bool
    window: tuple
    sinks: np.ndarray | None = None
    qv: np.ndarray | None = None     # (Tq,Hq,Dv) codes of the second query, or None


def varlen_fp8(seed: int, lens_q, lens_k=None, fmt: str = "e4m3", hq: int = 32, hkv: int = 8,
               d: int = 128, causal: bool = True, window=(-1, -1),
               descale: bool = True, with_sinks: bool = False,
               with_qv: bool = False) -> DenseFP8:
    """N(0,1) Q, K, V stored as FP8 codes of x / descale, descales per
    (sequence, KV head) from U[0.25, 4] (or none); sinks float32 N(0,1) per
    query head. Draw order: descales, Q, K, V, sinks, then qv (with the Q
    descales)."""
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = lens_q if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    b = len(lens_q)
    ds = [rng.uniform(0.25, 4.0, size=(b, hkv)).astype(np.float32) if descale else None
          for _ in range(3)]
    one = np.ones((b, hkv), np.float32)
    qd, kd, vd = (one if x is None else x for x in ds)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    seq_q = np.repeat(np.arange(b), lens_q)          # sequence of each packed row
    seq_k = np.repeat(np.arange(b), lens_k)
    grp = hq // hkv
    qinv = np.repeat(1.0 / qd, grp, axis=1).astype(np.float32)   # (B, Hq)
    kinv, vinv = (1.0 / kd).astype(np.float32), (1.0 / vd).astype(np.float32)

    def rows_q(r0, r1):                    # rows of q are (token, head)
        r = np.arange(r0, r1)
        return qinv[seq_q[r // hq], r % hq]

    def rows_kv(inv):
        def f(r0, r1):
            r = np.arange(r0, r1)
            return inv[seq_k[r // hkv], r % hkv]
        return f

    q = _normal_fp8(rng, (int(lens_q.sum()), hq, d), fmt, rows_q)
    k = _normal_fp8(rng, (int(lens_k.sum()), hkv, d), fmt, rows_kv(kinv))
    v = _normal_fp8(rng, (int(lens_k.sum()), hkv, d), fmt, rows_kv(vinv))
    sinks = rng.standard_normal(hq).astype(np.float32) if with_sinks else None
    qv = _normal_fp8(rng, (int(lens_q.sum()), hq, d), fmt, rows_q) if with_qv else None
    return DenseFP8(q, k, v, fmt, ds[0], ds[1], ds[2], cu_q, cu_k, 1.0 / np.sqrt(d), causal,
                    tuple(window), sinks, qv)


def varlen_prefill_fp8(seed: int = SEED_VARLEN_PREFILL_FP8) -> DenseFP8:
    """The varlen causal GQA prefill shape (8 sequences U[512, 4096], Hq=32,
    Hkv=8, D=128) with e4m3 Q/K/V codes and per-(sequence, KV head)
    descales."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4096, endpoint=True, size=8)
    return varlen_fp8(int(rng.integers(0, 2**63 - 1)), lens, fmt="e4m3")


@dataclasses.dataclass
class DenseKVFP8(DenseFP8):
    """A DenseFP8 problem whose keys also have an earlier part in a paged FP8
    cache: k_cache (P,page,Hkv,D), v_cache (P,page,Hkv,D) uint8 codes,
    block_table (B, max_pages) int32 (-1 past a sequence's pages),
    cache_seqlens (B)."""
    k_cache: np.ndarray = None
    v_cache: np.ndarray = None
    block_table: np.ndarray = None
    cache_seqlens: np.ndarray = None
    page_size: int = 0


def varlen_kvcache_fp8(seed: int, lens_q, lens_new, lens_cache, fmt: str = "e4m3",
                       hq: int = 32, hkv: int = 8, d: int = 128, page: int = 64,
                       causal: bool = True, window=(-1, -1), descale: bool = True,
                       with_sinks: bool = False) -> DenseKVFP8:
    """Chunked prefill on FP8 codes: per sequence lens_q queries and lens_new
    current K/V rows after lens_cache rows in a paged cache. Every value is
    N(0,1) stored as the FP8 code of x / descale, with the descales of its
    sequence (per KV head, U[0.25, 4], or none); a cache page takes those of
    the sequence that owns it (pages are not shared). Draw order: descales,
    page permutation, Q, K, V, K cache, V cache, sinks."""
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_new = np.asarray(lens_new, dtype=np.int64)
    lens_cache = np.asarray(lens_cache, dtype=np.int64)
    b = len(lens_q)
    ds = [rng.uniform(0.25, 4.0, size=(b, hkv)).astype(np.float32) if descale else None
          for _ in range(3)]
    one = np.ones((b, hkv), np.float32)
    qd, kd, vd = (one if x is None else x for x in ds)
    table, pool = _paged_table(rng, lens_cache, page)
    owner = np.zeros(max(1, pool), dtype=np.int64)
    for s, row in enumerate(table):
        owner[row[row >= 0]] = s
    pool = max(1, pool)
    seq_q = np.repeat(np.arange(b), lens_q)
    seq_k = np.repeat(np.arange(b), lens_new)
    qinv = np.repeat(1.0 / qd, hq // hkv, axis=1).astype(np.float32)   # (B, Hq)
    kinv, vinv = (1.0 / kd).astype(np.float32), (1.0 / vd).astype(np.float32)

    def rows_q(r0, r1):
        r = np.arange(r0, r1)
        return qinv[seq_q[r // hq], r % hq]

    def rows_new(inv):
        def f(r0, r1):
            r = np.arange(r0, r1)
            return inv[seq_k[r // hkv], r % hkv]
        return f

    def rows_cache(inv):                   # rows are (page, slot, head)
        def f(r0, r1):
            r = np.arange(r0, r1)
            return inv[owner[r // (page * hkv)], r % hkv]
        return f

    tq, tk = int(lens_q.sum()), int(lens_new.sum())
    q = _normal_fp8(rng, (tq, hq, d), fmt, rows_q)
    k = _normal_fp8(rng, (tk, hkv, d), fmt, rows_new(kinv))
    v = _normal_fp8(rng, (tk, hkv, d), fmt, rows_new(vinv))
    k_cache = _normal_fp8(rng, (pool, page, hkv, d), fmt, rows_cache(kinv))
    v_cache = _normal_fp8(rng, (pool, page, hkv, d), fmt, rows_cache(vinv))
    sinks = rng.standard_normal(hq).astype(np.float32) if with_sinks else None
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_new)]).astype(np.int32)
    return DenseKVFP8(q, k, v, fmt, ds[0], ds[1], ds[2], cu_q, cu_k, 1.0 / np.sqrt(d), causal,
                      tuple(window), sinks, k_cache=k_cache, v_cache=v_cache, block_table=table,
                      cache_seqlens=lens_cache.astype(np.int32), page_size=page)


def chunked_prefill_fp8(seed: int = SEED_CHUNKED_PREFILL_FP8, nseq: int = 8, chunk: int = 1024,
                        lo: int = 1024, hi: int = 8192, fmt: str = "e4m3") -> DenseKVFP8:
    """The chunked causal GQA prefill shape (nseq chunks of `chunk` new tokens
    after cached prefixes of U[lo, hi] tokens, Hq=32, Hkv=8, D=128, page 64) on
    FP8 codes with per-(sequence, KV head) descales."""
    rng = np.random.default_rng(seed)
    lens_cache = rng.integers(lo, hi, endpoint=True, size=nseq)
    lens = np.full(nseq, chunk)
    return varlen_kvcache_fp8(int(rng.integers(0, 2**63 - 1)), lens, lens, lens_cache, fmt)


def paged_decode_fp8(seed: int = SEED_PAGED_DECODE_FP8, batch: int = 64, lo: int = 1024,
                     hi: int = 32768, page: int = 64, hq: int = 32, hkv: int = 8,
                     d: int = 128, fmt: str = "e4m3") -> PagedFP8:
    """GQA decode with an FP8 cache: the paged-decode shape (one query token,
    cache_seqlens U[lo, hi], page 64, Hq=32, Hkv=8, D=128) with e4m3 Q/K/V
    codes and per-(batch, KV head) descales."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, endpoint=True, size=batch)
    return paged_fp8(int(rng.integers(0, 2**63 - 1)), lens, fmt, 1, hq, hkv, d, page)


def paged_decode(seed: int = SEED_PAGED_DECODE, batch: int = 64, lo: int = 1024,
                 hi: int = 32768, page: int = 64, hq: int = 32, hkv: int = 8,
                 d: int = 128) -> Paged:
    """GQA decode: one query token per sequence, cache lengths uniform in
    [lo, hi], bf16 N(0,1) K and V caches, non-causal, scale 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, endpoint=True, size=batch)
    return _paged_draw(rng, lens, 1, hq, hkv, d, d, page, False, False, None, False)


def varlen_prefill_qv(w: Dense, seed: int = SEED_VARLEN_PREFILL_QV) -> np.ndarray:
    """A bf16 N(0,1) qv (Tq, Hq, Dv) for a packed problem w, from its own seed."""
    rng = np.random.default_rng(seed)
    return _normal_bf16(rng, w.q.shape[:2] + (w.v.shape[2],))


def paged_decode_qv(w: Paged, seed: int = SEED_PAGED_DECODE_QV) -> np.ndarray:
    """A bf16 N(0,1) qv (B, Sq, Hq, Dv) for a paged problem w, from its own
    seed (w's draws stay those of its generator)."""
    rng = np.random.default_rng(seed)
    return _normal_bf16(rng, w.q.shape[:3] + (w.dv,))


def mla_decode(seed: int = SEED_MLA_DECODE, batch: int = 64, sq: int = 2, hq: int = 128,
               d: int = 576, dv: int = 512, page: int = 64, lo: int = 2048,
               hi: int = 16384) -> Paged:
    """MLA-absorbed decode: one latent+rope row of width d per cached token,
    one KV head, value = first dv entries of the row, scale 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, endpoint=True, size=batch)
    return _paged_draw(rng, lens, sq, hq, 1, d, dv, page, True, False, None, False)


def mla_mate_example(seed: int = 1013) -> Paged:
    """The shapes of the MATE minimal MLA example: q (1, 32, 8, 576) and
    k_cache (4, 16, 2, 576) N(0,1) bf16, block_table zeros (1, 4) (every
    logical page is physical page 0), page 16, cache_seqlens [32], value = the
    first 512 entries of a row, scale 1/sqrt(576). Draw order: Q, cache."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (1, 32, 8, 576))
    k_cache = _normal_bf16(rng, (4, 16, 2, 576))
    return Paged(q, k_cache, None, np.zeros((1, 4), np.int32), np.array([32], np.int32), 16, 512,
                 1.0 / np.sqrt(576), False)


@dataclasses.dataclass
class Sparse:
    """Top-k sparse MLA: q (B,Sq,Hq,D) bits, kv (B,Sk,1,D) bits, indices
    (B,Sq,1,topk) int32 with -1 marking unused slots, sinks (Hq) float32 or None."""
    q: np.ndarray
    kv: np.ndarray
    indices: np.ndarray
    sinks: np.ndarray | None
    dv: int
    scale: float
    sparse_mode: int

    @property
    def batch(self):
        return self.q.shape[0]


@dataclasses.dataclass
class SparsePaged:
    """Block-sparse MLA over a paged latent cache: q (B,Sq,Hq,D) bits,
    kv_cache (P,page,1,D) bits, block_table (B, max_pages) int32 (-1 past a
    sequence's pages), seqlens_kv (B) int32, indices (B,Sq,1,topk) int32 block
    numbers (-1 unused), block_size keys per index."""
    q: np.ndarray
    kv_cache: np.ndarray
    block_table: np.ndarray
    seqlens_kv: np.ndarray
    page_size: int
    indices: np.ndarray
    block_size: int
    sinks: np.ndarray | None
    dv: int
    scale: float
    sparse_mode: int


def sparse_paged(seed: int, lens_kv, sq: int, topk: int, block_size: int = 1, page: int = 64,
                 hq: int = 64, d: int = 576, dv: int = 512, sparse_mode: int = 3,
                 with_sinks: bool = True, spare_pages: int = 0) -> SparsePaged:
    """Per query token t of sequence b, topk distinct block numbers drawn
    without replacement from the blocks that hold keys of its bottom-right
    causal prefix [0, Lk_b - sq + t] (all of them, in random order, when there
    are fewer), padded with -1. Draw order: Q, cache, page permutation,
    indices, sinks."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens_kv, dtype=np.int64)
    batch = len(lens)
    nblk = (lens + page - 1) // page
    pool = max(1, int(nblk.sum()) + spare_pages)
    q = _normal_bf16(rng, (batch, sq, hq, d))
    kv = _normal_bf16(rng, (pool, page, 1, d))
    table, _ = _paged_table(rng, lens, page)
    idx = np.full((batch, sq, 1, topk), -1, dtype=np.int32)
    for b in range(batch):
        for t in range(sq):
            p = max(0, min(int(lens[b]), int(lens[b]) - sq + t + 1))
            nb = (p + block_size - 1) // block_size
            n = min(topk, nb)
            if n:
                idx[b, t, 0, :n] = rng.choice(nb, n, replace=False)
    sinks = rng.standard_normal(hq, dtype=np.float32) if with_sinks else None
    return SparsePaged(q, kv, table, lens.astype(np.int32), page, idx, block_size, sinks, dv,
                       1.0 / np.sqrt(d), sparse_mode)


def sparse_paged_blocks(seed: int = SEED_SPARSE_PAGED, batch: int = 4, sq: int = 4096,
                        sk: int = 32768, topk: int = 32, block_size: int = 64, page: int = 64,
                        hq: int = 64) -> SparsePaged:
    """Block-sparse MLA over a paged cache: the sparse-MLA shape (4 x 4096
    query tokens, 32768 cached keys per sequence, Hq=64, D=576, sinks) with
    32 blocks of 64 keys selected per token (2048 keys, as the token-sparse
    workload), page 64, mode 3."""
    return sparse_paged(seed, [sk] * batch, sq, topk, block_size, page, hq)


def sparse_mla(seed: int = SEED_SPARSE_MLA, batch: int = 4, sq: int = 4096, sk: int = 32768,
               hq: int = 64, d: int = 576, dv: int = 512, topk: int = 2048,
               sparse_mode: int = 3, with_sinks: bool = True,
               scale: float | None = None) -> Sparse:
    """Per query token t, topk distinct key indices drawn without replacement
    from its bottom-right causal prefix [0, sk - sq + t] (all of them, in random
    order, when the prefix is shorter than topk), padded with -1. One sink logit
    per query head, float32 N(0,1)."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (batch, sq, hq, d))
    kv = _normal_bf16(rng, (batch, sk, 1, d))
    idx = np.full((batch, sq, 1, topk), -1, dtype=np.int32)
    delta = sk - sq
    for b in range(batch):
        for t in range(sq):
            p = max(0, min(sk, delta + t + 1))
            n = min(topk, p)
            if n:
                idx[b, t, 0, :n] = rng.choice(p, n, replace=False)
    sinks = rng.standard_normal(hq, dtype=np.float32) if with_sinks else None
    return Sparse(q, kv, idx, sinks, dv, scale if scale is not None else 1.0 / np.sqrt(d),
                  sparse_mode)
