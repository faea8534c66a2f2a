"""ctypes binding of libattn_mi355.so.

Argument marshalling only: every function here checks that the torch tensors
match the shapes and dtypes of the C ABI (include/attn.h), passes their device
pointers and the current HIP stream, and turns a non-zero status into a Python
exception. All arithmetic runs in the library's kernels. There is no fallback:
when the library is missing or no GPU is present, calls raise.

Function names are those of the C ABI.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_mi355.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EEMPTY, ATTN_EHIP = range(5)
ATTN_BF16, ATTN_F32, ATTN_FP8_E4M3, ATTN_FP8_E5M2 = 0, 1, 2, 3
ATTN_GATHER_DECODE, ATTN_GATHER_MLA = 0, 1
FP8_FORMATS = {"e4m3": ATTN_FP8_E4M3, "e5m2": ATTN_FP8_E5M2}

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float

_SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_device_info": (_I, [_I, ctypes.POINTER(_I)]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                             _P, _P, _P, _P]),
    # q, k, v, cu_q, cu_k, batch, max_q, max_k, hq, hkv, d, dv, scale, causal, wl, wr, sinks,
    # mask, mask_heads, mask_ld, out, lse, stream
    "attn_fwd_varlen_mask": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                                  _P, _P, _I, _I, _P, _P, _P]),
    "attn_fwd_varlen_fp8": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                 _F, _I, _I, _I, _P, _P, _P, _P]),
    "attn_fwd_varlen_qv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                _P, _F, _I, _I, _I, _P, _I, _P, _P, _P]),
    "attn_fwd_varlen_kvcache": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                     _I, _I, _I, _F, _I, _I, _I, _P, _P, _I, _I, _P, _P, _P]),
    # q, qv, k, v, cu_q, cu_k, k_cache, v_cache, block_table, max_pages, cache_lens, page,
    # batch, max_q, hq, hkv, d, dv, scale, causal, wl, wr, sinks, only_qv, out, lse, stream
    "attn_fwd_varlen_kvcache_qv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I,
                                        _I, _I, _I, _I, _F, _I, _I, _I, _P, _I, _P, _P, _P]),
    "attn_fwd_varlen_kvcache_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I,
                                         _I, _I, _I, _I, _P, _P, _P, _F, _I, _I, _I, _P, _P, _P,
                                         _P]),
    "attn_plan_words": (ctypes.c_size_t, [_I, _I]),
    "attn_plan_splits": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                               _P, _I, _P, _P, _P]),
    # q, k_cache, v_cache, block_table, max_pages, lens, batch, sq, hq, hkv, d, dv, page, scale,
    # causal, mask, mask_heads, mask_ld, plan, max_splits, o_part, lse_part, stream
    "attn_decode_paged_mask": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                    _P, _I, _I, _P, _I, _P, _P, _P]),
    "attn_decode_paged_fp8": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                                   _P, _P, _F, _I, _P, _I, _P, _P, _P]),
    "attn_decode_paged_qv": (_I, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                  _P, _P, _P, _F, _I, _I, _P, _I, _P, _P, _P]),
    "attn_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P]),
    "mla_decode_paged": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _F, _I, _P, _I, _P, _P, _P]),
    "mla_sparse_fwd": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P]),
    "mla_sparse_paged_fwd": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                                  _P, _P, _P, _P]),
    "attn_decode_paged_noalloc_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                       _F, _I, _P, _I, _I, _I, _I, _P, _P, _P]),
    "attn_debug_gather_paged": (_I, [_I, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _I, _I, _P,
                                     _P, _P]),
    "attn_debug_gather_kvcache": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                       _I, _P, _P, _P]),
    "attn_debug_gather_sparse": (_I, [_P, _I, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _P,
                                      _P]),
}

_lib = None


class AttnError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Loads the library once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise AttnError(f"{path} is missing: build it with attention_attn_fwd_02_amd.build")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def _check(status: int):
    if status == ATTN_OK:
        return
    msg = load().attn_last_error().decode()
    name = load().attn_status_string(status).decode()
    text = f"{name}: {msg}"
    if status in (ATTN_EINVAL, ATTN_EEMPTY):
        raise ValueError(text)
    if status == ATTN_EUNSUPPORTED:
        raise NotImplementedError(text)
    raise AttnError(text)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _scale(scale, query):
    """The softmax scale; None means 1/sqrt(D) of the query's head dimension
    (the lite_boost flash_attention softmax_scale default)."""
    return 1.0 / math.sqrt(query.shape[-1]) if scale is None else float(scale)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts, dtype=None):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"expected {dtype}, got {t.dtype}")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------- prefill
def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    scale=None, causal=False, window=(-1, -1), sinks=None, out=None, lse=None,
                    return_lse=True):
    """q (Tq,Hq,D), k (Tk,Hkv,D), v (Tk,Hkv,Dv) bf16 or fp32; cu_seqlens int32
    (B+1). Returns (out (Tq,Hq,Dv), lse (Hq,Tq) fp32 or None)."""
    _dev(q, k, v)
    _dev(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v dtypes differ")
    tq, hq, d = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=q.dtype)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k),
                                  hq, hkv, d, dv, _dtype_code(q), _scale(scale, q),
                                  int(bool(causal)), int(window[0]), int(window[1]), _ptr(sinks),
                                  _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_fp8(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                        scale=None, fmt="e4m3", q_descale=None, k_descale=None, v_descale=None,
                        causal=False, window=(-1, -1), sinks=None, out=None, lse=None,
                        return_lse=True):
    """q (Tq,Hq,128), k (Tk,Hkv,128), v (Tk,Hkv,128) uint8 FP8 codes of fmt
    ("e4m3" or "e5m2"); descales float32 (B,Hkv) or None; cu_seqlens int32
    (B+1). Returns (out (Tq,Hq,128) bf16, lse (Hq,Tq) fp32 or None)."""
    _dev(q, k, v, dtype=torch.uint8)
    _dev(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    _dev(sinks, q_descale, k_descale, v_descale, dtype=torch.float32)
    tq, hq, d = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    batch = cu_seqlens_q.numel() - 1
    for t in (q_descale, k_descale, v_descale):
        if t is not None and tuple(t.shape) != (batch, hkv):
            raise ValueError("descales must be (batch, hkv)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, dv, FP8_FORMATS[fmt], _ptr(q_descale),
        _ptr(k_descale), _ptr(v_descale), _scale(scale, q), int(bool(causal)), int(window[0]),
        int(window[1]), _ptr(sinks), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_qv(q, qv, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                       scale=None, fmt=None, q_descale=None, k_descale=None, v_descale=None,
                       causal=False, window=(-1, -1), sinks=None, only_qv=False, out=None, lse=None,
                       return_lse=True):
    """Varlen attention with a second query qv (Tq,Hq,128) scored against the
    value rows. fmt None: bf16 tensors; "e4m3" / "e5m2": uint8 FP8 codes with
    optional float32 (B,Hkv) descales. only_qv: q and k are not used (may be
    None). Returns (out (Tq,Hq,128) bf16, lse (Hq,Tq) fp32 or None)."""
    el = torch.bfloat16 if fmt is None else torch.uint8
    _dev(q, qv, k, v, dtype=el)
    _dev(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    _dev(sinks, q_descale, k_descale, v_descale, dtype=torch.float32)
    if qv is None or v is None:
        raise ValueError("qv and v are required")
    tq, hq, dv = qv.shape
    hkv = v.shape[1]
    d = dv if only_qv or q is None else q.shape[2]
    batch = cu_seqlens_q.numel() - 1
    for t in (q_descale, k_descale, v_descale):
        if t is not None and tuple(t.shape) != (batch, hkv):
            raise ValueError("descales must be (batch, hkv)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=torch.bfloat16, device=qv.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=qv.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    code = ATTN_BF16 if fmt is None else FP8_FORMATS[fmt]
    _check(load().attn_fwd_varlen_qv(
        None if only_qv else _ptr(q), _ptr(qv), None if only_qv else _ptr(k), _ptr(v),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, int(max_seqlen_q), int(max_seqlen_k), hq,
        hkv, d, dv, code, _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        _scale(scale, qv if only_qv or q is None else q),
        int(bool(causal)), int(window[0]), int(window[1]), _ptr(sinks), int(bool(only_qv)),
        _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_mask(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, mask,
                         scale=None, causal=False, window=(-1, -1), sinks=None, out=None,
                         lse=None, return_lse=True):
    """attn_fwd_varlen (bf16) with an additive bf16 mask (1 or Hq, Tq, ld),
    ld a multiple of 64 and >= max_seqlen_k. Returns (out (Tq,Hq,Dv),
    lse (Hq,Tq) fp32 or None)."""
    _dev(q, k, v, mask, dtype=torch.bfloat16)
    _dev(cu_seqlens_q, cu_seqlens_k, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    tq, hq, d = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if mask.dim() != 3 or mask.shape[1] != tq:
        raise ValueError("mask must be (1 or Hq, Tq, ld)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=q.dtype)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen_mask(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, dv, _scale(scale, q),
        int(bool(causal)), int(window[0]), int(window[1]), _ptr(sinks), _ptr(mask), mask.shape[0],
        mask.shape[2], _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_kvcache(q, k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache, block_table,
                            cache_seqlens, max_seqlen_q, scale, causal=False, window=(-1, -1),
                            sinks=None, out=None, lse=None, return_lse=True, mask=None):
    """Current tokens q (Tq,Hq,D), k (Tk,Hkv,D), v (Tk,Hkv,Dv) with cu_seqlens
    as attn_fwd_varlen, over earlier tokens in k_cache (P,page,Hkv,D) and
    v_cache (P,page,Hkv,Dv), block_table (B,max_pages) and cache_seqlens (B)
    int32. bf16. mask: None or an additive bf16 mask (1 or Hq, Tq, ld), ld a
    multiple of 64. Returns (out (Tq,Hq,Dv), lse (Hq,Tq) fp32 or None)."""
    _dev(q, k, v, k_cache, v_cache, dtype=torch.bfloat16)
    _dev(cu_seqlens_q, cu_seqlens_k, block_table, cache_seqlens, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    _dev(mask, dtype=torch.bfloat16)
    tq, hq, d = q.shape
    hkv, dv = k.shape[1], v.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if mask is not None and (mask.dim() != 3 or mask.shape[1] != tq):
        raise ValueError("mask must be (1 or Hq, Tq, ld)")
    if k_cache.shape[2:] != (hkv, d) or v_cache.shape[2:] != (hkv, dv):
        raise ValueError("cache heads or widths differ from k, v")
    if block_table.dim() != 2 or block_table.shape[0] != batch or cache_seqlens.numel() != batch:
        raise ValueError("block_table must be (batch, max_pages) and cache_seqlens (batch)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=q.dtype)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen_kvcache(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
        k_cache.shape[1], batch, int(max_seqlen_q), hq, hkv, d, dv, ATTN_BF16, _scale(scale, q),
        int(bool(causal)), int(window[0]), int(window[1]), _ptr(sinks), _ptr(mask),
        0 if mask is None else mask.shape[0], 0 if mask is None else mask.shape[2], _ptr(out),
        _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_kvcache_qv(q, qv, k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache,
                               block_table, cache_seqlens, max_seqlen_q, scale=None,
                               causal=False, window=(-1, -1), sinks=None, only_qv=False,
                               out=None, lse=None, return_lse=True):
    """attn_fwd_varlen_kvcache (bf16, D = Dv = 128) with a second query qv
    (Tq,Hq,128) scored against the value rows, cached and current. only_qv:
    q, k and k_cache are not used (may be None). Returns (out (Tq,Hq,128) bf16,
    lse (Hq,Tq) fp32 or None)."""
    _dev(q, qv, k, v, k_cache, v_cache, dtype=torch.bfloat16)
    _dev(cu_seqlens_q, cu_seqlens_k, block_table, cache_seqlens, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    if qv is None or v is None or v_cache is None:
        raise ValueError("qv, v and v_cache are required")
    tq, hq, dv = qv.shape
    hkv = v_cache.shape[2]
    d = dv if only_qv or q is None else q.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if block_table.dim() != 2 or block_table.shape[0] != batch or cache_seqlens.numel() != batch:
        raise ValueError("block_table must be (batch, max_pages) and cache_seqlens (batch)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=torch.bfloat16, device=qv.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=qv.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen_kvcache_qv(
        _ptr(q), _ptr(qv), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), v_cache.shape[1], batch, int(max_seqlen_q), hq, hkv, d, dv,
        _scale(scale, qv if q is None else q), int(bool(causal)), int(window[0]),
        int(window[1]), _ptr(sinks), int(bool(only_qv)), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def attn_fwd_varlen_kvcache_fp8(q, k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache,
                                block_table, cache_seqlens, max_seqlen_q, scale=None,
                                fmt="e4m3", q_descale=None, k_descale=None, v_descale=None,
                                causal=False, window=(-1, -1), sinks=None, out=None, lse=None,
                                return_lse=True):
    """attn_fwd_varlen_kvcache on FP8 codes: q (Tq,Hq,128), k, v (Tk,Hkv,128)
    and k_cache, v_cache (P,page,Hkv,128) uint8 codes of fmt ("e4m3" or
    "e5m2"); descales float32 (B,Hkv) or None, one per (sequence, KV head) for
    its cached and current rows. Returns (out (Tq,Hq,128) bf16, lse (Hq,Tq)
    fp32 or None)."""
    _dev(q, k, v, k_cache, v_cache, dtype=torch.uint8)
    _dev(cu_seqlens_q, cu_seqlens_k, block_table, cache_seqlens, dtype=torch.int32)
    _dev(sinks, q_descale, k_descale, v_descale, dtype=torch.float32)
    tq, hq, d = q.shape
    hkv, dv = k_cache.shape[2], v_cache.shape[3]
    batch = cu_seqlens_q.numel() - 1
    if k_cache.shape[3] != d or (k is not None and k.shape[1:] != (hkv, d)) or \
            (v is not None and v.shape[1:] != (hkv, dv)):
        raise ValueError("cache heads or widths differ from q, k, v")
    if block_table.dim() != 2 or block_table.shape[0] != batch or cache_seqlens.numel() != batch:
        raise ValueError("block_table must be (batch, max_pages) and cache_seqlens (batch)")
    for t in (q_descale, k_descale, v_descale):
        if t is not None and tuple(t.shape) != (batch, hkv):
            raise ValueError("descales must be (batch, hkv)")
    if out is None:
        out = torch.empty((tq, hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_fwd_varlen_kvcache_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
        k_cache.shape[1], batch, int(max_seqlen_q), hq, hkv, d, dv, FP8_FORMATS[fmt],
        _ptr(q_descale), _ptr(k_descale), _ptr(v_descale), _scale(scale, q), int(bool(causal)),
        int(window[0]), int(window[1]), _ptr(sinks), _ptr(out), _ptr(lse), _stream()))
    return out, lse


# -------------------------------------------------------------------- planner
def attn_plan_words(batch, max_splits):
    return int(load().attn_plan_words(int(batch), int(max_splits)))


def attn_plan_splits(cache_seqlens, page_size, units_per_block, num_cu, waves, max_splits,
                     min_blocks, plan=None):
    _dev(cache_seqlens, dtype=torch.int32)
    batch = cache_seqlens.numel()
    if plan is None:
        plan = torch.zeros(attn_plan_words(batch, max_splits), dtype=torch.int32,
                           device=cache_seqlens.device)
    _dev(plan, dtype=torch.int32)
    _check(load().attn_plan_splits(_ptr(cache_seqlens), batch, int(page_size),
                                   int(units_per_block), int(num_cu), int(waves), int(max_splits),
                                   int(min_blocks), _ptr(plan), _stream()))
    return plan


def attn_device_info(device=0):
    n = _I(0)
    _check(load().attn_device_info(int(device), ctypes.byref(n)))
    return n.value


# --------------------------------------------------------------------- decode
def attn_decode_paged(q, k_cache, v_cache, block_table, cache_seqlens, plan, max_splits,
                      scale=None, causal=False, o_partial=None, lse_partial=None, mask=None):
    """q (B,Sq,Hq,D), caches (P,page,Hkv,D|Dv) bf16. Returns partials
    (B*max_splits, Sq*Hq, Dv) and (B*max_splits, Sq*Hq) fp32. With D = 576
    (MLA rows) v_cache is None and Dv = 512, the first entries of each row.
    mask: None or an additive bf16 mask (B, 1 or Hq, Sq, ld), ld a multiple
    of 64 and >= every cache length (attn_decode_paged_mask)."""
    _dev(q, k_cache, v_cache, mask, dtype=torch.bfloat16)
    _dev(block_table, cache_seqlens, plan, dtype=torch.int32)
    b, sq, hq, d = q.shape
    page, hkv = k_cache.shape[1], k_cache.shape[2]
    dv = 512 if v_cache is None and d == 576 else v_cache.shape[3]
    if o_partial is None:
        o_partial = torch.empty((b * max_splits, sq * hq, dv), dtype=torch.float32,
                                device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((b * max_splits, sq * hq), dtype=torch.float32, device=q.device)
    _dev(o_partial, lse_partial, dtype=torch.float32)
    if mask is not None:
        if mask.dim() != 4 or mask.shape[0] != b or mask.shape[2] != sq:
            raise ValueError("mask must be (B, 1 or Hq, Sq, ld)")
        _check(load().attn_decode_paged_mask(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
            _ptr(cache_seqlens), b, sq, hq, hkv, d, dv, page, _scale(scale, q),
            int(bool(causal)), _ptr(mask), mask.shape[1], mask.shape[3], _ptr(plan),
            int(max_splits), _ptr(o_partial), _ptr(lse_partial), _stream()))
        return o_partial, lse_partial
    _check(load().attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                    block_table.shape[1], _ptr(cache_seqlens), b, sq, hq, hkv, d,
                                    dv, page, ATTN_BF16, _scale(scale, q), int(bool(causal)),
                                    _ptr(plan), int(max_splits), _ptr(o_partial),
                                    _ptr(lse_partial), _stream()))
    return o_partial, lse_partial


def attn_decode_paged_fp8(q, k_cache, v_cache, block_table, cache_seqlens, plan, max_splits,
                          scale=None, fmt="e4m3", q_descale=None, k_descale=None, v_descale=None,
                          causal=False, o_partial=None, lse_partial=None):
    """q (B,Sq,Hq,D), caches (P,page,Hkv,D|Dv) uint8 FP8 codes of fmt ("e4m3" or
    "e5m2"); descales float32 (B,Hkv) or None. Returns partials as
    attn_decode_paged."""
    _dev(q, k_cache, v_cache, dtype=torch.uint8)
    _dev(block_table, cache_seqlens, plan, dtype=torch.int32)
    _dev(q_descale, k_descale, v_descale, dtype=torch.float32)
    b, sq, hq, d = q.shape
    page, hkv, dv = k_cache.shape[1], k_cache.shape[2], v_cache.shape[3]
    for t in (q_descale, k_descale, v_descale):
        if t is not None and tuple(t.shape) != (b, hkv):
            raise ValueError("descales must be (batch, hkv)")
    if o_partial is None:
        o_partial = torch.empty((b * max_splits, sq * hq, dv), dtype=torch.float32,
                                device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((b * max_splits, sq * hq), dtype=torch.float32, device=q.device)
    _dev(o_partial, lse_partial, dtype=torch.float32)
    _check(load().attn_decode_paged_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), b, sq, hq, hkv, d, dv, page, FP8_FORMATS[fmt], _ptr(q_descale),
        _ptr(k_descale), _ptr(v_descale), _scale(scale, q), int(bool(causal)), _ptr(plan),
        int(max_splits), _ptr(o_partial), _ptr(lse_partial), _stream()))
    return o_partial, lse_partial


def attn_decode_paged_qv(q, qv, k_cache, v_cache, block_table, cache_seqlens, plan, max_splits,
                         scale=None, fmt=None, q_descale=None, k_descale=None, v_descale=None,
                         causal=False, only_qv=False, o_partial=None, lse_partial=None):
    """Decode with a second query qv (B,Sq,Hq,Dv) scored against the value
    rows. fmt None: bf16 tensors; "e4m3" / "e5m2": uint8 FP8 codes with
    optional float32 (B,Hkv) descales. only_qv: q and k_cache are not used
    (may be None). Returns partials as attn_decode_paged."""
    el = torch.bfloat16 if fmt is None else torch.uint8
    _dev(q, qv, k_cache, v_cache, dtype=el)
    _dev(block_table, cache_seqlens, plan, dtype=torch.int32)
    _dev(q_descale, k_descale, v_descale, dtype=torch.float32)
    if qv is None or v_cache is None:
        raise ValueError("qv and v_cache are required")
    b, sq, hq, dv = qv.shape
    page, hkv = v_cache.shape[1], v_cache.shape[2]
    d = dv if only_qv or q is None else q.shape[3]
    for t in (q_descale, k_descale, v_descale):
        if t is not None and tuple(t.shape) != (b, hkv):
            raise ValueError("descales must be (batch, hkv)")
    if o_partial is None:
        o_partial = torch.empty((b * max_splits, sq * hq, dv), dtype=torch.float32,
                                device=qv.device)
    if lse_partial is None:
        lse_partial = torch.empty((b * max_splits, sq * hq), dtype=torch.float32,
                                  device=qv.device)
    _dev(o_partial, lse_partial, dtype=torch.float32)
    code = ATTN_BF16 if fmt is None else FP8_FORMATS[fmt]
    _check(load().attn_decode_paged_qv(
        None if only_qv else _ptr(q), _ptr(qv), None if only_qv else _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), b, sq, hq,
        hkv, d, dv, page, code, _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        _scale(scale, qv if only_qv or q is None else q),
        int(bool(causal)), int(bool(only_qv)), _ptr(plan), int(max_splits), _ptr(o_partial),
        _ptr(lse_partial), _stream()))
    return o_partial, lse_partial


def attn_combine(o_partial, lse_partial, plan, batch, seqlen_q, hq, max_splits, sinks=None,
                 out_dtype=torch.bfloat16, out=None, lse=None, return_lse=True):
    _dev(o_partial, lse_partial, dtype=torch.float32)
    _dev(plan, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    dv = o_partial.shape[2]
    if out is None:
        out = torch.empty((batch, seqlen_q, hq, dv), dtype=out_dtype, device=o_partial.device)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq, seqlen_q), dtype=torch.float32, device=o_partial.device)
    _dev(out)
    _dev(lse, dtype=torch.float32)
    _check(load().attn_combine(_ptr(o_partial), _ptr(lse_partial), _ptr(plan), int(batch),
                               int(seqlen_q), int(hq), dv, int(max_splits), _ptr(sinks),
                               _dtype_code(out), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def mla_decode_paged(q, kv_cache, block_table, cache_seqlens, plan, max_splits, scale=None,
                     causal=False, o_partial=None, lse_partial=None):
    """q (B,Sq,Hq,576), kv_cache (P,page,1,576) bf16; partials with Dv = 512."""
    _dev(q, kv_cache, dtype=torch.bfloat16)
    _dev(block_table, cache_seqlens, plan, dtype=torch.int32)
    b, sq, hq, d = q.shape
    if d != 576 or kv_cache.shape[3] != 576 or kv_cache.shape[2] != 1:
        raise NotImplementedError("MLA decode expects 576-wide rows and one KV head")
    if o_partial is None:
        o_partial = torch.empty((b * max_splits, sq * hq, 512), dtype=torch.float32,
                                device=q.device)
    if lse_partial is None:
        lse_partial = torch.empty((b * max_splits, sq * hq), dtype=torch.float32, device=q.device)
    _dev(o_partial, lse_partial, dtype=torch.float32)
    _check(load().mla_decode_paged(_ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   block_table.shape[1], _ptr(cache_seqlens), b, sq, hq,
                                   kv_cache.shape[1], _scale(scale, q), int(bool(causal)),
                                   _ptr(plan), int(max_splits), _ptr(o_partial), _ptr(lse_partial),
                                   _stream()))
    return o_partial, lse_partial


def mla_sparse_fwd(q, kv, sparse_indices, scale=None, sparse_mode=3, sinks=None, out=None,
                   lse=None, return_lse=True):
    """q (B,Sq,Hq,576), kv (B,Sk,1,576) bf16, indices (B,Sq,1,topk) int32."""
    _dev(q, kv, dtype=torch.bfloat16)
    _dev(sparse_indices, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    b, sq, hq, d = q.shape
    sk = kv.shape[1]
    if d != 576 or kv.shape[3] != 576 or kv.shape[2] != 1:
        raise NotImplementedError("sparse MLA expects 576-wide rows and one KV head")
    topk = sparse_indices.shape[-1]
    if out is None:
        out = torch.empty((b, sq, hq, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    _check(load().mla_sparse_fwd(_ptr(q), _ptr(kv), _ptr(sparse_indices), topk, b, sq, sk, hq,
                                 _scale(scale, q), int(sparse_mode), _ptr(sinks), _ptr(out),
                                 _ptr(lse), _stream()))
    return out, lse


def mla_sparse_paged_fwd(q, kv_cache, block_table, seqlens_kv, sparse_indices, scale=None,
                         sparse_block_size=1, sparse_mode=3, sinks=None, out=None, lse=None,
                         return_lse=True):
    """q (B,Sq,Hq,576) bf16, kv_cache (P,page,1,576) bf16, block_table
    (B,max_pages) and seqlens_kv (B) int32, indices (B,Sq,1,topk) int32."""
    _dev(q, kv_cache, dtype=torch.bfloat16)
    _dev(block_table, seqlens_kv, sparse_indices, dtype=torch.int32)
    _dev(sinks, dtype=torch.float32)
    b, sq, hq, d = q.shape
    if d != 576 or kv_cache.shape[3] != 576 or kv_cache.shape[2] != 1:
        raise NotImplementedError("sparse MLA expects 576-wide rows and one KV head")
    if out is None:
        out = torch.empty((b, sq, hq, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, dtype=torch.float32)
    _check(load().mla_sparse_paged_fwd(
        _ptr(q), _ptr(kv_cache), kv_cache.shape[0], kv_cache.shape[1], _ptr(block_table),
        block_table.shape[1], _ptr(seqlens_kv), _ptr(sparse_indices), sparse_indices.shape[-1],
        int(sparse_block_size), b, sq, hq, _scale(scale, q), int(sparse_mode), _ptr(sinks),
        _ptr(out), _ptr(lse), _stream()))
    return out, lse


def _cache_dtype(t, fmt):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype != torch.uint8:
        raise ValueError("caches must be bfloat16 or uint8 FP8 codes")
    return FP8_FORMATS[fmt]


def attn_debug_gather_paged(kernel, k_cache, v_cache, block_table, cache_seqlens, plan,
                            max_splits, dump_rows, fmt="e4m3"):
    """Rows staged in LDS by the decode kernel's own gather (test only):
    returns (k_rows, v_rows), each (B, dump_rows, Hkv, D) of the cache type
    (v_rows is None for the MLA kernel); rows past a sequence's length stay
    zero. kernel: ATTN_GATHER_DECODE or ATTN_GATHER_MLA."""
    _dev(k_cache, v_cache)
    _dev(block_table, cache_seqlens, plan, dtype=torch.int32)
    b = cache_seqlens.shape[0]
    _, page, hkv, d = k_cache.shape
    kd = torch.zeros((b, int(dump_rows), hkv, d), dtype=k_cache.dtype, device=k_cache.device)
    vd = None if kernel == ATTN_GATHER_MLA else torch.zeros_like(kd)
    _check(load().attn_debug_gather_paged(
        int(kernel), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), b, hkv, d, page, _cache_dtype(k_cache, fmt), _ptr(plan),
        int(max_splits), int(dump_rows), _ptr(kd), _ptr(vd), _stream()))
    return kd, vd


def attn_debug_gather_kvcache(k, v, cu_seqlens_q, cu_seqlens_k, k_cache, v_cache, block_table,
                              cache_seqlens, dump_rows, fmt="e4m3"):
    """Keys (cache rows, then current rows) staged by the cache-plus-current
    prefill's own gather (test only): (k_rows, v_rows), each (B, dump_rows,
    Hkv, D)."""
    _dev(k, v, k_cache, v_cache)
    _dev(cu_seqlens_q, cu_seqlens_k, block_table, cache_seqlens, dtype=torch.int32)
    b = cache_seqlens.shape[0]
    _, page, hkv, d = k_cache.shape
    kd = torch.zeros((b, int(dump_rows), hkv, d), dtype=k_cache.dtype, device=k_cache.device)
    vd = torch.zeros_like(kd)
    _check(load().attn_debug_gather_kvcache(
        _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens), page, b, hkv, d,
        _cache_dtype(k_cache, fmt), int(dump_rows), _ptr(kd), _ptr(vd), _stream()))
    return kd, vd


def attn_debug_gather_sparse(kv, sparse_indices, sparse_mode=3, block_table=None,
                             seqlens_kv=None, sparse_block_size=1):
    """Expanded key lists staged by the sparse MLA kernel's own gather (test
    only): (B, Sq, topk * sparse_block_size, 576) bf16; skipped keys hold row
    0 of the sequence (dense kv (B, Sk, 1, 576)) or of the pool (paged)."""
    _dev(kv, dtype=torch.bfloat16)
    _dev(sparse_indices, block_table, seqlens_kv, dtype=torch.int32)
    b, sq, _, topk = sparse_indices.shape
    rows = topk * int(sparse_block_size)
    dst = torch.zeros((b, sq, rows, kv.shape[-1]), dtype=kv.dtype, device=kv.device)
    paged = block_table is not None
    _check(load().attn_debug_gather_sparse(
        _ptr(kv), 0 if paged else kv.shape[1], _ptr(block_table),
        block_table.shape[1] if paged else 0, _ptr(seqlens_kv), kv.shape[1] if paged else 0,
        _ptr(sparse_indices), topk, int(sparse_block_size), b, sq, int(sparse_mode), rows,
        _ptr(dst), _stream()))
    return dst


# ------------------------------------------------------- composed decode calls
# The split planner sizes splits so that the decode grid holds about
# num_cu * waves workgroups. Plans as (max_splits, waves, min_blocks), tuned
# on MI355X for each decode shape; the composed calls below default to them,
# and the benchmark and the full-size parity tests use the same tuples.
GQA_DECODE_PLAN = (16, 8, 2)       # bf16 K and V tiles: 8 workgroups per CU
FP8_DECODE_PLAN = (16, 16, 2)      # FP8: two KV heads per workgroup, twice the splits
ONLY_QV_DECODE_PLAN = (16, 16, 2)  # V-only tiles: half the bytes, twice the workgroups
# bf16 at D = 64 with an even number of KV heads runs two KV heads per
# workgroup (128-byte head rows), so its plan doubles the splits as FP8's
GQA_D64_DECODE_PLAN = (16, 16, 2)
MLA_DECODE_PLAN = (4, 3, 8)        # 128-row MLA tiles: at most 4 splits, >= 8 pages each
GQA_ROWS_PER_WG = 16
MLA_ROWS_PER_WG = 128


def _num_cu(device):
    return attn_device_info(device.index if device.index is not None else 0)


def paged_decode(q, k_cache, v_cache, block_table, cache_seqlens, scale=None, causal=False,
                 sinks=None, max_splits=GQA_DECODE_PLAN[0], waves=None,
                 min_blocks=GQA_DECODE_PLAN[2], num_cu=None, out_dtype=torch.bfloat16,
                 mask=None):
    """plan -> attn_decode_paged (or attn_decode_paged_mask) -> attn_combine.
    Returns (out (B,Sq,Hq,Dv), lse (B,Hq,Sq), plan). waves defaults to the
    measured plan of the head dimension (GQA_DECODE_PLAN, or
    GQA_D64_DECODE_PLAN for D = 64 with an even number of KV heads)."""
    b, sq, hq, d = q.shape
    hkv = k_cache.shape[2]
    if waves is None:
        waves = (GQA_D64_DECODE_PLAN[1] if d == 64 and hkv % 2 == 0 else GQA_DECODE_PLAN[1])
    rows = sq * (hq // max(1, hkv))
    upb = hkv * ((rows + GQA_ROWS_PER_WG - 1) // GQA_ROWS_PER_WG)
    plan = attn_plan_splits(cache_seqlens, k_cache.shape[1], upb, num_cu or _num_cu(q.device),
                            waves, max_splits, min_blocks)
    op, lp = attn_decode_paged(q, k_cache, v_cache, block_table, cache_seqlens, plan, max_splits,
                               scale, causal, mask=mask)
    out, lse = attn_combine(op, lp, plan, b, sq, hq, max_splits, sinks, out_dtype)
    return out, lse, plan


def paged_decode_fp8(q, k_cache, v_cache, block_table, cache_seqlens, scale=None, fmt="e4m3",
                     q_descale=None, k_descale=None, v_descale=None, causal=False,
                     max_splits=FP8_DECODE_PLAN[0], waves=FP8_DECODE_PLAN[1],
                     min_blocks=FP8_DECODE_PLAN[2], num_cu=None):
    """plan -> attn_decode_paged_fp8 -> attn_combine (bfloat16 out). FP8 tiles
    are half the bytes of bf16 ones, so the default plan aims at twice as
    many workgroups per CU as paged_decode's (measured on MI355X)."""
    b, sq, hq, _ = q.shape
    hkv = k_cache.shape[2]
    rows = sq * (hq // max(1, hkv))
    upb = hkv * ((rows + GQA_ROWS_PER_WG - 1) // GQA_ROWS_PER_WG)
    plan = attn_plan_splits(cache_seqlens, k_cache.shape[1], upb, num_cu or _num_cu(q.device),
                            waves, max_splits, min_blocks)
    op, lp = attn_decode_paged_fp8(q, k_cache, v_cache, block_table, cache_seqlens, plan,
                                   max_splits, scale, fmt, q_descale, k_descale, v_descale,
                                   causal)
    out, lse = attn_combine(op, lp, plan, b, sq, hq, max_splits)
    return out, lse, plan


def paged_decode_qv(q, qv, k_cache, v_cache, block_table, cache_seqlens, scale=None, fmt=None,
                    q_descale=None, k_descale=None, v_descale=None, causal=False, only_qv=False,
                    max_splits=16, waves=None, min_blocks=2, num_cu=None):
    """plan -> attn_decode_paged_qv -> attn_combine (bfloat16 out). The plan
    defaults are the measured ones of each tile kind: paged_decode's for bf16
    K and V tiles, paged_decode_fp8's for FP8 tiles, and twice the workgroups
    per CU for the V-only tiles of only_qv (measured on MI355X)."""
    b, sq, hq, _ = qv.shape
    hkv = v_cache.shape[2]
    rows = sq * (hq // max(1, hkv))
    upb = hkv * ((rows + GQA_ROWS_PER_WG - 1) // GQA_ROWS_PER_WG)
    waves = waves or (ONLY_QV_DECODE_PLAN[1] if only_qv else
                      GQA_DECODE_PLAN[1] if fmt is None else FP8_DECODE_PLAN[1])
    plan = attn_plan_splits(cache_seqlens, v_cache.shape[1], upb, num_cu or _num_cu(qv.device),
                            waves, max_splits, min_blocks)
    op, lp = attn_decode_paged_qv(q, qv, k_cache, v_cache, block_table, cache_seqlens, plan,
                                  max_splits, scale, fmt, q_descale, k_descale, v_descale,
                                  causal, only_qv)
    out, lse = attn_combine(op, lp, plan, b, sq, hq, max_splits)
    return out, lse, plan


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, scale=None,
                              causal=False, sinks=None, max_splits=GQA_DECODE_PLAN[0],
                              waves=GQA_DECODE_PLAN[1], min_blocks=GQA_DECODE_PLAN[2],
                              num_cu=None, out=None, lse=None):
    """Plan, split decode and combine in one call with the plan and partials
    in the library's fixed scratch array (no allocation by the library; out
    and lse are allocated here only when not given). Returns (out (B,Sq,Hq,Dv)
    bf16, lse (B,Hq,Sq) fp32). v_cache is None for the MLA row (D = 576)."""
    _dev(q, k_cache, v_cache, dtype=torch.bfloat16)
    _dev(block_table, cache_seqlens, dtype=torch.int32)
    b, sq, hq, d = q.shape
    page, hkv = k_cache.shape[1], k_cache.shape[2]
    dv = 512 if v_cache is None and d == 576 else v_cache.shape[3]
    if out is None:
        out = torch.empty((b, sq, hq, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    _dev(out, dtype=torch.bfloat16)
    _dev(lse, sinks, dtype=torch.float32)
    _check(load().attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), b, sq, hq, hkv, d, dv, page, ATTN_BF16, _scale(scale, q),
        int(bool(causal)), _ptr(sinks), int(num_cu or _num_cu(q.device)), int(waves),
        int(max_splits), int(min_blocks), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def mla_decode(q, kv_cache, block_table, cache_seqlens, scale=None, causal=False,
               max_splits=MLA_DECODE_PLAN[0], waves=MLA_DECODE_PLAN[1],
               min_blocks=MLA_DECODE_PLAN[2], num_cu=None):
    """plan -> MLA decode -> attn_combine (dv = 512). kv_cache (P, page, Hkv,
    576): Hkv = 1 runs mla_decode_paged, Hkv > 1 attn_decode_paged with
    d = 576, dv = 512 (the same kernel)."""
    b, sq, hq, _ = q.shape
    hkv = kv_cache.shape[2]
    rows = sq * (hq // hkv)
    upb = hkv * ((rows + MLA_ROWS_PER_WG - 1) // MLA_ROWS_PER_WG)
    plan = attn_plan_splits(cache_seqlens, kv_cache.shape[1], upb, num_cu or _num_cu(q.device),
                            waves, max_splits, min_blocks)
    if hkv == 1:
        op, lp = mla_decode_paged(q, kv_cache, block_table, cache_seqlens, plan, max_splits,
                                  scale, causal)
    else:
        op, lp = attn_decode_paged(q, kv_cache, None, block_table, cache_seqlens, plan,
                                   max_splits, scale, causal)
    out, lse = attn_combine(op, lp, plan, b, sq, hq, max_splits)
    return out, lse, plan
