"""CPU checks of the seeded input generators: every field of every problem
type has the element type and shape its consumers (kernels and oracle)
expect, and the generators are deterministic. A field shifted by a change to
a problem's dataclass shows up here rather than on the GPU."""
import numpy as np

from attention_attn_fwd_02_amd import inputs


def _check(arr, dtype, shape):
    assert isinstance(arr, np.ndarray), type(arr)
    assert arr.dtype == np.dtype(dtype), (arr.dtype, dtype)
    assert arr.shape == tuple(shape), (arr.shape, shape)


def test_varlen_fields():
    w = inputs.varlen(1, [3, 5], [4, 6], hq=4, hkv=2, d=64, with_sinks=True, with_qv=True)
    _check(w.q, np.uint16, (8, 4, 64))
    _check(w.k, np.uint16, (10, 2, 64))
    _check(w.v, np.uint16, (10, 2, 64))
    _check(w.qv, np.uint16, (8, 4, 64))
    _check(w.cu_seqlens_q, np.int32, (3,))
    _check(w.cu_seqlens_k, np.int32, (3,))
    _check(w.sinks, np.float32, (4,))
    assert w.dtype == "bf16" and w.causal and w.window == (-1, -1)


def test_varlen_kvcache_fields():
    w = inputs.varlen_kvcache(2, [3, 5], [3, 5], [40, 7], hq=4, hkv=2, d=64, page=16,
                              with_sinks=True)
    _check(w.q, np.uint16, (8, 4, 64))
    _check(w.k, np.uint16, (8, 2, 64))
    assert w.k_cache.dtype == np.uint16 and w.k_cache.shape[1:] == (16, 2, 64)
    assert w.v_cache.dtype == np.uint16 and w.v_cache.shape == w.k_cache.shape
    assert w.block_table.dtype == np.int32 and w.block_table.shape[0] == 2
    _check(w.cache_seqlens, np.int32, (2,))
    assert w.page_size == 16 and w.qv is None
    _check(w.sinks, np.float32, (4,))


def test_paged_fields():
    w = inputs.paged(3, [20, 70], sq=2, hq=4, hkv=2, d=64, page=16, with_sinks=True,
                     with_qv=True)
    _check(w.q, np.uint16, (2, 2, 4, 64))
    _check(w.qv, np.uint16, (2, 2, 4, 64))
    assert w.k_cache.dtype == np.uint16 and w.k_cache.shape[1:] == (16, 2, 64)
    assert w.block_table.dtype == np.int32
    _check(w.cache_seqlens, np.int32, (2,))
    assert w.page_size == 16 and w.dv == 64
    f = inputs.paged_fp8(4, [20, 70], "e5m2", sq=2, hq=4, hkv=2, page=16, with_qv=True)
    _check(f.q, np.uint8, (2, 2, 4, 128))
    _check(f.qv, np.uint8, (2, 2, 4, 128))
    assert f.k_cache.dtype == np.uint8 and f.v_cache.dtype == np.uint8
    for ds in (f.q_descale, f.k_descale, f.v_descale):
        _check(ds, np.float32, (2, 2))
    assert f.fmt == "e5m2" and f.block_table.dtype == np.int32


def test_varlen_fp8_fields():
    w = inputs.varlen_fp8(5, [3, 5], [4, 6], fmt="e4m3", hq=4, hkv=2, with_sinks=True,
                          with_qv=True)
    _check(w.q, np.uint8, (8, 4, 128))
    _check(w.k, np.uint8, (10, 2, 128))
    _check(w.qv, np.uint8, (8, 4, 128))
    for ds in (w.q_descale, w.k_descale, w.v_descale):
        _check(ds, np.float32, (2, 2))
    _check(w.sinks, np.float32, (4,))


def test_sparse_fields():
    w = inputs.sparse_paged(6, [100, 40], 3, 8, block_size=4, page=16, hq=16, spare_pages=1)
    assert w.q.dtype == np.uint16 and w.q.shape == (2, 3, 16, 576)
    assert w.kv_cache.dtype == np.uint16 and w.kv_cache.shape[1:] == (16, 1, 576)
    assert w.indices.dtype == np.int32 and w.indices.shape == (2, 3, 1, 8)
    assert w.block_table.dtype == np.int32 and w.seqlens_kv.dtype == np.int32
    assert w.block_size == 4 and w.page_size == 16 and w.dv == 512


def test_generators_are_deterministic():
    a = inputs.varlen_kvcache(7, [3], [3], [20], hq=4, hkv=2, d=64, page=16)
    b = inputs.varlen_kvcache(7, [3], [3], [20], hq=4, hkv=2, d=64, page=16)
    for name in ("q", "k", "v", "k_cache", "v_cache", "block_table"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
