"""Run-to-run determinism of the split decode + combine, the MLA decode and
both sparse MLA paths: two calls on the same inputs give bitwise identical O
and LSE. Every kernel has a fixed reduction order (no atomics; the combine
sums the splits of a row in split order), which these tests check.
[MindSpore Lite "lite_boost.layers.flash_attention" page: the `deterministic`
parameter asks for a reproducible result]"""
import pytest
import torch

from attention_attn_fwd_02_amd import binding as B
from attention_attn_fwd_02_amd import inputs
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu


def same(name, a, b):
    for x, y in zip(a, b):
        assert x.shape == y.shape and torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16
                                                  else x.view(torch.int32),
                                                  y.view(torch.int16) if y.dtype == torch.bfloat16
                                                  else y.view(torch.int32)), f"{name}: differs"
    log(f"[{name}] bitwise identical over two runs")


def test_paged_decode_deterministic():
    w = inputs.paged_decode()
    log("case determinism paged_decode")
    args = [dev(x) for x in (w.q, w.k_cache, w.v_cache, w.block_table, w.cache_seqlens)]
    r1 = B.paged_decode(*args, w.scale)
    r2 = B.paged_decode(*args, w.scale)
    torch.cuda.synchronize()
    same("paged_decode", r1[:2], r2[:2])


def test_paged_decode_fp8_deterministic():
    w = inputs.paged_decode_fp8()
    log("case determinism paged_decode_fp8")
    args = [dev(x) for x in (w.q, w.k_cache, w.v_cache, w.block_table, w.cache_seqlens)]
    ds = [dev(x) for x in (w.q_descale, w.k_descale, w.v_descale)]
    r1 = B.paged_decode_fp8(*args, w.scale, w.fmt, *ds)
    r2 = B.paged_decode_fp8(*args, w.scale, w.fmt, *ds)
    torch.cuda.synchronize()
    same("paged_decode_fp8", r1[:2], r2[:2])


def test_mla_decode_deterministic():
    w = inputs.mla_decode()
    log("case determinism mla_decode")
    args = [dev(x) for x in (w.q, w.k_cache, w.block_table, w.cache_seqlens)]
    r1 = B.mla_decode(*args, w.scale)
    r2 = B.mla_decode(*args, w.scale)
    torch.cuda.synchronize()
    same("mla_decode", r1[:2], r2[:2])


def test_mla_sparse_deterministic():
    s = inputs.sparse_mla(7300, batch=2, sq=256, sk=8192, hq=64, topk=2048)
    log("case determinism mla_sparse_fwd")
    args = [dev(x) for x in (s.q, s.kv, s.indices)]
    r1 = B.mla_sparse_fwd(*args, s.scale, 3, dev(s.sinks))
    r2 = B.mla_sparse_fwd(*args, s.scale, 3, dev(s.sinks))
    torch.cuda.synchronize()
    same("mla_sparse_fwd", r1, r2)


def test_mla_sparse_paged_deterministic():
    w = inputs.sparse_paged(7400, [8192, 3000], 128, 32, block_size=64, page=64, spare_pages=3)
    log("case determinism mla_sparse_paged_fwd")
    args = [dev(x) for x in (w.q, w.kv_cache, w.block_table, w.seqlens_kv, w.indices)]
    r1 = B.mla_sparse_paged_fwd(*args, w.scale, w.block_size, 3, dev(w.sinks))
    r2 = B.mla_sparse_paged_fwd(*args, w.scale, w.block_size, 3, dev(w.sinks))
    torch.cuda.synchronize()
    same("mla_sparse_paged_fwd", r1, r2)
