"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/attn.h, and rejects bad host arguments with the documented
status codes before any device work (so these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

from attention_attn_fwd_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    return B.load()


def test_header_lists_the_abi():
    names = declared()
    for n in ["attn_fwd_varlen", "attn_plan_words", "attn_plan_splits", "attn_decode_paged",
              "attn_combine", "mla_decode_paged", "attn_fwd_varlen_kvcache", "attn_decode_paged_fp8", "attn_fwd_varlen_fp8", "attn_decode_paged_qv", "attn_fwd_varlen_qv", "mla_sparse_paged_fwd", "mla_sparse_fwd", "attn_debug_gather_paged",
              "attn_debug_gather_kvcache", "attn_debug_gather_sparse",
              "attn_status_string", "attn_last_error", "attn_device_info"]:
        assert n in names


def test_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in declared():
        assert hasattr(raw, n), f"{n} not exported"
    assert sorted(B.exported_symbols()) == declared()


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ATTN_OK"
    assert lib.attn_status_string(3) == b"ATTN_EEMPTY"
    assert lib.attn_status_string(99) == b"ATTN_UNKNOWN"


P = 0x1000  # a non-null pointer value; never dereferenced by the host checks


def varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, batch=2, mq=8, mk=8, hq=4, hkv=2, d=128, dv=128, dtype=0,
             scale=0.1, causal=1, wl=-1, wr=-1, sinks=None, out=P, lse=None, stream=None)
    a.update(kw)
    return lib.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["batch"], a["mq"],
                               a["mk"], a["hq"], a["hkv"], a["d"], a["dv"], a["dtype"],
                               a["scale"], a["causal"], a["wl"], a["wr"], a["sinks"], a["out"],
                               a["lse"], a["stream"])


def test_varlen_host_checks(lib):
    assert varlen(lib, batch=0) == B.ATTN_EEMPTY
    assert varlen(lib, hq=0) == B.ATTN_EEMPTY
    assert varlen(lib, q=None) == B.ATTN_EINVAL
    assert varlen(lib, hq=6, hkv=4) == B.ATTN_EINVAL
    assert varlen(lib, wl=-2) == B.ATTN_EINVAL
    assert varlen(lib, scale=float("nan")) == B.ATTN_EINVAL
    assert varlen(lib, scale=0.0) == B.ATTN_EINVAL
    assert varlen(lib, scale=-0.1) == B.ATTN_EINVAL
    assert varlen(lib, d=96, dv=96) == B.ATTN_EUNSUPPORTED
    assert varlen(lib, d=128, dv=64) == B.ATTN_EUNSUPPORTED
    assert varlen(lib, dtype=7) == B.ATTN_EUNSUPPORTED
    assert b"dtype 7" in lib.attn_last_error()


def test_varlen_mask_host_checks(lib):
    def call(**kw):
        a = dict(q=P, k=P, v=P, cq=P, ck=P, batch=2, mq=8, mk=100, hq=4, hkv=2, d=128, dv=128,
                 scale=0.1, causal=1, wl=-1, wr=-1, mask=P, mh=1, mld=128)
        a.update(kw)
        return lib.attn_fwd_varlen_mask(
            a["q"], a["k"], a["v"], a["cq"], a["ck"], a["batch"], a["mq"], a["mk"], a["hq"],
            a["hkv"], a["d"], a["dv"], a["scale"], a["causal"], a["wl"], a["wr"], None,
            a["mask"], a["mh"], a["mld"], P, None, None)
    assert call(mask=None) == B.ATTN_EINVAL
    assert call(mh=3) == B.ATTN_EINVAL
    assert call(mld=100) == B.ATTN_EINVAL
    assert call(mk=200) == B.ATTN_EINVAL
    assert b"max_seqlen_k" in lib.attn_last_error()
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(hq=6, hkv=4) == B.ATTN_EINVAL
    assert call(d=96, dv=96) == B.ATTN_EUNSUPPORTED


def test_error_message_set(lib):
    assert varlen(lib, hq=6, hkv=4) == B.ATTN_EINVAL
    assert b"multiple" in lib.attn_last_error()


def test_varlen_kvcache_host_checks(lib):
    def call(**kw):
        a = dict(q=P, k=P, v=P, cq=P, ck=P, kc=P, vc=P, bt=P, mp=4, lens=P, page=64, batch=2,
                 mq=8, hq=8, hkv=2, d=128, dv=128, dtype=0, scale=0.1, causal=1, wl=-1, wr=-1,
                 mask=None, mh=0, mld=0)
        a.update(kw)
        return lib.attn_fwd_varlen_kvcache(
            a["q"], a["k"], a["v"], a["cq"], a["ck"], a["kc"], a["vc"], a["bt"], a["mp"],
            a["lens"], a["page"], a["batch"], a["mq"], a["hq"], a["hkv"], a["d"], a["dv"],
            a["dtype"], a["scale"], a["causal"], a["wl"], a["wr"], None, a["mask"], a["mh"],
            a["mld"], P, None, None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(mp=0) == B.ATTN_EEMPTY
    assert call(page=0) == B.ATTN_EEMPTY
    assert call(bt=None) == B.ATTN_EINVAL
    assert call(lens=None) == B.ATTN_EINVAL
    assert call(kc=None) == B.ATTN_EINVAL
    assert call(hq=6, hkv=4) == B.ATTN_EINVAL
    assert call(wr=-3) == B.ATTN_EINVAL
    assert call(dtype=1) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=128) == B.ATTN_EUNSUPPORTED
    assert call(d=96, dv=96) == B.ATTN_EUNSUPPORTED
    assert call(page=24) == B.ATTN_EUNSUPPORTED
    assert b"page_size" in lib.attn_last_error()
    assert call(mask=P, mh=3, mld=64) == B.ATTN_EINVAL
    assert call(mask=P, mh=1, mld=100) == B.ATTN_EINVAL


def test_plan_host_checks(lib):
    assert lib.attn_plan_words(4, 16) == 3 + 4 + 4 * 4 * 16
    assert lib.attn_plan_words(0, 16) == 0
    assert lib.attn_plan_splits(P, 0, 64, 1, 256, 4, 16, 4, P, None) == B.ATTN_EEMPTY
    assert lib.attn_plan_splits(P, 4, 64, 1, 256, 4, 17, 4, P, None) == B.ATTN_EINVAL
    assert lib.attn_plan_splits(P, 4, 64, 1, 256, 4, 0, 4, P, None) == B.ATTN_EINVAL
    assert lib.attn_plan_splits(None, 4, 64, 1, 256, 4, 16, 4, P, None) == B.ATTN_EINVAL
    assert lib.attn_plan_splits(P, 4, 0, 1, 256, 4, 16, 4, P, None) == B.ATTN_EINVAL


def test_decode_host_checks(lib):
    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, sq=1, hq=32, hkv=8, d=128, dv=128,
                 page=64, dtype=0, scale=0.1, causal=0, plan=P, ms=16, op=P, lp=P)
        a.update(kw)
        return lib.attn_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["mp"], a["lens"],
                                     a["batch"], a["sq"], a["hq"], a["hkv"], a["d"], a["dv"],
                                     a["page"], a["dtype"], a["scale"], a["causal"], a["plan"],
                                     a["ms"], a["op"], a["lp"], None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(mp=0) == B.ATTN_EEMPTY
    assert call(plan=None) == B.ATTN_EINVAL
    assert call(ms=17) == B.ATTN_EINVAL
    assert call(hq=12) == B.ATTN_EINVAL
    assert call(d=96, dv=96) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=128) == B.ATTN_EUNSUPPORTED
    assert call(dtype=1) == B.ATTN_EUNSUPPORTED
    assert call(page=24) == B.ATTN_EUNSUPPORTED
    # the MLA row (576 / 512) reads V from the key rows: v_cache NULL or k_cache
    assert call(d=576, dv=512, vc=P + 4096) == B.ATTN_EUNSUPPORTED
    assert b"v_cache" in lib.attn_last_error()
    assert call(d=576, dv=256, vc=None) == B.ATTN_EINVAL   # not the MLA shape: V required
    assert call(d=576, dv=512, vc=None, bt=None) == B.ATTN_EINVAL


def test_decode_mask_host_checks(lib):
    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, sq=1, hq=8, hkv=2, d=128, dv=128,
                 page=64, scale=0.1, causal=0, mask=P, mh=1, mld=128, plan=P, ms=4)
        a.update(kw)
        return lib.attn_decode_paged_mask(
            a["q"], a["kc"], a["vc"], a["bt"], a["mp"], a["lens"], a["batch"], a["sq"], a["hq"],
            a["hkv"], a["d"], a["dv"], a["page"], a["scale"], a["causal"], a["mask"], a["mh"],
            a["mld"], a["plan"], a["ms"], P, P, None)
    assert call(mask=None) == B.ATTN_EINVAL
    assert call(mh=3) == B.ATTN_EINVAL
    assert call(mld=96) == B.ATTN_EINVAL
    assert call(plan=None) == B.ATTN_EINVAL
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(d=576, dv=512, vc=None) == B.ATTN_EUNSUPPORTED
    assert b"decode mask" in lib.attn_last_error()
    assert call(d=96, dv=96) == B.ATTN_EUNSUPPORTED


def test_decode_fp8_host_checks(lib):
    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, sq=1, hq=32, hkv=8, d=128, dv=128,
                 page=64, fmt=B.ATTN_FP8_E4M3, scale=0.1, causal=0, plan=P, ms=16, op=P, lp=P)
        a.update(kw)
        return lib.attn_decode_paged_fp8(a["q"], a["kc"], a["vc"], a["bt"], a["mp"], a["lens"],
                                         a["batch"], a["sq"], a["hq"], a["hkv"], a["d"], a["dv"],
                                         a["page"], a["fmt"], None, None, None, a["scale"],
                                         a["causal"], a["plan"], a["ms"], a["op"], a["lp"], None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(plan=None) == B.ATTN_EINVAL
    assert call(hq=12) == B.ATTN_EINVAL
    assert call(scale=-1.0) == B.ATTN_EINVAL
    assert call(fmt=B.ATTN_BF16) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=64) == B.ATTN_EUNSUPPORTED
    assert call(page=24) == B.ATTN_EUNSUPPORTED
    assert b"fp8_format" in (call(fmt=7) and lib.attn_last_error())


def test_varlen_fp8_host_checks(lib):
    def call(**kw):
        a = dict(q=P, k=P, v=P, cq=P, ck=P, batch=2, mq=100, mk=100, hq=8, hkv=2, d=128, dv=128,
                 fmt=B.ATTN_FP8_E4M3, scale=0.1, causal=1, wl=-1, wr=-1, out=P)
        a.update(kw)
        return lib.attn_fwd_varlen_fp8(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["batch"],
                                       a["mq"], a["mk"], a["hq"], a["hkv"], a["d"], a["dv"],
                                       a["fmt"], None, None, None, a["scale"], a["causal"],
                                       a["wl"], a["wr"], None, a["out"], None, None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(mq=0) == B.ATTN_EEMPTY
    assert call(k=None) == B.ATTN_EINVAL
    assert call(hq=7) == B.ATTN_EINVAL
    assert call(wl=-2) == B.ATTN_EINVAL
    assert call(scale=0.0) == B.ATTN_EINVAL
    assert call(scale=float("nan")) == B.ATTN_EINVAL
    assert call(fmt=B.ATTN_F32) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=64) == B.ATTN_EUNSUPPORTED
    assert b"fp8_format" in (call(fmt=9) and lib.attn_last_error())


def test_decode_qv_host_checks(lib):
    def call(**kw):
        a = dict(q=P, qv=P, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, sq=1, hq=32, hkv=8, d=128,
                 dv=128, page=64, dtype=B.ATTN_BF16, qd=None, scale=0.1, causal=0, only=0,
                 plan=P, ms=16, op=P, lp=P)
        a.update(kw)
        return lib.attn_decode_paged_qv(a["q"], a["qv"], a["kc"], a["vc"], a["bt"], a["mp"],
                                        a["lens"], a["batch"], a["sq"], a["hq"], a["hkv"],
                                        a["d"], a["dv"], a["page"], a["dtype"], a["qd"], None,
                                        None, a["scale"], a["causal"], a["only"], a["plan"],
                                        a["ms"], a["op"], a["lp"], None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(qv=None) == B.ATTN_EINVAL
    assert call(q=None) == B.ATTN_EINVAL
    assert call(kc=None) == B.ATTN_EINVAL
    assert call(vc=None, only=1) == B.ATTN_EINVAL
    assert call(hq=12) == B.ATTN_EINVAL
    assert call(ms=17) == B.ATTN_EINVAL
    assert call(scale=-1.0) == B.ATTN_EINVAL
    assert call(qd=P) == B.ATTN_EINVAL          # descales with bf16 inputs
    assert call(dtype=B.ATTN_F32) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=64) == B.ATTN_EUNSUPPORTED
    assert call(page=24) == B.ATTN_EUNSUPPORTED


def test_varlen_qv_host_checks(lib):
    def call(**kw):
        a = dict(q=P, qv=P, k=P, v=P, cq=P, ck=P, batch=2, mq=100, mk=100, hq=8, hkv=2, d=128,
                 dv=128, dtype=B.ATTN_BF16, qd=None, scale=0.1, causal=1, wl=-1, wr=-1, only=0,
                 out=P)
        a.update(kw)
        return lib.attn_fwd_varlen_qv(a["q"], a["qv"], a["k"], a["v"], a["cq"], a["ck"],
                                      a["batch"], a["mq"], a["mk"], a["hq"], a["hkv"], a["d"],
                                      a["dv"], a["dtype"], a["qd"], None, None, a["scale"],
                                      a["causal"], a["wl"], a["wr"], None, a["only"], a["out"],
                                      None, None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(qv=None) == B.ATTN_EINVAL
    assert call(q=None) == B.ATTN_EINVAL
    assert call(k=None) == B.ATTN_EINVAL
    assert call(v=None, only=1) == B.ATTN_EINVAL
    assert call(hq=7) == B.ATTN_EINVAL
    assert call(wr=-3) == B.ATTN_EINVAL
    assert call(scale=0.0) == B.ATTN_EINVAL
    assert call(qd=P) == B.ATTN_EINVAL
    assert call(dtype=B.ATTN_F32) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=64) == B.ATTN_EUNSUPPORTED


def test_misaligned_tensors_rejected(lib):
    """Element tensors must be 16-byte aligned: an 8-byte offset is EINVAL
    before anything is enqueued."""
    M = P + 8
    assert lib.attn_fwd_varlen(P, M, P, P, P, 2, 100, 100, 8, 2, 128, 128, B.ATTN_BF16, 0.1, 1,
                               -1, -1, None, P, None, None) == B.ATTN_EINVAL
    assert b"aligned" in lib.attn_last_error()
    assert lib.attn_fwd_varlen_fp8(P, P, P, P, P, 2, 100, 100, 8, 2, 128, 128,
                                   B.ATTN_FP8_E4M3, None, None, None, 0.1, 1, -1, -1, None, M,
                                   None, None) == B.ATTN_EINVAL
    assert lib.attn_decode_paged(P, P, M, P, 4, P, 2, 1, 32, 8, 128, 128, 64, B.ATTN_BF16, 0.1,
                                 0, P, 16, P, P, None) == B.ATTN_EINVAL
    assert lib.attn_combine(M, P, P, 2, 1, 32, 128, 16, None, B.ATTN_BF16, P, None,
                            None) == B.ATTN_EINVAL
    assert lib.mla_sparse_fwd(P, M, P, 2048, 1, 4, 64, 64, 0.1, 3, None, P, None,
                              None) == B.ATTN_EINVAL


def test_mla_and_sparse_host_checks(lib):
    assert lib.mla_decode_paged(P, P, P, 4, P, 0, 1, 128, 64, 0.1, 0, P, 16, P, P,
                                None) == B.ATTN_EEMPTY
    assert lib.mla_decode_paged(P, P, P, 4, P, 2, 1, 120, 24, 0.1, 0, P, 16, P, P,
                                None) == B.ATTN_EUNSUPPORTED   # page not a multiple of 16
    assert lib.mla_decode_paged(P, P, P, 4, P, 2, 1, 128, 64, 0.1, 0, P, 0, P, P,
                                None) == B.ATTN_EINVAL
    assert lib.mla_sparse_fwd(P, P, P, 2048, 1, 1, 10, 64, 0.1, 1, None, P, None,
                              None) == B.ATTN_EINVAL
    assert lib.mla_sparse_fwd(P, P, P, 0, 1, 1, 10, 64, 0.1, 3, None, P, None,
                              None) == B.ATTN_EEMPTY
    assert lib.mla_sparse_fwd(None, P, P, 16, 1, 1, 10, 64, 0.1, 3, None, P, None,
                              None) == B.ATTN_EINVAL
    # per-sequence row byte offsets must fit 32 bits
    assert lib.mla_sparse_fwd(P, P, P, 16, 1, 1, 3728271, 64, 0.1, 0, None, P, None,
                              None) == B.ATTN_EUNSUPPORTED


def test_sparse_paged_host_checks(lib):
    def call(**kw):
        a = dict(q=P, kc=P, nb=100, page=64, bt=P, mp=4, lens=P, idx=P, topk=2048, bs=1, batch=2,
                 sq=4, hq=64, scale=0.1, mode=3)
        a.update(kw)
        return lib.mla_sparse_paged_fwd(a["q"], a["kc"], a["nb"], a["page"], a["bt"], a["mp"],
                                        a["lens"], a["idx"], a["topk"], a["bs"], a["batch"],
                                        a["sq"], a["hq"], a["scale"], a["mode"], None, P, None,
                                        None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(nb=0) == B.ATTN_EEMPTY
    assert call(bt=None) == B.ATTN_EINVAL
    assert call(mode=1) == B.ATTN_EINVAL
    assert call(bs=3) == B.ATTN_EINVAL
    assert call(bs=256) == B.ATTN_EINVAL
    assert call(hq=8) == B.ATTN_EUNSUPPORTED
    assert call(nb=60000, page=64) == B.ATTN_EUNSUPPORTED   # pool rows x 1152 B above 2^32


def test_combine_host_checks(lib):
    assert lib.attn_combine(P, P, P, 0, 1, 32, 128, 16, None, 0, P, None, None) == B.ATTN_EEMPTY
    assert lib.attn_combine(P, P, P, 2, 1, 32, 126, 16, None, 0, P, None, None) == \
        B.ATTN_EUNSUPPORTED
    assert lib.attn_combine(P, P, P, 2, 1, 32, 128, 16, None, 5, P, None, None) == \
        B.ATTN_EUNSUPPORTED
    assert lib.attn_combine(None, P, P, 2, 1, 32, 128, 16, None, 0, P, None, None) == \
        B.ATTN_EINVAL


def test_gather_host_checks(lib):
    def paged(**kw):
        a = dict(kernel=B.ATTN_GATHER_DECODE, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, hkv=2,
                 d=128, page=64, dtype=B.ATTN_BF16, plan=P, ms=16, rows=100, kd=P, vd=P)
        a.update(kw)
        return lib.attn_debug_gather_paged(a["kernel"], a["kc"], a["vc"], a["bt"], a["mp"],
                                           a["lens"], a["batch"], a["hkv"], a["d"], a["page"],
                                           a["dtype"], a["plan"], a["ms"], a["rows"], a["kd"],
                                           a["vd"], None)
    assert paged(kernel=5) == B.ATTN_EINVAL
    assert paged(batch=0) == B.ATTN_EEMPTY
    assert paged(rows=0) == B.ATTN_EEMPTY
    assert paged(vd=None) == B.ATTN_EINVAL
    assert paged(kernel=B.ATTN_GATHER_MLA, vc=None, vd=None) == B.ATTN_EUNSUPPORTED   # d != 576
    assert paged(d=96) == B.ATTN_EUNSUPPORTED
    assert paged(d=64, dtype=B.ATTN_FP8_E4M3) == B.ATTN_EUNSUPPORTED
    assert paged(page=24) == B.ATTN_EUNSUPPORTED
    assert paged(ms=17) == B.ATTN_EINVAL
    assert paged(kd=P + 8) == B.ATTN_EINVAL

    def kvc(**kw):
        a = dict(k=P, v=P, cq=P, ck=P, kc=P, vc=P, bt=P, mp=4, lens=P, page=64, batch=2, hkv=2,
                 d=128, dtype=B.ATTN_BF16, rows=100, kd=P, vd=P)
        a.update(kw)
        return lib.attn_debug_gather_kvcache(a["k"], a["v"], a["cq"], a["ck"], a["kc"], a["vc"],
                                             a["bt"], a["mp"], a["lens"], a["page"], a["batch"],
                                             a["hkv"], a["d"], a["dtype"], a["rows"], a["kd"],
                                             a["vd"], None)
    assert kvc(batch=0) == B.ATTN_EEMPTY
    assert kvc(bt=None) == B.ATTN_EINVAL
    assert kvc(d=64) == B.ATTN_EUNSUPPORTED
    assert kvc(dtype=B.ATTN_F32) == B.ATTN_EUNSUPPORTED

    def sparse(**kw):
        a = dict(kv=P, sk=1000, bt=None, mp=0, lens=None, page=0, idx=P, topk=64, bs=1, batch=2,
                 sq=4, mode=3, rows=64, dst=P)
        a.update(kw)
        return lib.attn_debug_gather_sparse(a["kv"], a["sk"], a["bt"], a["mp"], a["lens"],
                                            a["page"], a["idx"], a["topk"], a["bs"], a["batch"],
                                            a["sq"], a["mode"], a["rows"], a["dst"], None)
    assert sparse(topk=0) == B.ATTN_EEMPTY
    assert sparse(sk=0) == B.ATTN_EEMPTY
    assert sparse(bt=P) == B.ATTN_EINVAL          # paged pool without lengths and page size
    assert sparse(mode=1) == B.ATTN_EINVAL
    assert sparse(bs=3) == B.ATTN_EINVAL
    assert sparse(bs=2) == B.ATTN_EINVAL          # 128 keys do not fit 64 rows


def test_default_softmax_scale():
    # An omitted scale means 1/sqrt(head dim of the query that is scored).
    import math

    import torch
    q = torch.empty((3, 2, 128))
    assert B._scale(None, q) == pytest.approx(1.0 / math.sqrt(128))
    assert B._scale(0.25, q) == 0.25
    assert B._scale(None, torch.empty((1, 1, 1, 576))) == pytest.approx(1.0 / 24.0)


def test_varlen_kvcache_fp8_host_checks(lib):
    def call(**kw):
        a = dict(q=P, k=P, v=P, kc=P, vc=P, bt=P, mp=4, lens=P, page=64, batch=2, mq=100, hq=8,
                 hkv=2, d=128, dv=128, fmt=B.ATTN_FP8_E4M3, scale=0.1, wl=-1, wr=-1, out=P)
        a.update(kw)
        return lib.attn_fwd_varlen_kvcache_fp8(
            a["q"], a["k"], a["v"], P, P, a["kc"], a["vc"], a["bt"], a["mp"], a["lens"],
            a["page"], a["batch"], a["mq"], a["hq"], a["hkv"], a["d"], a["dv"], a["fmt"], None,
            None, None, a["scale"], 1, a["wl"], a["wr"], None, a["out"], None, None)
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(page=0) == B.ATTN_EEMPTY
    assert call(kc=None) == B.ATTN_EINVAL
    assert call(bt=None) == B.ATTN_EINVAL
    assert call(hq=7) == B.ATTN_EINVAL
    assert call(wr=-3) == B.ATTN_EINVAL
    assert call(scale=-1.0) == B.ATTN_EINVAL
    assert call(fmt=B.ATTN_BF16) == B.ATTN_EUNSUPPORTED
    assert call(d=64, dv=64) == B.ATTN_EUNSUPPORTED
    assert call(page=24) == B.ATTN_EUNSUPPORTED
    assert call(q=P + 8) == B.ATTN_EINVAL


def test_noalloc_host_checks(lib):
    def call(**kw):
        a = dict(q=P, kc=P, vc=P, bt=P, mp=4, lens=P, batch=2, sq=1, hq=32, hkv=8, d=128, dv=128,
                 page=64, dtype=0, scale=0.1, ncu=256, waves=8, ms=16, mb=2, out=P)
        a.update(kw)
        return lib.attn_decode_paged_noalloc(
            a["q"], a["kc"], a["vc"], a["bt"], a["mp"], a["lens"], a["batch"], a["sq"], a["hq"],
            a["hkv"], a["d"], a["dv"], a["page"], a["dtype"], a["scale"], 0, None, a["ncu"],
            a["waves"], a["ms"], a["mb"], a["out"], None, None)
    need = lib.attn_decode_paged_noalloc_bytes(64, 1, 32, 128, 16)
    assert 16 << 20 < need < 18 << 20          # the paged-decode workload fits
    assert lib.attn_decode_paged_noalloc_bytes(0, 1, 32, 128, 16) == 0
    assert call(batch=0) == B.ATTN_EEMPTY
    assert call(hq=12) == B.ATTN_EINVAL
    assert call(out=None) == B.ATTN_EINVAL
    assert call(waves=0) == B.ATTN_EINVAL
    assert call(ms=17) == B.ATTN_EINVAL
    assert call(d=96, dv=96) == B.ATTN_EUNSUPPORTED
    # 4096 x 16 splits x 32 rows x 128 floats: far above the fixed scratch
    assert call(batch=4096) == B.ATTN_EINVAL
    assert b"scratch" in lib.attn_last_error()


def test_build_debug_defines(monkeypatch):
    """ATTN_BUILD_DEFINES adds -D flags to every compile and accepts nothing else."""
    from attention_attn_fwd_02_amd import build
    monkeypatch.delenv("ATTN_BUILD_DEFINES", raising=False)
    assert build._defines() == []
    monkeypatch.setenv("ATTN_BUILD_DEFINES", "-DATTN_LDS_POISON=1")
    assert build._defines() == ["-DATTN_LDS_POISON=1"]
    monkeypatch.setenv("ATTN_BUILD_DEFINES", "-DATTN_LDS_POISON=1 -O0")
    with pytest.raises(ValueError):
        build._defines()
