"""Benchmark of the fused attention forward on one MI355X.

Headline: varlen causal GQA prefill (8 sequences with lengths U[512, 4096],
Hq=32, Hkv=8, D=128, bf16), in attention TFLOP/s. One step = one
attn_fwd_varlen call over the whole packed batch (the single kernel of the
prefill path). The same JSON line carries the other workloads as
`secondary` entries: paged GQA decode (KV-read GB/s, step = plan + split
decode + combine) with a bf16 and with an FP8 cache, MLA-absorbed paged
decode, chunked prefill over a paged cache, sparse MLA with sinks and
block-sparse MLA over a paged cache, and their qv / FP8 / mask variants.

Inputs are seeded synthetic tensors already resident in HBM when timing
starts. Protocol per workload (time_steps): its step runs untimed for
--ramp-ms milliseconds (from idle the GPU takes about 40 ms of continuous
work to leave its low clocks), then W warm-up steps, then K timed steps,
each after an untimed 512 MiB read that evicts the Infinity Cache; every
step has its own pair of HIP events on the stream the kernels run on, and
`value` is the median. The same K steps run back to back without eviction
give the `warm` side figures.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill,...]
                [--no-cpu] [--no-secondary]
python bench.py --profile-summary DIR --workload KEY --bench-json FILE
                (no GPU work: writes profiles/<kernel>_<workload>.md from a
                rocprofv3 kernel trace and the bench line of the same run)
python bench.py --traffic-from FETCH_DIR WRITE_DIR [CLOCK_DIR] --workload KEY
                (no GPU work: writes the kernel's HBM-traffic record)
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (AMD published spec)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (AMD published spec)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA (AMD published spec)
PEAK_CLOCK_GHZ = 2.4        # the engine clock those peaks assume
# FP8 prefill: Q.K^T (half the flops) runs on FP8 MFMA, P.V on bf16 MFMA
PEAK_FP8_MIX_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)

METRIC = "attention TFLOP/s (varlen prefill) and KV-read GB/s (paged decode), 1 MI355X"
PREFILL_WORKLOAD = ("varlen causal GQA prefill: 8 sequences, lengths U[512,4096] packed with "
                    "cu_seqlens, Hq=32, Hkv=8, D=128, bf16 Q/K/V ~ N(0,1), scale 1/sqrt(128), "
                    "bf16 O + fp32 LSE (seed 1002)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


# ------------------------------------------------------------------- timing
RAMP_MS = [200.0]
EVICT_BYTES = 512 << 20   # more than the 256 MB Infinity Cache (MALL)
_EVICT = []


def ramp(fn, ms):
    """Untimed: runs fn back to back for about `ms` milliseconds (host clock,
    synchronising every 4 calls), at most 20000 calls."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms and n < 20000:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        n += 4


def _evictor():
    """A callable that reads a 512 MiB buffer (one reduction kernel writing 64
    floats). Reading it leaves the Infinity Cache full of the buffer's clean
    lines: the next step finds none of its inputs there, and the dirty lines
    of the step before (its outputs) are written back during this untimed
    read, not during the next step. A write of the buffer would leave up to
    256 MB of dirty lines whose write-back fell inside the next timed step."""
    import torch
    if not _EVICT:
        buf = torch.ones(EVICT_BYTES // 4, dtype=torch.float32, device="cuda").view(64, -1)
        out = torch.empty(64, dtype=torch.float32, device="cuda")
        _EVICT.append(lambda: torch.sum(buf, dim=1, out=out))
    return _EVICT[0]


def time_steps(fn, steps, warmup):
    """The timing protocol of every workload. Ramps the clocks (ramp), runs fn
    `warmup` times untimed, then times `steps` steps, each preceded on the same
    stream by an untimed 512 MiB read that evicts the Infinity Cache (see
    _evictor), so no step finds its inputs there from the step before. The
    evictions and the steps are enqueued back to back (one synchronisation
    before and after),
    so the GPU never idles between steps and its clocks stay where a
    continuous workload holds them. Each step is bracketed by its own pair of
    HIP events on the current stream (the stream every call is launched on).

    Returns dict(ms = median milliseconds per step (the reported figure),
    ms_mean = their mean, ms_warm = milliseconds per step of `steps` steps run
    back to back with no eviction, the inputs then partly served from the
    Infinity Cache)."""
    import torch
    ramp(fn, RAMP_MS[0])
    for _ in range(warmup):
        fn()
    evict = _evictor()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        evict()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return dict(ms=float(np.median(times)), ms_mean=float(np.mean(times)),
                ms_warm=start.elapsed_time(stop) / steps)


# ----------------------------------------------------------------- workloads
def prefill_flops(lens, hq=32, d=128):
    # 4*D per (query row, visible key): 2*D for QK^T and 2*D for P.V; a causal
    # row t sees t+1 keys.
    return sum(4.0 * d * hq * (int(L) * (int(L) + 1) / 2) for L in lens)


def chunk_flops(lq, lc, hq, d):
    # query t of a chunk sees the cache and the chunk's rows 0..t
    return sum(4.0 * d * hq * (int(n) * int(c) + int(n) * (int(n) + 1) / 2)
               for n, c in zip(lq, lc))


class Run:
    """One workload ready to time: step() is the whole user-visible step,
    kernel() its dominant kernel alone (the same callable for one-kernel
    steps); work / kernel_work are the algorithmic flops or bytes of one
    step / one kernel launch in the unit of the workload's metric."""

    def __init__(self, step, work, kernel=None, kernel_work=None, workload="", extra=None):
        self.step, self.work = step, work
        self.kernel = kernel or step
        self.kernel_work = work if kernel_work is None else kernel_work
        self.workload = workload
        self.extra = extra or {}


def run_prefill():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.varlen_prefill()
    lens = np.diff(w.cu_seqlens_q)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cq, ck = dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
    out = torch.empty((int(lens.sum()), 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((32, int(lens.sum())), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen(q, k, v, cq, ck, int(lens.max()), int(lens.max()), w.scale, True,
                          out=out, lse=lse)

    in_bytes = w.q.nbytes + w.k.nbytes + w.v.nbytes
    r = Run(step, prefill_flops(lens), workload=PREFILL_WORKLOAD,
            extra=dict(lens=lens.tolist(),
                       algorithmic_bytes_per_launch=in_bytes + out.numel() * 2 + lse.numel() * 4))
    r.w = w
    return r


def run_tiny():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.tiny_dense()
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cq, ck = dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
    out = torch.empty_like(q)
    lse = torch.empty((w.q.shape[1], w.q.shape[0]), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen(q, k, v, cq, ck, 128, 128, w.scale, False, out=out, lse=lse)

    return Run(step, 4.0 * 64 * 4 * 128 * 128,
               workload="B=1, Sq=Sk=128, Hq=Hkv=4, D=64, fp32 Q/K/V ~ N(0,1), non-causal, scale "
                        "1/8, O and LSE out (seed 1001)")


def run_prefill_fp8():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.varlen_prefill_fp8()
    lens = np.diff(w.cu_seqlens_q)
    t = dict(q=dev(w.q), k=dev(w.k), v=dev(w.v), cq=dev(w.cu_seqlens_q), ck=dev(w.cu_seqlens_k),
             qd=dev(w.q_descale), kd=dev(w.k_descale), vd=dev(w.v_descale))
    hq, d = w.q.shape[1], w.q.shape[2]
    out = torch.empty((int(lens.sum()), hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, int(lens.sum())), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen_fp8(t["q"], t["k"], t["v"], t["cq"], t["ck"], int(lens.max()),
                              int(lens.max()), w.scale, w.fmt, t["qd"], t["kd"], t["vd"],
                              causal=True, out=out, lse=lse)

    return Run(step, prefill_flops(lens, hq, d),
               workload="varlen causal GQA prefill: 8 sequences U[512,4096] (drawn "
                        f"{lens.tolist()}), Hq=32, Hkv=8, D=128, e4m3 codes with per-(sequence, "
                        "KV head) descales, bf16 out (seed 1009)")


def run_prefill_qv():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.varlen_prefill()
    qvh = inputs.varlen_prefill_qv(w)
    lens = np.diff(w.cu_seqlens_q)
    q, qv, k, v = dev(w.q), dev(qvh), dev(w.k), dev(w.v)
    cq, ck = dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
    hq, d = w.q.shape[1], w.q.shape[2]
    out = torch.empty((int(lens.sum()), hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, int(lens.sum())), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen_qv(q, qv, k, v, cq, ck, int(lens.max()), int(lens.max()), w.scale,
                             causal=True, out=out, lse=lse)

    # q.k, qv.v and p.v: 6 D flop per visible (row, key) pair
    return Run(step, prefill_flops(lens, hq, d) * 6 / 4,
               workload="the varlen causal GQA prefill workload (seed 1002) with a bf16 qv "
                        "(T,32,128) N(0,1) (seed 1011); scores q.k + qv.v; 6 D flop per visible "
                        "(row, key) pair")


def _decode_buffers(b, sq, hq, dv, ms):
    import torch
    op = torch.empty((b * ms, sq * hq, dv), dtype=torch.float32, device="cuda")
    lp = torch.empty((b * ms, sq * hq), dtype=torch.float32, device="cuda")
    out = torch.empty((b, sq, hq, dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")
    return op, lp, out, lse


def run_decode():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.paged_decode()
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    bt, lens = dev(w.block_table), dev(w.cache_seqlens)
    ncu = B.attn_device_info(0)
    b, sq, hq, d = w.q.shape
    hkv = w.k_cache.shape[2]
    ms_, waves, mb = B.GQA_DECODE_PLAN
    upb = hkv * ((sq * hq // hkv + 15) // 16)
    plan = B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb)
    op, lp, out, lse = _decode_buffers(b, sq, hq, 128, ms_)

    def kernel():
        B.attn_decode_paged(q, kc, vc, bt, lens, plan, ms_, w.scale, False, op, lp)

    def step():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        kernel()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 + 128) * 2
    alg = kv_bytes + w.q.nbytes + out.numel() * 2 + lse.numel() * 4 + nblk * 4
    splits = int(plan[0].item())
    return Run(step, alg, kernel,
               workload="paged GQA decode: batch 64, 1 query token, cache_seqlens U[1024,32768], "
                        "page 64, Hq=32, Hkv=8, D=128, bf16; plan + split decode (<=16 splits) + "
                        f"combine per step; {splits} splits (seed 1003)",
               extra=dict(splits=splits, plan=list(B.GQA_DECODE_PLAN)))


def run_decode_fp8():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.paged_decode_fp8()
    q, kc, vc = dev(w.q), dev(w.k_cache), dev(w.v_cache)
    qd, kd, vd = dev(w.q_descale), dev(w.k_descale), dev(w.v_descale)
    bt, lens = dev(w.block_table), dev(w.cache_seqlens)
    ncu = B.attn_device_info(0)
    b, sq, hq, d = w.q.shape
    hkv = w.k_cache.shape[2]
    ms_, waves, mb = B.FP8_DECODE_PLAN
    upb = hkv * ((sq * hq // hkv + 15) // 16)
    plan = B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb)
    op, lp, out, lse = _decode_buffers(b, sq, hq, 128, ms_)

    def kernel():
        B.attn_decode_paged_fp8(q, kc, vc, bt, lens, plan, ms_, w.scale, w.fmt, qd, kd, vd,
                                False, op, lp)

    def step():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        kernel()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 + 128)               # one byte per code
    alg = (kv_bytes + w.q.nbytes + out.numel() * 2 + lse.numel() * 4 + nblk * 4
           + 3 * b * hkv * 4)
    splits = int(plan[0].item())
    return Run(step, alg, kernel,
               workload="paged GQA decode with an FP8 cache: batch 64, 1 query token, "
                        "cache_seqlens U[1024,32768], page 64, Hq=32, Hkv=8, D=128, e4m3 codes "
                        "with per-(batch, KV head) descales, bf16 out; plan + split decode "
                        f"(<=16 splits) + combine per step; {splits} splits (seed 1007)",
               extra=dict(splits=splits, plan=list(B.FP8_DECODE_PLAN),
                          cached_tokens=total_len))


def _run_decode_qv(only_qv):
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.paged_decode()
    qvh = inputs.paged_decode_qv(w)
    q, qv, kc, vc = dev(w.q), dev(qvh), dev(w.k_cache), dev(w.v_cache)
    bt, lens = dev(w.block_table), dev(w.cache_seqlens)
    ncu = B.attn_device_info(0)
    b, sq, hq, d = w.q.shape
    hkv = w.k_cache.shape[2]
    # V-only tiles are half the bytes: twice the workgroups per CU
    ms_, waves, mb = B.ONLY_QV_DECODE_PLAN if only_qv else B.GQA_DECODE_PLAN
    upb = hkv * ((sq * hq // hkv + 15) // 16)
    plan = B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb)
    op, lp, out, lse = _decode_buffers(b, sq, hq, 128, ms_)
    qq, kk = (None, None) if only_qv else (q, kc)

    def kernel():
        B.attn_decode_paged_qv(qq, qv, kk, vc, bt, lens, plan, ms_, w.scale, None, causal=False,
                               only_qv=only_qv, o_partial=op, lse_partial=lp)

    def step():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        kernel()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 if only_qv else 256) * 2   # V only with only_qv
    alg = (kv_bytes + qvh.nbytes + (0 if only_qv else w.q.nbytes) + out.numel() * 2 +
           lse.numel() * 4 + nblk * 4)
    what = ("qv alone (only_qv: V read, K not)" if only_qv
            else "q . k + qv . v scores (K and V read)")
    splits = int(plan[0].item())
    return Run(step, alg, kernel,
               workload="the paged GQA decode workload (seed 1003) with a bf16 qv (B,1,32,128) "
                        f"N(0,1) (seed 1010); {what}; plan + split decode + combine; {splits} "
                        "splits",
               extra=dict(splits=splits))


def run_decode_qv():
    return _run_decode_qv(False)


def run_decode_only_qv():
    return _run_decode_qv(True)


def run_mla():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.mla_decode()
    q, kc = dev(w.q), dev(w.k_cache)
    bt, lens = dev(w.block_table), dev(w.cache_seqlens)
    ncu = B.attn_device_info(0)
    b, sq, hq, d = w.q.shape
    ms_, waves, mb = B.MLA_DECODE_PLAN
    upb = (sq * hq + B.MLA_ROWS_PER_WG - 1) // B.MLA_ROWS_PER_WG
    plan = B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb)
    op, lp, out, lse = _decode_buffers(b, sq, hq, 512, ms_)

    def kernel():
        B.mla_decode_paged(q, kc, bt, lens, plan, ms_, w.scale, False, op, lp)

    def step():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        kernel()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    flops = total_len * sq * hq * 2.0 * (576 + 512)
    alg_bytes = total_len * 1152 + w.q.nbytes + out.numel() * 2 + lse.numel() * 4
    splits = int(plan[0].item())
    return Run(step, flops, kernel,
               workload="MLA-absorbed paged decode: batch 64, 2 query tokens, Hq=128, Hkv=1, "
                        "D=576 (V = first 512), page 64, cache_seqlens U[2048,16384], bf16; plan "
                        f"+ split decode + combine; {splits} splits (seed 1004)",
               extra=dict(splits=splits, plan=list(B.MLA_DECODE_PLAN), alg_bytes=alg_bytes))


def run_chunked(with_mask=False):
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.chunked_prefill()
    lq = np.diff(w.cu_seqlens_q)
    lc = w.cache_seqlens.astype(np.int64)
    t = dict(q=dev(w.q), k=dev(w.k), v=dev(w.v), cq=dev(w.cu_seqlens_q), ck=dev(w.cu_seqlens_k),
             kc=dev(w.k_cache), vc=dev(w.v_cache), bt=dev(w.block_table),
             lens=dev(w.cache_seqlens))
    hq, d = w.q.shape[1], w.q.shape[2]
    out = torch.empty((int(lq.sum()), hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, int(lq.sum())), dtype=torch.float32, device="cuda")
    mask = None
    if with_mask:
        # one shared bf16 mask over every key of every row: N(0,1) values
        ld = ((int((lq + lc).max()) + 63) // 64) * 64
        mask = dev(inputs.chunked_mask(int(lq.sum()), ld))

    def step():
        B.attn_fwd_varlen_kvcache(t["q"], t["k"], t["v"], t["cq"], t["ck"], t["kc"], t["vc"],
                                  t["bt"], t["lens"], int(lq.max()), w.scale, True, out=out,
                                  lse=lse, mask=mask)

    if with_mask:
        text = ("the chunked-prefill workload (seed 1006) with one bf16 additive mask shared by "
                "all heads, N(0,1) over every (row, key), streamed beside K/V")
    else:
        text = ("chunked causal GQA prefill: 8 sequences, 1024 new tokens each after a paged "
                f"cache of U[1024,8192] tokens (drawn {lc.tolist()}), page 64, Hq=32, Hkv=8, "
                "D=128, bf16; attn_fwd_varlen_kvcache (seed 1006)")
    return Run(step, chunk_flops(lq, lc, hq, d), workload=text)


def run_chunked_mask():
    return run_chunked(True)


def run_chunked_fp8():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.chunked_prefill_fp8()
    lq = np.diff(w.cu_seqlens_q)
    lc = w.cache_seqlens.astype(np.int64)
    t = [dev(x) for x in (w.q, w.k, w.v, w.cu_seqlens_q, w.cu_seqlens_k, w.k_cache, w.v_cache,
                          w.block_table, w.cache_seqlens)]
    ds = [dev(x) for x in (w.q_descale, w.k_descale, w.v_descale)]
    hq, d = w.q.shape[1], w.q.shape[2]
    out = torch.empty((int(lq.sum()), hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, int(lq.sum())), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen_kvcache_fp8(*t, int(lq.max()), w.scale, w.fmt, *ds, causal=True,
                                      out=out, lse=lse)

    return Run(step, chunk_flops(lq, lc, hq, d),
               workload="the chunked-prefill shape (8 sequences, 1024 new tokens each after a "
                        f"paged cache of U[1024,8192] tokens (drawn {lc.tolist()}), page 64, "
                        "Hq=32, Hkv=8, D=128) on e4m3 codes with per-(sequence, KV head) "
                        "descales, bf16 out; attn_fwd_varlen_kvcache_fp8 (seed 1012)")


def run_sparse():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    s = inputs.sparse_mla()
    q, kv, idx, sinks = dev(s.q), dev(s.kv), dev(s.indices), dev(s.sinks)
    b, sq, hq, d = s.q.shape
    out = torch.empty((b, sq, hq, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")

    def step():
        B.mla_sparse_fwd(q, kv, idx, s.scale, 3, sinks, out, lse)

    valid = int((s.indices >= 0).sum())     # every drawn index lies in its causal prefix
    return Run(step, valid * hq * 2.0 * (576 + 512),
               workload="top-2048 sparse MLA with per-head sinks: 4 x 4096 query tokens, 32768 "
                        "keys, Hq=64, D=576 (V = first 512), bf16 (seed 1005)",
               extra=dict(gathered_bytes=valid * 1152))


def run_sparse_paged():
    import torch
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.sparse_paged_blocks()
    q, kc, bt = dev(w.q), dev(w.kv_cache), dev(w.block_table)
    lens, idx, sinks = dev(w.seqlens_kv), dev(w.indices), dev(w.sinks)
    b, sq, hq, d = w.q.shape
    out = torch.empty((b, sq, hq, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")

    def step():
        B.mla_sparse_paged_fwd(q, kc, bt, lens, idx, w.scale, w.block_size, 3, sinks, out, lse)

    # every drawn block lies in its token's causal prefix; count its keys there
    valid = 0
    for bi in range(b):
        lk = int(w.seqlens_kv[bi])
        lim = lk - sq + np.arange(sq)                                   # last visible key
        blk = w.indices[bi, :, 0, :].astype(np.int64)
        n = np.clip(lim[:, None] - blk * w.block_size + 1, 0, w.block_size)
        valid += int(np.where(blk >= 0, n, 0).sum())
    return Run(step, valid * hq * 2.0 * (576 + 512),
               workload="block-sparse MLA over a paged latent cache: 4 x 4096 query tokens, 32768 "
                        "keys per sequence in pages of 64, 32 blocks of 64 keys per token "
                        "(sparse_block_size 64), Hq=64, D=576 (V = first 512), sinks, bf16 "
                        "(seed 1008)",
               extra=dict(gathered_bytes=valid * 1152))


PREFILL_SRC = ("kernels_prefill.hip", "prefill_bf16.h", "attn_core.h", "paged.h",
               "device_common.h", "launch.h")
DECODE_SRC = ("kernels_decode.hip", "attn_core.h", "attn_wide.h", "prefill_bf16.h", "paged.h",
              "device_common.h", "launch.h")
TF, GB = "TFLOP/s", "GB/s"

# key: (runner, metric, unit, bound, peak, kernel base name, profile stem, kernel sources,
#       divisor of the step counts for the slowest workloads)
WORKLOADS = {
    "prefill": (run_prefill, METRIC, TF, "mfma", PEAK_BF16_TFLOPS, "k_varlen_bf16",
                "k_varlen_bf16_d128_varlen_prefill", PREFILL_SRC, 1),
    "tiny": (run_tiny, "latency of one call (tiny dense attention, fp32)", "us", "latency", None,
             "k_varlen_f32", "k_varlen_f32_d64_tiny_dense", PREFILL_SRC, 1),
    "prefill_fp8": (run_prefill_fp8, "attention TFLOP/s (varlen prefill, FP8 e4m3 Q/K/V)", TF,
                    "mfma", PEAK_FP8_MIX_TFLOPS, "k_varlen_fp8",
                    "k_varlen_fp8_d128_varlen_prefill", PREFILL_SRC, 1),
    "prefill_qv": (run_prefill_qv, "attention TFLOP/s (varlen prefill with qv)", TF, "mfma",
                   PEAK_BF16_TFLOPS, "k_varlen_qv", "k_varlen_qv_d128_varlen_prefill",
                   PREFILL_SRC, 1),
    "decode": (run_decode, "KV-read GB/s (paged decode)", GB, "hbm", PEAK_HBM_GBS, "k_decode",
               "k_decode_gqa_paged_decode", DECODE_SRC, 1),
    "decode_fp8": (run_decode_fp8, "KV-read GB/s (paged decode, FP8 e4m3 Q/K/V)", GB, "hbm",
                   PEAK_HBM_GBS, "k_decode", "k_decode_gqa_fp8_paged_decode", DECODE_SRC, 1),
    "decode_qv": (run_decode_qv, "KV-read GB/s (paged decode, qv)", GB, "hbm", PEAK_HBM_GBS,
                  "k_decode", "k_decode_gqa_qv_paged_decode", DECODE_SRC, 1),
    "decode_only_qv": (run_decode_only_qv, "KV-read GB/s (paged decode, only_qv)", GB, "hbm",
                       PEAK_HBM_GBS, "k_decode", "k_decode_gqa_only_qv_paged_decode", DECODE_SRC,
                       1),
    "mla": (run_mla, "MLA paged decode TFLOP/s", TF, "mfma", PEAK_BF16_TFLOPS, "k_decode_wide",
            "k_decode_wide_mla_decode", DECODE_SRC, 1),
    "chunked": (run_chunked, "chunked prefill TFLOP/s (cache + new K/V)", TF, "mfma",
                PEAK_BF16_TFLOPS, "k_varlen_bf16", "k_varlen_bf16_kvcache_chunked_prefill",
                PREFILL_SRC, 1),
    "chunked_mask": (run_chunked_mask, "chunked prefill TFLOP/s (cache + new K/V, additive mask)",
                     TF, "mfma", PEAK_BF16_TFLOPS, "k_varlen_bf16",
                     "k_varlen_bf16_kvcache_mask_chunked_prefill", PREFILL_SRC, 1),
    "chunked_fp8": (run_chunked_fp8, "chunked prefill TFLOP/s (cache + new K/V, FP8 e4m3 Q/K/V)",
                    TF, "mfma", PEAK_FP8_MIX_TFLOPS, "k_varlen_fp8_kvc",
                    "k_varlen_fp8_kvcache_chunked_prefill", PREFILL_SRC, 1),
    "sparse": (run_sparse, "sparse MLA + sink TFLOP/s", TF, "mfma", PEAK_BF16_TFLOPS, "k_sparse",
               "k_sparse_sparse_mla", DECODE_SRC, 4),
    "sparse_paged": (run_sparse_paged, "block-sparse paged MLA + sink TFLOP/s", TF, "mfma",
                     PEAK_BF16_TFLOPS, "k_sparse", "k_sparse_paged_block_sparse_mla", DECODE_SRC,
                     4),
}
PEAK_NOTES = {
    "prefill_fp8": "half the flops (Q.K^T) on FP8 MFMA (5033 TFLOP/s), half (P.V) on bf16 MFMA "
                   "(2517 TFLOP/s): the harmonic mix",
    "chunked_fp8": "Q.K^T on FP8 MFMA, P.V on bf16 MFMA: the harmonic mix",
}


# ------------------------------------------- counter records and trace summaries
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read and 1 GiB written
COPY_KERNEL_TAG = "neg"       # torch.neg(src, out=dst) runs one elementwise kernel
N_XCD, N_SIMD = 8, 1024       # MI355X: GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs


def traffic_path(key):
    return os.path.join(ROOT, "profiles", WORKLOADS[key][6] + "_traffic.txt")


def source_digest(key):
    """Digest of the sources and compile flags of the workload's kernel."""
    from attention_attn_fwd_02_amd import build
    h = hashlib.sha256()
    for name in WORKLOADS[key][7]:
        with open(os.path.join(build.CSRC, name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()[:16]


def counter_record(key):
    """The committed counter record of the workload's kernel, or None when it
    does not match the current sources of that kernel."""
    try:
        with open(traffic_path(key)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_digest(key):
        return None
    return rec


def base_name(full):
    """k_decode from 'void attn::(anonymous namespace)::k_decode<...>(...)'."""
    head = full.replace("(anonymous namespace)::", "").split("<")[0].split("(")[0]
    return head.split("::")[-1].split(" ")[-1]


def _csv_rows(d, pattern):
    for fn in glob.glob(os.path.join(d, "**", pattern), recursive=True):
        with open(fn) as f:
            yield from csv.DictReader(f)


def _kernel_dispatches(d, kernel):
    """Per-dispatch counter values of the named kernel (exact base name) in a
    rocprofv3 --pmc output folder: {dispatch id: {counter: value, 'dur': s}}."""
    out = {}
    for r in _csv_rows(d, "*counter_collection.csv"):
        if base_name(r["Kernel_Name"]) != kernel:
            continue
        e = out.setdefault(int(r["Dispatch_Id"]), {})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp"):
            e["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    return out


def write_traffic(key, fetch_dir, write_dir, command, clock_dir=None):
    """Builds the counter record of the workload's kernel from two rocprofv3
    --pmc runs of `bench.py --only KEY --no-secondary --no-cpu
    --copy-calibration` (FETCH_SIZE, then WRITE_SIZE, both KiB per dispatch)
    and optionally the engine clock and MFMA busy fraction from a third
    (GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES with --kernel-trace)."""
    kernel = WORKLOADS[key][5]

    def one(d, counter):
        copy = [float(r["Counter_Value"]) for r in _csv_rows(d, "*counter_collection.csv")
                if r["Counter_Name"] == counter and COPY_KERNEL_TAG in r["Kernel_Name"]
                and "attn" not in r["Kernel_Name"]]
        ker = [e[counter] for e in _kernel_dispatches(d, kernel).values() if counter in e]
        if len(copy) != 1 or not ker:
            raise SystemExit(f"{d}: expected one calibration copy and {kernel} dispatches, got "
                             f"{len(copy)} and {len(ker)}")
        return copy[0], sum(ker) / len(ker), len(ker)

    copy_f, k_f_kib, n_f = one(fetch_dir, "FETCH_SIZE")
    copy_w, k_w_kib, n_w = one(write_dir, "WRITE_SIZE")
    f_f = COPY_BYTES / (copy_f * 1024)
    f_w = COPY_BYTES / (copy_w * 1024)
    rec = {
        "kernel": kernel, "workload": key,
        "bytes_per_launch": k_f_kib * 1024 * f_f + k_w_kib * 1024 * f_w,
        "fetch_kib_per_launch": k_f_kib, "write_kib_per_launch": k_w_kib,
        "dispatches": [n_f, n_w],
        "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_f,
                        "copy_write_kib": copy_w, "fetch_factor": f_f, "write_factor": f_w},
        "source_sha256_16": source_digest(key),
        "command": command,
    }
    if clock_dir:
        d = _kernel_dispatches(clock_dir, kernel)
        ids = [i for i in sorted(d) if "GRBM_GUI_ACTIVE" in d[i] and "dur" in d[i]]
        timed = ids[len(ids) // 2:]   # the later half: after the clock ramp
        ghz = statistics.median(d[i]["GRBM_GUI_ACTIVE"] / N_XCD / d[i]["dur"] / 1e9
                                for i in timed)
        rec["clock"] = {"ghz_median": ghz, "dispatches": len(timed)}
        if all("SQ_VALU_MFMA_BUSY_CYCLES" in d[i] for i in timed):
            rec["clock"]["mfma_busy_frac_median"] = statistics.median(
                d[i]["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / (d[i]["GRBM_GUI_ACTIVE"] / N_XCD)
                for i in timed)
    with open(traffic_path(key), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def profile_summary(key, trace_dir, bench_json, command):
    """Writes profiles/<stem>.md: the per-kernel statistics of a rocprofv3
    --kernel-trace run of `bench.py --only KEY --no-secondary --no-cpu`,
    kernels grouped by their exact instance name, next to the bench line of
    the same run."""
    stats = {}
    for r in _csv_rows(trace_dir, "*kernel_trace.csv"):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        stats.setdefault(r["Kernel_Name"], []).append(dur)
    if not stats:
        raise SystemExit(f"no kernel trace in {trace_dir}")
    main_kernel = WORKLOADS[key][5]
    with open(bench_json) as f:
        line = json.loads([ln for ln in f if ln.startswith("{")][-1])
    ent = next(e for e in [line] + line["secondary"] if e.get("key") == key)
    workload = ent["workload"] if "workload" in ent else ent["config"]["workload"]
    rows = sorted(stats.items(), key=lambda kv: -sum(kv[1]))
    out = [f"# rocprofv3 kernel trace: {main_kernel} ({key})", "",
           f"Workload: {workload}", "",
           "Command (from the repository root on the MI355X box):", "", "    " + command, "",
           "Kernels are grouped by their full instance name (exact match). bench.py runs, per "
           "workload, 200 ms of untimed steps to raise the clocks, the warm-up steps, the timed "
           "steps (each after an untimed 512 MiB Infinity-Cache eviction read) and as many "
           "back to back; the profiler averages every launch.", "",
           "| Kernel | Calls | Avg (us) | Median (us) | Min (us) | Max (us) |",
           "|---|---|---|---|---|---|"]
    for name, d in rows:
        short = name.replace("attn::(anonymous namespace)::", "").replace("attn::", "")
        short = short.replace("void ", "")[:160]
        mark = " **(main)**" if base_name(name) == main_kernel else ""
        out.append(f"| `{short}`{mark} | {len(d)} | {np.mean(d):.1f} | {np.median(d):.1f} | "
                   f"{min(d):.1f} | {max(d):.1f} |")
    rf = ent["roofline"]
    if rf["achieved"] is None:     # latency workload
        out += ["", f"bench.py, same run: {ent['value']:.1f} us per call (median, evicted "
                    f"cache); {ent['warm']['value']:.1f} us back to back."]
    else:
        out += ["", f"bench.py, same run: {ent['ms_per_step']:.4f} ms per step (median, evicted "
                    f"cache) = {ent['value']:.1f} {ent['unit']}; main kernel "
                    f"{rf.get('kernel_ms', ent['ms_per_step']):.4f} ms = {rf['achieved']:.1f} "
                    f"{rf['unit']} ({100 * rf['frac']:.1f} % of {rf['peak']:.0f})."]
    path = os.path.join(ROOT, "profiles", WORKLOADS[key][6] + ".md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)


def counters_summary(key, dirs, command):
    """Writes profiles/<stem>_counters.md: per-dispatch medians of every counter
    in rocprofv3 --pmc folders of `bench.py --only KEY --no-secondary --no-cpu`
    runs (one counter set per folder), for the workload's main kernel (exact
    base name; the later half of its dispatches, after the clock ramp), with
    the fractions they imply. SQ cycle counters share one unit, so their
    ratios need no scaling; GRBM_GUI_ACTIVE sums the 8 XCDs' engine cycles."""
    kernel = WORKLOADS[key][5]
    vals = {}
    for d in dirs:
        disp = _kernel_dispatches(d, kernel)
        ids = sorted(disp)
        for i in ids[len(ids) // 2:]:
            for c, v in disp[i].items():
                if c != "dur":
                    vals.setdefault(c, []).append(v)
    med = {c: statistics.median(v) for c, v in vals.items()}
    n = {c: len(v) for c, v in vals.items()}
    rows = [f"| {c} | {med[c]:.4g} | {n[c]} |" for c in sorted(med)]
    derived = []
    if "GRBM_GUI_ACTIVE" in med:
        cyc = med["GRBM_GUI_ACTIVE"] / N_XCD
        derived.append(f"engine cycles per dispatch: {cyc:.4g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            derived.append(f"MFMA busy per SIMD: {100 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / N_SIMD / cyc:.1f} %")
    wc = med.get("SQ_WAVE_CYCLES")
    if wc:
        for c, what in (("SQ_WAIT_INST_ANY", "waiting on a counter (vmcnt/lgkmcnt)"),
                        ("SQ_WAIT_INST_LDS", "waiting on LDS"),
                        ("SQ_ACTIVE_INST_VALU", "issuing VALU (MFMA included)"),
                        ("SQ_ACTIVE_INST_LDS", "issuing LDS instructions"),
                        ("SQ_WAIT_ANY", "waiting (any)")):
            if c in med:
                derived.append(f"{what}: {100 * med[c] / wc:.1f} % of wave cycles ({c})")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        derived.append(f"bf16 MFMA flops per dispatch: {med['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g}")
    out = [f"# rocprofv3 counters: {kernel} ({key})", "",
           "Commands (from the repository root on the MI355X box; one counter set per run):", "",
           "    " + command, "",
           f"Medians per dispatch of {kernel} (exact base name), the later half of its "
           "dispatches in each run:", "",
           "| Counter | Median per dispatch | Dispatches |", "|---|---|---|", *rows, "",
           "Derived:", "", *[f"- {x}" for x in derived]]
    path = os.path.join(ROOT, "profiles", WORKLOADS[key][6] + "_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(path)


# ---------------------------------------------------------------- the lines
def measure(key, steps, warmup):
    runner, metric, unit, bound, peak, kernel, _, _, div = WORKLOADS[key]
    r = runner()
    k, w = max(1, steps // div), max(1, warmup // div)
    if key == "tiny":
        k = max(steps, 50)
    t = time_steps(r.step, k, w)
    tk = t if r.kernel is r.step else time_steps(r.kernel, k, w)
    scale = 1e12 if unit == TF else 1e9
    ent = {"key": key, "metric": metric, "unit": unit, "ms_per_step": t["ms"], "steps": k,
           "workload": r.workload}
    if unit == "us":
        ent.update(value=t["ms"] * 1e3, higher_is_better=False,
                   warm={"ms_per_step": t["ms_warm"], "value": t["ms_warm"] * 1e3},
                   roofline={"bound": "latency", "achieved": None, "peak": None, "unit": "us",
                             "frac": None, "traffic": None, "kernel": kernel})
        return ent, r
    value = r.work / (t["ms"] * 1e-3) / scale
    achieved = r.kernel_work / (tk["ms"] * 1e-3) / scale
    rec = counter_record(key)
    ent.update(value=value, warm={"ms_per_step": t["ms_warm"],
                                  "value": r.work / (t["ms_warm"] * 1e-3) / scale})
    rf = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
          "frac": achieved / peak, "traffic": None if rec is None else rec["bytes_per_launch"],
          "kernel": kernel, "kernel_ms": tk["ms"], "kernel_ms_mean": tk["ms_mean"],
          "kernel_warm_ms": tk["ms_warm"], "algorithmic_per_launch": r.kernel_work,
          "algorithmic_unit": "flop" if unit == TF else "byte"}
    if rec is not None and "clock" in rec:
        ghz = rec["clock"]["ghz_median"]
        rf.update(clock_ghz_measured=ghz, peak_at_measured_clock=peak * ghz / PEAK_CLOCK_GHZ,
                  frac_at_measured_clock=achieved / (peak * ghz / PEAK_CLOCK_GHZ),
                  clock_source=os.path.relpath(traffic_path(key), ROOT))
        if "mfma_busy_frac_median" in rec["clock"]:
            rf["mfma_busy_frac_measured"] = rec["clock"]["mfma_busy_frac_median"]
    if key in PEAK_NOTES:
        rf["peak_note"] = PEAK_NOTES[key]
    ent["roofline"] = rf
    if unit == GB:
        ent["frac_of_hbm_peak_whole_op"] = value / PEAK_HBM_GBS
    for name in ("splits",):
        if name in r.extra:
            ent[name] = r.extra[name]
    if "plan" in r.extra:
        ent["plan_max_splits_waves_min_blocks"] = r.extra["plan"]
    if "cached_tokens" in r.extra:
        ent["cached_tokens_per_s"] = r.extra["cached_tokens"] / (t["ms"] * 1e-3)
    if "gathered_bytes" in r.extra:
        ent["gathered_gbs"] = r.extra["gathered_bytes"] / (t["ms"] * 1e-3) / 1e9
    if "alg_bytes" in r.extra:   # MLA: its HBM side, reported beside the MFMA bound
        ent["kv_read_gbs"] = r.extra["alg_bytes"] / (t["ms"] * 1e-3) / 1e9
        ent["frac_of_hbm_peak"] = ent["kv_read_gbs"] / PEAK_HBM_GBS
    return ent, r


def cpu_baseline(pre):
    """The float64 oracle as it stands, timed on the host on the prefill
    workload: all eight sequences and 32 heads (about 10 s of host work on 16
    threads; the sample is the whole job)."""
    from threadpoolctl import threadpool_info
    from oracle import attention as orc
    w = pre.w
    lens = pre.extra["lens"]
    seqs = list(range(len(lens)))
    q, k, v = w.f32("q"), w.f32("k"), w.f32("v")
    t0 = time.perf_counter()
    orc.attention_varlen(q, k, v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True, seqs=seqs)
    dt = time.perf_counter() - t0
    flops = prefill_flops(lens)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 numpy oracle on all {len(seqs)} sequences (lengths {lens}) of "
                      f"the prefill workload, all 32 heads; {dt:.1f} s wall; BLAS threads "
                      f"{threads}, host affinity {len(os.sched_getaffinity(0))} cpus, "
                      f"os.cpu_count() {os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="untimed back-to-back steps before the warmup of each workload")
    ap.add_argument("--only", default=",".join(WORKLOADS),
                    help="comma-separated workloads; the prefill (if listed) heads the line")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the first workload of --only (the prefill by default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB elementwise kernel, so that a counter "
                         "profile of this run can scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--workload", default="prefill",
                    help="the workload of --traffic-from / --profile-summary")
    ap.add_argument("--traffic-from", nargs="+", metavar="DIR",
                    help="no GPU work: write the workload kernel's counter record from two "
                         "rocprofv3 --pmc folders (FETCH_SIZE, WRITE_SIZE) and optionally a "
                         "third (GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES with --kernel-trace)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="no GPU work: write profiles/<kernel>_<workload>.md from a rocprofv3 "
                         "--kernel-trace folder and --bench-json (the line of the same run)")
    ap.add_argument("--counters-summary", nargs="+", metavar="DIR",
                    help="no GPU work: write profiles/<kernel>_<workload>_counters.md from "
                         "rocprofv3 --pmc folders of the workload")
    ap.add_argument("--bench-json", default="")
    ap.add_argument("--command", default="", help="the profiling command, stored with a record")
    args = ap.parse_args()
    RAMP_MS[0] = max(0.0, args.ramp_ms)
    if args.traffic_from:
        if len(args.traffic_from) not in (2, 3):
            ap.error("--traffic-from takes FETCH_DIR WRITE_DIR [CLOCK_DIR]")
        write_traffic(args.workload, *args.traffic_from[:2], args.command,
                      args.traffic_from[2] if len(args.traffic_from) == 3 else None)
        return
    if args.profile_summary:
        profile_summary(args.workload, args.profile_summary, args.bench_json, args.command)
        return
    if args.counters_summary:
        counters_summary(args.workload, args.counters_summary, args.command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs on a single GPU "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from attention_attn_fwd_02_amd import binding as B
    B.load()
    only = [k for k in args.only.split(",") if k]
    for k in only:
        if k not in WORKLOADS:
            ap.error(f"unknown workload {k}")
    head_key = "prefill" if "prefill" in only else only[0]
    if args.no_secondary:
        only = [head_key]
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)   # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    lines, runs = {}, {}
    for key in [head_key] + [k for k in only if k != head_key]:
        log(f"{key} ...")
        ent, r = measure(key, args.steps, args.warmup)
        lines[key], runs[key] = ent, r
        log(f"{key} {ent['ms_per_step']:.4f} ms/step (warm {ent['warm']['ms_per_step']:.4f}) "
            f"{ent['value']:.1f} {ent['unit']}")
    cpu = None
    if not args.no_cpu and head_key == "prefill":
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(runs["prefill"])
        log(f"cpu {cpu['value']:.6f} TFLOP/s")

    head = lines[head_key]
    rf = dict(head["roofline"])
    if head_key == "prefill":
        rf["algorithmic_bytes_per_launch"] = runs["prefill"].extra["algorithmic_bytes_per_launch"]
        # the convention of most published causal-attention rates: 2*D*Hq*sum L^2
        # (half of 4*D*Hq*L^2), which leaves out the diagonal's L extra pairs
        fa = sum(2.0 * 128 * 32 * int(L) * int(L) for L in runs["prefill"].extra["lens"])
        rf["fa_style"] = {"flop_per_launch": fa,
                          "value": fa / (head["ms_per_step"] * 1e-3) / 1e12,
                          "unit": "TFLOP/s"}
    rec = {
        "metric": METRIC if head_key == "prefill" else head["metric"],
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": RAMP_MS[0],
        "ms_per_step": head["ms_per_step"],
        "timing": "median over the timed steps, each after an untimed 512 MiB read that evicts "
                  "the Infinity Cache (steps and evictions enqueued back to back); `warm` = the "
                  "same number of steps back to back without eviction",
        "warm": head["warm"],
        "higher_is_better": head.get("higher_is_better", True),
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if head_key != "tiny" else "f32",
        "data": "synthetic",
        "key": head_key,
        "config": ({"workload": head["workload"], "global_batch": 8,
                    "seq_len": f"U[512,4096] (drawn {runs[head_key].extra.get('lens')})",
                    "heads_q": 32, "heads_kv": 8, "head_dim": 128, "causal": True,
                    "parallelism": "none (1 GPU)"} if head_key == "prefill" else
                   {"workload": head["workload"], "parallelism": "none (1 GPU)"}),
        "roofline": rf,
        "cpu_baseline": cpu,
        "secondary": [lines[k] for k in lines if k != head_key],
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
