"""Benchmark of the fused attention forward on one MI355X.

Headline: varlen causal GQA prefill (8 sequences with lengths U[512, 4096],
Hq=32, Hkv=8, D=128, bf16), in attention TFLOP/s. One step = one
attn_fwd_varlen call over the whole packed batch (the single kernel of the
prefill path). The same JSON line carries the other workloads as
`secondary` entries: paged GQA decode (KV-read GB/s, step = plan + split
decode + combine) with a bf16 and with an FP8 cache, MLA-absorbed paged
decode, chunked prefill over a paged cache, sparse MLA with sinks and
block-sparse MLA over a paged cache.

Inputs are seeded synthetic tensors already resident in HBM when timing
starts. Every timed region is bracketed by torch.cuda.synchronize() and
timed with HIP events on the stream the kernels are launched on. Before the
W warmup steps of each workload, its step runs untimed for --ramp-ms
milliseconds: from idle the GPU takes about 40 ms of continuous work to
leave its low clocks (prefill steps run 25 % slower over the first 10 ms),
so a few warmup steps alone would time the clock ramp, not the kernels.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill,...]
                [--no-cpu] [--no-secondary]
"""
import argparse
import json
import os
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


RAMP_MS = [200.0]


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


def time_steps(fn, steps, warmup):
    """Ramps the clocks (ramp), runs fn warmup times untimed, then `steps`
    times between two HIP events on the current stream; returns milliseconds
    per step."""
    import torch
    ramp(fn, RAMP_MS[0])
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


_EVICT = []


def time_cold(fn, n):
    """Median over n steps, each timed alone after a 1 GiB write that evicts
    the 256 MB Infinity Cache (the eviction is outside the timed region)."""
    import torch
    if not _EVICT:
        _EVICT.append(torch.empty(1 << 28, dtype=torch.float32, device="cuda"))
    buf = _EVICT[0]
    times = []
    for i in range(n):
        buf.fill_(float(i))
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return float(np.median(times))


def prefill_flops(lens, hq=32, d=128):
    # 4*D per (query row, visible key): 2*D for QK^T and 2*D for P.V; a causal
    # row t sees t+1 keys.
    return sum(4.0 * d * hq * (int(L) * (int(L) + 1) / 2) for L in lens)


def bench_prefill(steps, warmup):
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.varlen_prefill()
    lens = np.diff(w.cu_seqlens_q)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cq, ck = dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
    out = None
    lse = None

    def step():
        B.attn_fwd_varlen(q, k, v, cq, ck, int(lens.max()), int(lens.max()), w.scale, True,
                          out=out_buf, lse=lse_buf)

    import torch
    out_buf = torch.empty((int(lens.sum()), 32, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.empty((32, int(lens.sum())), dtype=torch.float32, device="cuda")
    ms = time_steps(step, steps, warmup)
    ms_cold = time_cold(step, 9)
    flops = prefill_flops(lens)
    tflops = flops / (ms * 1e-3) / 1e12
    in_bytes = (w.q.nbytes + w.k.nbytes + w.v.nbytes)
    out_bytes = out_buf.numel() * 2 + lse_buf.numel() * 4
    return dict(ms=ms, ms_cold=ms_cold, tflops=tflops, flops=flops, lens=lens.tolist(), w=w,
                bytes=in_bytes + out_bytes)


def bench_tiny(steps, warmup):
    from attention_attn_fwd_02_amd import binding as B
    from attention_attn_fwd_02_amd import inputs
    w = inputs.tiny_dense()
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    cq, ck = dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
    import torch
    out = torch.empty_like(q)
    lse = torch.empty((w.q.shape[1], w.q.shape[0]), dtype=torch.float32, device="cuda")

    def step():
        B.attn_fwd_varlen(q, k, v, cq, ck, 128, 128, w.scale, False, out=out, lse=lse)

    ms = time_steps(step, max(steps, 50), warmup)
    return dict(ms=ms, us=ms * 1e3)


def bench_prefill_fp8(steps, warmup):
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

    ms = time_steps(step, steps, warmup)
    flops = prefill_flops(lens, hq, d)
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12, lens=lens.tolist())


def bench_prefill_qv(steps, warmup):
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

    ms = time_steps(step, steps, warmup)
    # q.k, qv.v and p.v: 6 D flop per visible (row, key) pair
    flops = prefill_flops(lens, hq, d) * 6 / 4
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12)


def bench_decode(steps, warmup):
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
    op = torch.empty((b * ms_, sq * hq, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((b * ms_, sq * hq), dtype=torch.float32, device="cuda")
    out = torch.empty((b, sq, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")

    def full():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        B.attn_decode_paged(q, kc, vc, bt, lens, plan, ms_, w.scale, False, op, lp)
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    def decode_only():
        B.attn_decode_paged(q, kc, vc, bt, lens, plan, ms_, w.scale, False, op, lp)

    ms_full = time_steps(full, steps, warmup)
    ms_dec = time_steps(decode_only, steps, warmup)
    ms_cold = time_cold(full, 9)
    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 + 128) * 2
    alg_bytes = kv_bytes + w.q.nbytes + out.numel() * 2 + lse.numel() * 4 + nblk * 4
    return dict(ms=ms_full, ms_kernel=ms_dec, ms_cold=ms_cold, bytes=alg_bytes, kv_bytes=kv_bytes,
                gbs=alg_bytes / (ms_full * 1e-3) / 1e9, gbs_kernel=alg_bytes / (ms_dec * 1e-3) / 1e9,
                splits=int(plan[0].item()))


def bench_decode_qv(steps, warmup, only_qv=False):
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
    op = torch.empty((b * ms_, sq * hq, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((b * ms_, sq * hq), dtype=torch.float32, device="cuda")
    out = torch.empty((b, sq, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")
    qq, kk = (None, None) if only_qv else (q, kc)

    def decode_only():
        B.attn_decode_paged_qv(qq, qv, kk, vc, bt, lens, plan, ms_, w.scale, None, causal=False,
                               only_qv=only_qv, o_partial=op, lse_partial=lp)

    def full():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        decode_only()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    ms_full = time_steps(full, steps, warmup)
    ms_dec = time_steps(decode_only, steps, warmup)
    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 if only_qv else 256) * 2   # V only with only_qv
    alg_bytes = (kv_bytes + qvh.nbytes + (0 if only_qv else w.q.nbytes) + out.numel() * 2 +
                 lse.numel() * 4 + nblk * 4)
    return dict(ms=ms_full, ms_kernel=ms_dec, bytes=alg_bytes,
                gbs=alg_bytes / (ms_full * 1e-3) / 1e9, gbs_kernel=alg_bytes / (ms_dec * 1e-3) / 1e9,
                splits=int(plan[0].item()))


def bench_decode_fp8(steps, warmup):
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
    op = torch.empty((b * ms_, sq * hq, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((b * ms_, sq * hq), dtype=torch.float32, device="cuda")
    out = torch.empty((b, sq, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")

    def decode_only():
        B.attn_decode_paged_fp8(q, kc, vc, bt, lens, plan, ms_, w.scale, w.fmt, qd, kd, vd,
                                False, op, lp)

    def full():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        decode_only()
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    ms_full = time_steps(full, steps, warmup)
    ms_dec = time_steps(decode_only, steps, warmup)
    ms_cold = time_cold(full, 9)
    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    nblk = int(((w.cache_seqlens + 63) // 64).sum())
    kv_bytes = total_len * hkv * (128 + 128)               # one byte per code
    alg_bytes = (kv_bytes + w.q.nbytes + out.numel() * 2 + lse.numel() * 4 + nblk * 4
                 + 3 * b * hkv * 4)
    return dict(ms=ms_full, ms_kernel=ms_dec, ms_cold=ms_cold, bytes=alg_bytes, kv_bytes=kv_bytes,
                tokens=total_len, gbs=alg_bytes / (ms_full * 1e-3) / 1e9,
                gbs_kernel=alg_bytes / (ms_dec * 1e-3) / 1e9, splits=int(plan[0].item()))


def bench_mla(steps, warmup):
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
    op = torch.empty((b * ms_, sq * hq, 512), dtype=torch.float32, device="cuda")
    lp = torch.empty((b * ms_, sq * hq), dtype=torch.float32, device="cuda")
    out = torch.empty((b, sq, hq, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device="cuda")

    def full():
        B.attn_plan_splits(lens, 64, upb, ncu, waves, ms_, mb, plan=plan)
        B.mla_decode_paged(q, kc, bt, lens, plan, ms_, w.scale, False, op, lp)
        B.attn_combine(op, lp, plan, b, sq, hq, ms_, None, torch.bfloat16, out, lse)

    def decode_only():
        B.mla_decode_paged(q, kc, bt, lens, plan, ms_, w.scale, False, op, lp)

    ms_full = time_steps(full, steps, warmup)
    ms_dec = time_steps(decode_only, steps, warmup)
    ms_cold = time_cold(full, 9)
    total_len = int(w.cache_seqlens.astype(np.int64).sum())
    flops = total_len * sq * hq * 2.0 * (576 + 512)
    alg_bytes = total_len * 1152 + w.q.nbytes + out.numel() * 2 + lse.numel() * 4
    return dict(ms=ms_full, ms_kernel=ms_dec, ms_cold=ms_cold, flops=flops, bytes=alg_bytes,
                tflops=flops / (ms_full * 1e-3) / 1e12, gbs=alg_bytes / (ms_full * 1e-3) / 1e9,
                tflops_kernel=flops / (ms_dec * 1e-3) / 1e12, splits=int(plan[0].item()))


def bench_sparse(steps, warmup):
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

    ms = time_steps(step, max(1, steps // 4), max(1, warmup // 2))
    valid = int((s.indices >= 0).sum())     # every drawn index lies in its causal prefix
    flops = valid * hq * 2.0 * (576 + 512)
    gathered = valid * 1152
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12,
                gathered_gbs=gathered / (ms * 1e-3) / 1e9)


def bench_chunked(steps, warmup, with_mask=False):
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

    ms = time_steps(step, steps, warmup)
    # query t of a chunk sees the cache and the chunk's rows 0..t
    flops = sum(4.0 * d * hq * (int(n) * int(c) + int(n) * (int(n) + 1) / 2)
                for n, c in zip(lq, lc))
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12, lc=lc.tolist())


def bench_chunked_fp8(steps, warmup):
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

    ms = time_steps(step, steps, warmup)
    flops = sum(4.0 * d * hq * (int(n) * int(c) + int(n) * (int(n) + 1) / 2)
                for n, c in zip(lq, lc))
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12, lc=lc.tolist())


def bench_sparse_paged(steps, warmup):
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

    ms = time_steps(step, max(1, steps // 4), max(1, warmup // 2))
    # every drawn block lies in its token's causal prefix; count its keys there
    valid = 0
    for bi in range(b):
        lk = int(w.seqlens_kv[bi])
        lim = lk - sq + np.arange(sq)                                   # last visible key
        blk = w.indices[bi, :, 0, :].astype(np.int64)
        first = blk * w.block_size
        n = np.clip(lim[:, None] - first + 1, 0, w.block_size)
        valid += int(np.where(blk >= 0, n, 0).sum())
    flops = valid * hq * 2.0 * (576 + 512)
    return dict(ms=ms, flops=flops, tflops=flops / (ms * 1e-3) / 1e12,
                gathered_gbs=valid * 1152 / (ms * 1e-3) / 1e9)


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "k_varlen_bf16_d128_traffic.txt")
# the sources the prefill kernel is compiled from (its translation unit)
PREFILL_SOURCES = ("kernels_prefill.hip", "prefill_bf16.h", "device_common.h", "launch.h")
COPY_BYTES = 1 << 30          # the calibration copy: 1 GiB read and 1 GiB written
COPY_KERNEL_TAG = "neg"       # torch.neg(src, out=dst) runs one elementwise kernel


def prefill_source_digest():
    """Digest of the prefill kernel's sources and compile flags."""
    import hashlib
    from attention_attn_fwd_02_amd import build
    h = hashlib.sha256()
    for name in PREFILL_SOURCES:
        with open(os.path.join(build.CSRC, name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()[:16]


def prefill_record():
    """The committed counter profile of the prefill kernel, or None when it
    does not match the current prefill sources."""
    try:
        with open(TRAFFIC_PATH) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("prefill_source_sha256_16") != prefill_source_digest():
        return None
    return rec


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter profile of this
    kernel (FETCH_SIZE + WRITE_SIZE, scaled by the same counters read on a
    plain copy of known size), or None when no such profile matches the
    current prefill sources."""
    rec = prefill_record()
    return None if rec is None else rec.get("bytes_per_launch")


N_XCD, N_SIMD = 8, 1024      # MI355X: GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs


def measured_clock(clock_dir):
    """Engine clock and MFMA busy fraction during the timed prefill launches,
    from a rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES
    --kernel-trace run of `bench.py --only prefill --no-secondary --no-cpu`:
    per dispatch, GRBM_GUI_ACTIVE / 8 XCDs / duration, median over the last
    20 dispatches (the timed steps come after the clock ramp and warm-up)."""
    import csv
    import glob
    import statistics
    d = {}
    for fn in glob.glob(os.path.join(clock_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if "k_varlen_bf16" not in r["Kernel_Name"] or "PrefillCfg<128" not in r["Kernel_Name"]:
                    continue
                e = d.setdefault(int(r["Dispatch_Id"]), {})
                e[r["Counter_Name"]] = float(r["Counter_Value"])
                e["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    ids = sorted(d)
    if len(ids) < 29:
        raise SystemExit(f"expected >= 29 prefill dispatches in {clock_dir}, got {len(ids)}")
    # bench.py's order: ramp, 3 warm-up, 20 timed, then 9 cold-cache steps
    timed = ids[-29:-9]
    ghz = statistics.median(d[i]["GRBM_GUI_ACTIVE"] / N_XCD / d[i]["dur"] / 1e9 for i in timed)
    busy = statistics.median(d[i]["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD /
                             (d[i]["GRBM_GUI_ACTIVE"] / N_XCD) for i in timed)
    return {"ghz_median": ghz, "mfma_busy_frac_median": busy, "dispatches": len(timed)}


def write_traffic(fetch_dir, write_dir, command, clock_dir=None):
    """Builds the traffic record from two rocprofv3 --pmc runs of
    `bench.py --only prefill --no-secondary --no-cpu --copy-calibration`
    (one with FETCH_SIZE, one with WRITE_SIZE; both in KiB per dispatch),
    and optionally the engine clock from a third (measured_clock)."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == counter:
                        out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    def split(rs):
        copy = [v for n, v in rs if COPY_KERNEL_TAG in n and "attn" not in n]
        pre = [v for n, v in rs if "k_varlen_bf16" in n and "PrefillCfg<128" in n]
        if len(copy) != 1 or not pre:
            raise SystemExit(f"expected one calibration copy and prefill dispatches, got "
                             f"{len(copy)} and {len(pre)}")
        return copy[0], sum(pre) / len(pre), len(pre)

    copy_f, pre_f, n_f = split(rows(fetch_dir, "FETCH_SIZE"))
    copy_w, pre_w, n_w = split(rows(write_dir, "WRITE_SIZE"))
    k_f = COPY_BYTES / (copy_f * 1024)
    k_w = COPY_BYTES / (copy_w * 1024)
    rec = {
        "kernel": "k_varlen_bf16<PrefillCfg<128, 4, 32, 3, 3>> (varlen causal prefill, D=128)",
        "bytes_per_launch": pre_f * 1024 * k_f + pre_w * 1024 * k_w,
        "fetch_kib_per_launch": pre_f, "write_kib_per_launch": pre_w,
        "dispatches": [n_f, n_w],
        "calibration": {"copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_f,
                        "copy_write_kib": copy_w, "fetch_factor": k_f, "write_factor": k_w},
        "prefill_source_sha256_16": prefill_source_digest(),
        "command": command,
    }
    if clock_dir:
        rec["clock"] = measured_clock(clock_dir)
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_baseline(pre):
    """The float64 oracle as it stands, timed on the host on the prefill
    workload: all eight sequences and 32 heads (about 10 s of host work on 16
    threads; the sample is the whole job)."""
    from threadpoolctl import threadpool_info
    from oracle import attention as orc
    w = pre["w"]
    seqs = list(range(len(pre["lens"])))
    q, k, v = w.f32("q"), w.f32("k"), w.f32("v")
    t0 = time.perf_counter()
    orc.attention_varlen(q, k, v, w.cu_seqlens_q, w.cu_seqlens_k, w.scale, True, seqs=seqs)
    dt = time.perf_counter() - t0
    lens = [pre["lens"][i] for i in seqs]
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
    ap.add_argument("--only",
                    default="prefill,tiny,prefill_fp8,prefill_qv,decode,decode_fp8,decode_qv,"
                            "decode_only_qv,mla,chunked,chunked_mask,chunked_fp8,sparse,sparse_paged")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy, so that a "
                         "counter profile of this run can scale FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs="+", metavar="DIR",
                    help="no GPU work: write the prefill traffic record from two "
                         "rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) and "
                         "optionally a third (GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES "
                         "with --kernel-trace) for the engine clock")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command, stored with the traffic record")
    args = ap.parse_args()
    RAMP_MS[0] = max(0.0, args.ramp_ms)
    if args.traffic_from:
        if len(args.traffic_from) not in (2, 3):
            ap.error("--traffic-from takes FETCH_DIR WRITE_DIR [CLOCK_DIR]")
        write_traffic(*args.traffic_from[:2], args.traffic_command,
                      args.traffic_from[2] if len(args.traffic_from) == 3 else None)
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
    only = set(args.only.split(","))
    if args.no_secondary:
        only &= {"prefill"}
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)   # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    log("prefill ...")
    pre = bench_prefill(args.steps, args.warmup)
    log(f"prefill {pre['ms']:.3f} ms  {pre['tflops']:.1f} TFLOP/s")
    traffic = measured_traffic()
    secondary = []
    if "tiny" in only:
        log("tiny dense fp32 ...")
        ti = bench_tiny(args.steps, args.warmup)
        log(f"tiny {ti['us']:.1f} us per call")
        secondary.append({
            "metric": "latency of one call (tiny dense attention, fp32)", "value": ti["us"],
            "unit": "us", "higher_is_better": False, "ms_per_step": ti["ms"],
            "workload": "B=1, Sq=Sk=128, Hq=Hkv=4, D=64, fp32 Q/K/V ~ N(0,1), non-causal, scale "
                        "1/8, O and LSE out (seed 1001); back-to-back calls on one stream",
            "roofline": {"bound": "latency", "achieved": None, "peak": None, "unit": "us",
                         "frac": None, "traffic": None, "kernel": "k_varlen_f32 (D=64)"}})
    if "prefill_fp8" in only:
        log("prefill fp8 ...")
        p8 = bench_prefill_fp8(args.steps, args.warmup)
        log(f"prefill_fp8 {p8['ms']:.3f} ms {p8['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "attention TFLOP/s (varlen prefill, FP8 e4m3 Q/K/V)", "value": p8["tflops"],
            "unit": "TFLOP/s", "ms_per_step": p8["ms"],
            "workload": "varlen causal GQA prefill: 8 sequences U[512,4096] (drawn "
                        f"{p8['lens']}), Hq=32, Hkv=8, D=128, e4m3 codes with per-(sequence, KV "
                        "head) descales, bf16 out (seed 1009)",
            "roofline": {"bound": "mfma", "achieved": p8["tflops"], "peak": PEAK_FP8_MIX_TFLOPS,
                         "unit": "TFLOP/s", "frac": p8["tflops"] / PEAK_FP8_MIX_TFLOPS,
                         "traffic": None, "kernel": "k_varlen_fp8 (D=128)",
                         "peak_note": "half the flops (Q.K^T) on FP8 MFMA (5033 TFLOP/s), "
                                      "half (P.V) on bf16 MFMA (2517 TFLOP/s): the harmonic "
                                      "mix"}})
    if "prefill_qv" in only:
        log("prefill qv ...")
        pq = bench_prefill_qv(args.steps, args.warmup)
        log(f"prefill_qv {pq['ms']:.3f} ms {pq['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "attention TFLOP/s (varlen prefill with qv)", "value": pq["tflops"],
            "unit": "TFLOP/s", "ms_per_step": pq["ms"],
            "workload": "the varlen causal GQA prefill workload (seed 1002) with a bf16 qv "
                        "(T,32,128) N(0,1) (seed 1011); scores q.k + qv.v; 6 D flop per visible "
                        "(row, key) pair",
            "roofline": {"bound": "mfma", "achieved": pq["tflops"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": pq["tflops"] / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "k_varlen_qv (D=128)"}})
    if "decode" in only:
        log("paged decode ...")
        dec = bench_decode(args.steps, args.warmup)
        log(f"decode {dec['ms']:.3f} ms (kernel {dec['ms_kernel']:.3f}) {dec['gbs']:.0f} GB/s")
        secondary.append({
            "metric": "KV-read GB/s (paged decode)", "value": dec["gbs"], "unit": "GB/s",
            "ms_per_step": dec["ms"],
            "cold_cache": {"ms_per_step_median": dec["ms_cold"],
                           "value": dec["bytes"] / (dec["ms_cold"] * 1e-3) / 1e9},
            "workload": "paged GQA decode: batch 64, 1 query token, cache_seqlens U[1024,32768], "
                        "page 64, Hq=32, Hkv=8, D=128, bf16; plan + split decode (<=16 splits) + "
                        f"combine per step; {dec['splits']} splits (seed 1003)",
            "roofline": {"bound": "hbm", "achieved": dec["gbs_kernel"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": dec["gbs_kernel"] / PEAK_HBM_GBS,
                         "traffic": None, "kernel": "k_decode (GQA)",
                         "kernel_ms": dec["ms_kernel"]},
            "frac_of_hbm_peak_whole_op": dec["gbs"] / PEAK_HBM_GBS})
    if "decode_fp8" in only:
        log("paged decode fp8 ...")
        d8 = bench_decode_fp8(args.steps, args.warmup)
        log(f"decode_fp8 {d8['ms']:.3f} ms (kernel {d8['ms_kernel']:.3f}) {d8['gbs']:.0f} GB/s")
        secondary.append({
            "metric": "KV-read GB/s (paged decode, FP8 e4m3 Q/K/V)", "value": d8["gbs"],
            "unit": "GB/s", "ms_per_step": d8["ms"],
            "cached_tokens_per_s": d8["tokens"] / (d8["ms"] * 1e-3),
            "cold_cache": {"ms_per_step_median": d8["ms_cold"],
                           "value": d8["bytes"] / (d8["ms_cold"] * 1e-3) / 1e9},
            "workload": "paged GQA decode with an FP8 cache: batch 64, 1 query token, "
                        "cache_seqlens U[1024,32768], page 64, Hq=32, Hkv=8, D=128, e4m3 codes "
                        "with per-(batch, KV head) descales, bf16 out; plan + split decode "
                        f"(<=16 splits) + combine per step; {d8['splits']} splits (seed 1007)",
            "roofline": {"bound": "hbm", "achieved": d8["gbs_kernel"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": d8["gbs_kernel"] / PEAK_HBM_GBS,
                         "traffic": None, "kernel": "k_decode (GQA, FP8)",
                         "kernel_ms": d8["ms_kernel"]},
            "frac_of_hbm_peak_whole_op": d8["gbs"] / PEAK_HBM_GBS})
    for key, only_qv in (("decode_qv", False), ("decode_only_qv", True)):
        if key not in only:
            continue
        log(f"{key} ...")
        dq = bench_decode_qv(args.steps, args.warmup, only_qv)
        log(f"{key} {dq['ms']:.3f} ms (kernel {dq['ms_kernel']:.3f}) {dq['gbs']:.0f} GB/s")
        what = ("qv alone (only_qv: V read, K not)" if only_qv
                else "q . k + qv . v scores (K and V read)")
        secondary.append({
            "metric": f"KV-read GB/s (paged decode, {'only_qv' if only_qv else 'qv'})",
            "value": dq["gbs"], "unit": "GB/s", "ms_per_step": dq["ms"],
            "workload": "the paged GQA decode workload (seed 1003) with a bf16 qv "
                        f"(B,1,32,128) N(0,1) (seed 1010); {what}; plan + split decode + "
                        f"combine; {dq['splits']} splits",
            "roofline": {"bound": "hbm", "achieved": dq["gbs_kernel"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": dq["gbs_kernel"] / PEAK_HBM_GBS,
                         "traffic": None, "kernel": "k_decode (GQA, qv)",
                         "kernel_ms": dq["ms_kernel"]},
            "frac_of_hbm_peak_whole_op": dq["gbs"] / PEAK_HBM_GBS})
    if "mla" in only:
        log("mla decode ...")
        mla = bench_mla(args.steps, args.warmup)
        log(f"mla {mla['ms']:.3f} ms {mla['tflops']:.1f} TFLOP/s {mla['gbs']:.0f} GB/s")
        secondary.append({
            "metric": "MLA paged decode TFLOP/s", "value": mla["tflops"], "unit": "TFLOP/s",
            "ms_per_step": mla["ms"], "kv_read_gbs": mla["gbs"],
            "cold_cache": {"ms_per_step_median": mla["ms_cold"],
                           "value": mla["flops"] / (mla["ms_cold"] * 1e-3) / 1e12},
            "frac_of_hbm_peak": mla["gbs"] / PEAK_HBM_GBS,
            "workload": "MLA-absorbed paged decode: batch 64, 2 query tokens, Hq=128, Hkv=1, "
                        "D=576 (V = first 512), page 64, cache_seqlens U[2048,16384], bf16; plan "
                        f"+ split decode + combine; {mla['splits']} splits (seed 1004)",
            "roofline": {"bound": "mfma", "achieved": mla["tflops_kernel"],
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": mla["tflops_kernel"] / PEAK_BF16_TFLOPS, "traffic": None,
                         "kernel": "k_decode (MLA)", "kernel_ms": mla["ms_kernel"]}})
    if "chunked" in only:
        log("chunked prefill ...")
        ch = bench_chunked(args.steps, args.warmup)
        log(f"chunked {ch['ms']:.3f} ms {ch['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "chunked prefill TFLOP/s (cache + new K/V)", "value": ch["tflops"],
            "unit": "TFLOP/s", "ms_per_step": ch["ms"],
            "workload": "chunked causal GQA prefill: 8 sequences, 1024 new tokens each after a "
                        f"paged cache of U[1024,8192] tokens (drawn {ch['lc']}), page 64, "
                        "Hq=32, Hkv=8, D=128, bf16; attn_fwd_varlen_kvcache (seed 1006)",
            "roofline": {"bound": "mfma", "achieved": ch["tflops"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ch["tflops"] / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "k_varlen_bf16 (cache + current, D=128)"}})
    if "chunked_mask" in only:
        log("chunked prefill with mask ...")
        cm = bench_chunked(args.steps, args.warmup, with_mask=True)
        log(f"chunked_mask {cm['ms']:.3f} ms {cm['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "chunked prefill TFLOP/s (cache + new K/V, additive mask)",
            "value": cm["tflops"], "unit": "TFLOP/s", "ms_per_step": cm["ms"],
            "workload": "the chunked-prefill workload (seed 1006) with one bf16 additive mask "
                        "shared by all heads, N(0,1) over every (row, key), streamed beside K/V",
            "roofline": {"bound": "mfma", "achieved": cm["tflops"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": cm["tflops"] / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "k_varlen_bf16 (cache + current, mask)"}})
    if "chunked_fp8" in only:
        log("chunked prefill fp8 ...")
        c8 = bench_chunked_fp8(args.steps, args.warmup)
        log(f"chunked_fp8 {c8['ms']:.3f} ms {c8['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "chunked prefill TFLOP/s (cache + new K/V, FP8 e4m3 Q/K/V)",
            "value": c8["tflops"], "unit": "TFLOP/s", "ms_per_step": c8["ms"],
            "workload": "the chunked-prefill shape (8 sequences, 1024 new tokens each after a "
                        f"paged cache of U[1024,8192] tokens (drawn {c8['lc']}), page 64, Hq=32, "
                        "Hkv=8, D=128) on e4m3 codes with per-(sequence, KV head) descales, bf16 "
                        "out; attn_fwd_varlen_kvcache_fp8 (seed 1012)",
            "roofline": {"bound": "mfma", "achieved": c8["tflops"], "peak": PEAK_FP8_MIX_TFLOPS,
                         "unit": "TFLOP/s", "frac": c8["tflops"] / PEAK_FP8_MIX_TFLOPS,
                         "traffic": None, "kernel": "k_varlen_fp8_kvc (D=128)",
                         "peak_note": "Q.K^T on FP8 MFMA, P.V on bf16 MFMA: the harmonic mix"}})
    if "sparse" in only:
        log("sparse mla ...")
        sp = bench_sparse(args.steps, args.warmup)
        log(f"sparse {sp['ms']:.3f} ms {sp['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "sparse MLA + sink TFLOP/s", "value": sp["tflops"], "unit": "TFLOP/s",
            "ms_per_step": sp["ms"], "gathered_gbs": sp["gathered_gbs"],
            "workload": "top-2048 sparse MLA with per-head sinks: 4 x 4096 query tokens, 32768 "
                        "keys, Hq=64, D=576 (V = first 512), bf16 (seed 1005)",
            "roofline": {"bound": "mfma", "achieved": sp["tflops"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": sp["tflops"] / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "k_sparse"}})

    if "sparse_paged" in only:
        log("block-sparse paged mla ...")
        sp2 = bench_sparse_paged(args.steps, args.warmup)
        log(f"sparse_paged {sp2['ms']:.3f} ms {sp2['tflops']:.1f} TFLOP/s")
        secondary.append({
            "metric": "block-sparse paged MLA + sink TFLOP/s", "value": sp2["tflops"],
            "unit": "TFLOP/s", "ms_per_step": sp2["ms"], "gathered_gbs": sp2["gathered_gbs"],
            "workload": "block-sparse MLA over a paged latent cache: 4 x 4096 query tokens, "
                        "32768 keys per sequence in pages of 64, 32 blocks of 64 keys per token "
                        "(sparse_block_size 64), Hq=64, D=576 (V = first 512), sinks, bf16 "
                        "(seed 1008)",
            "roofline": {"bound": "mfma", "achieved": sp2["tflops"], "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": sp2["tflops"] / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "k_sparse (paged)"}})

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(pre)
        log(f"cpu {cpu['value']:.6f} TFLOP/s")

    rec = {
        "metric": "attention TFLOP/s (varlen prefill) and KV-read GB/s (paged decode), 1 MI355X",
        "value": pre["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": RAMP_MS[0],
        "ms_per_step": pre["ms"],
        "cold_cache": {"ms_per_step_median": pre["ms_cold"],
                       "value": pre["flops"] / (pre["ms_cold"] * 1e-3) / 1e12,
                       "note": "each step timed alone after a 1 GiB write that evicts the "
                               "Infinity Cache; value and ms_per_step above time K steps "
                               "back to back"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREFILL_WORKLOAD, "global_batch": 8,
                   "seq_len": f"U[512,4096] (drawn {pre['lens']})", "heads_q": 32, "heads_kv": 8,
                   "head_dim": 128, "causal": True, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": pre["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": pre["tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": "k_varlen_bf16 (D=128)",
                     "algorithmic_flops_per_launch": pre["flops"],
                     "algorithmic_bytes_per_launch": pre["bytes"]},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    prec = prefill_record()
    if prec and "clock" in prec:
        # the same kernel's engine clock in the committed counter run: the peak
        # scales with it (MFMA throughput per cycle is fixed)
        ghz = prec["clock"]["ghz_median"]
        peak_clk = PEAK_BF16_TFLOPS * ghz / PEAK_CLOCK_GHZ
        rec["roofline"].update({
            "clock_ghz_measured": ghz, "peak_at_measured_clock": peak_clk,
            "frac_at_measured_clock": pre["tflops"] / peak_clk,
            "mfma_busy_frac_measured": prec["clock"]["mfma_busy_frac_median"],
            "clock_source": "GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration over the timed "
                            "launches of a rocprofv3 counter run (" +
                            os.path.relpath(TRAFFIC_PATH, ROOT) + ")"})
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
