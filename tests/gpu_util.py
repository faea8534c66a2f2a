"""Helpers for the GPU tests: host arrays <-> device tensors, and the
element-by-element comparison against the float64 oracle."""
import sys

import numpy as np
import torch

# Tolerances (max-abs): bf16 outputs 2e-2, float32 LSE 1e-3. For the float32
# path the output is compared at 1e-4: inputs are exact and every operation is
# a float32 FMA/exp2/log2, so errors are a few float32 ulps of O(1) values
# accumulated over at most a few thousand terms.
TOL_O_BF16 = 2e-2
TOL_O_F32 = 1e-4
TOL_LSE = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    """uint16 bf16 bits -> bf16 tensor; float32/int32 arrays as they are."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) else t.cpu().numpy()


def compare(name, o_gpu, lse_gpu, o_ref, lse_ref, tol_o, tol_lse=TOL_LSE, mask=None):
    """Compares outputs where the oracle computed them (non-NaN); rows the
    oracle marks empty (LSE = -inf) must be -inf on the GPU and have O = 0."""
    o = host(o_gpu).astype(np.float64)
    l = host(lse_gpu).astype(np.float64)
    sel = ~np.isnan(o_ref)
    if mask is not None:
        sel &= mask
    assert np.isfinite(o[sel]).all(), f"{name}: non-finite output"
    err_o = float(np.abs(o[sel] - o_ref[sel]).max()) if sel.any() else 0.0
    lsel = ~np.isnan(lse_ref)
    fin = lsel & np.isfinite(lse_ref)
    empty = lsel & np.isneginf(lse_ref)
    err_l = float(np.abs(l[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    rel = float(np.linalg.norm(o[sel] - o_ref[sel]) / max(1e-30, np.linalg.norm(o_ref[sel])))
    log(f"[{name}] max|dO|={err_o:.3e} rel_fro={rel:.3e} max|dLSE|={err_l:.3e} "
        f"rows={int(fin.sum())} empty={int(empty.sum())}")
    assert np.isneginf(l[empty]).all(), f"{name}: empty rows must have LSE = -inf"
    assert err_o <= tol_o, f"{name}: output error {err_o} > {tol_o}"
    assert err_l <= tol_lse, f"{name}: LSE error {err_l} > {tol_lse}"
    return err_o, err_l


def assert_plan_equal(got, ref, batch, max_splits):
    """The GPU plan equals the oracle's bit for bit where it is defined: the
    header, split_ptr, the total_splits triples and the work order."""
    got = np.asarray(got)
    n = 3 + batch + 3 * int(ref[0])
    assert np.array_equal(got[:n], ref[:n]), \
        f"plan mismatch at {np.nonzero(got[:n] != ref[:n])[0][:8]}"
    o = 3 + batch + 3 * batch * max_splits
    t = int(ref[0])
    assert np.array_equal(got[o:o + t], ref[o:o + t]), \
        f"work order mismatch at {np.nonzero(got[o:o + t] != ref[o:o + t])[0][:8]}"
