"""Compiles the HIP sources under csrc/ into libattn_mi355.so (gfx950 only).

Usage: python -m attention_attn_fwd_02_amd.build   (or build() from Python)
Each .hip file is compiled to an object in parallel, then linked in-tree next
to this file, where the binding loads it.

ATTN_BUILD_DEFINES (environment, optional): extra -D flags for a debug build,
e.g. ATTN_BUILD_DEFINES=-DATTN_LDS_POISON=1 fills every LDS block with NaN
bits before its DMA, so that a read ahead of a missing wait shows up as NaN in
the GPU tests. Rebuild without it before measuring.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn_mi355.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code; hipcc's host pass
# does not know the feature and warns about it, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _defines():
    extra = os.environ.get("ATTN_BUILD_DEFINES", "").split()
    bad = [f for f in extra if not f.startswith("-D")]
    if bad:
        raise ValueError(f"ATTN_BUILD_DEFINES takes -D flags only, got {bad}")
    return extra


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *_defines(), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, errs in results:
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
