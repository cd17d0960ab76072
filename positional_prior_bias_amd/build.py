"""Build libbam.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m positional_prior_bias_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled with hipcc for gfx950 only, then linked
into positional_prior_bias_amd/libbam.so.  Packed fp32 VALU instructions are
disabled on the device side (``-packed-fp32-ops``); hipcc's host pass prints a
harmless warning that it does not know that feature.  ``-fno-honor-nans`` lets
max/min lower to single instructions: no kernel here produces a NaN from inputs
that meet include/bam.h's preconditions (finite q, k, v and parameters): masked
logits are -inf, every exp2 argument is guarded against -inf - -inf, and the
distance table's entries are finite for finite parameters.  Symbols are hidden by
default: libbam.so exports only the entry points include/bam.h declares.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbam.so")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbam.so")
    return h


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [_hipcc(), *CXXFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose: bool = False, extra=()) -> str:
    """Compile every kernel source and link libbam.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    for obj, warn in results:
        if warn and verbose:
            print(f"[{os.path.basename(obj)}] {warn}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
