"""Build libbitlinear.so in-tree with hipcc for gfx950.

Each .hip file is compiled to an object under csrc/_build/ (in parallel), then
linked into bit_gemm_int8_amd/libbitlinear.so.  Always rebuilds."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libbitlinear.so")
SOURCES = ["api.hip", "quant_act.hip", "pack.hip", "gemv.hip", "gemv_stream.hip", "gemv_stream_mt.hip",
           "gemv_mfma.hip",
           "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 14 dwords of scalar kernel arguments arrive preloaded in
    # SGPRs where the firmware supports it (the code object keeps a load
    # path): decode-sized launches start their loads ~0.2 us sooner
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if l.strip() and noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
