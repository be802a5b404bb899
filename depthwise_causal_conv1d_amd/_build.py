"""Builds the gfx950 HIP library ``libdcconv.so`` in-tree with hipcc.

Run as ``python -m depthwise_causal_conv1d_amd._build``.  The library is built
for gfx950 (MI355X) only.  Packed-FP32 instruction selection is switched off for
all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdcconv.so")
SOURCES = ["abi.hip", "update.hip", "update_tokens.hip", "prefill.hip", "update_ring.hip", "copy_control.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libdcconv.so`` (always rebuilds)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    for proc, src in procs:
        _, err = proc.communicate()
        # hipcc's host pass does not know the packed-fp32 feature and says so
        noise = "not a recognized feature for this target"
        err = "\n".join(x for x in err.splitlines() if noise not in x)
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
