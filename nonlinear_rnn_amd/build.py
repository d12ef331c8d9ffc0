"""Build libprn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m nonlinear_rnn_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libprn.so")
SOURCES = ["prn_api.hip", "proj.hip"]
ARCH = os.environ.get("PRN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU instructions are disabled: plain fp32 code only.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libprn)")


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    t0 = time.time()
    if verbose:
        print("[prn build]", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    if verbose and (r.stderr.strip()):
        sys.stderr.write(r.stderr[-4000:])
    os.replace(tmp, LIB)
    if verbose:
        print(f"[prn build] {LIB} built in {time.time() - t0:.1f} s", flush=True)
    return LIB


if __name__ == "__main__":
    build()
