"""Loader of oracle/c/unroll.c: the sequential unroll of the diagonal GRU /
LSTM in plain C (float64, OpenMP over channels).

Test infrastructure: only tests, the smoke check and the bench's CPU
baseline use it.  build() compiles it with gcc; unroll() runs it on host
arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "unroll.c")
LIB = os.path.join(HERE, "c", "liboracle_unroll.so")
_L = None


def build(verbose: bool = True) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print("[oracle build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(verbose=False)
        L = ctypes.CDLL(LIB)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_unroll.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, vp, i64, vp, vp]
        L.oracle_unroll.restype = ctypes.c_int
        _L = L
    return _L


def unroll(cell: str, xp, a, h0=None, cu_seqlens=None) -> np.ndarray:
    """h of the unroll, (B, T, d) float64.  xp (B, T, G, d) is read as
    float32 (the stored values; bf16 widens exactly), a as float64, h0
    (rows, S, d) as float64 or None for zeros."""
    xp = np.ascontiguousarray(xp, dtype=np.float32)
    a = np.ascontiguousarray(a, dtype=np.float64)
    B, T, G, d = xp.shape
    h0c = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    out = np.empty((B, T, d), dtype=np.float64)
    rc = _lib().oracle_unroll(0 if cell == "gru" else 1, B, T, d, xp.ctypes.data, a.ctypes.data,
                              None if h0c is None else h0c.ctypes.data, 0 if cu is None else cu.size - 1,
                              None if cu is None else cu.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_unroll rejected its arguments")
    return out
