"""Storage-dtype rounding for iterates held in fp32 or bf16.

The FAQs page (Turing GPUs; Triton loads through load_acc/store_acc) says
the algebra stays in fp32 whatever the storage dtype; values are rounded only
when stored.  bf16 keeps the top 16 bits of an IEEE fp32 value; rounding is
to nearest, ties to even (the usual float32 -> bfloat16 conversion).
"""
from __future__ import annotations

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float64/float32 values to the nearest bf16 value (ties to even).

    Goes through float32 first (round-to-nearest-even), then drops the low
    16 bits of the fp32 pattern with round-to-nearest-even on the dropped
    half.  NaN stays NaN; Inf stays Inf.  Returns float64 values.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16          # carry into the exponent is the correct overflow to Inf
    u = (u << 16).astype(np.uint32)
    out = u.view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def bf16_from_bits(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def store(x, dtype: str) -> np.ndarray:
    """The value a storage slot of ``dtype`` ('f32' | 'bf16' | 'f64') holds for x."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


def load(arr, dtype: str) -> np.ndarray:
    """Upcast stored values (float32 array, or bf16 bits as uint16) to float64."""
    if dtype == "bf16":
        return bf16_from_bits(arr)
    return np.asarray(arr).astype(np.float64)
