"""Critical Newton depth K*(T), written out plainly (float64).  TEST
INFRASTRUCTURE ONLY, like the rest of this package.

Source: the FAQs ("What is critical Newton depth (K*)?") and the Numerics
contract ("2. Lab campaign"): K*(T) is the smallest Newton iteration count
whose result still matches the plain sequential for-loop within tau
(about 1e-4 in fp32) at sequence length T; the measured envelopes become a
per-T table that the training config resolves K from.

Readings (listed in the design notes): the agreement norm is max-abs over h
(as everywhere in these pages); the Newton result is taken with the
iterates stored in the storage dtype; K* is None when no K up to K_max
agrees.
"""
from __future__ import annotations

import numpy as np

from .newton import max_abs, newton, sequential


def agreement_errors(cell, xp, a, K_max, h0=None, cu_seqlens=None, dtype="f64"):
    """[max|h^(K) - h_seq| for K = 1..K_max] on one input."""
    S = 1 if cell == "gru" else 2
    seq, _ = sequential(cell, xp, a, h0=h0, cu_seqlens=cu_seqlens)
    out = newton(cell, xp, a, K_max, h0=h0, cu_seqlens=cu_seqlens, dtype=dtype, keep_iterates=True)
    return [max_abs(Hk[..., S - 1, :] - seq[..., S - 1, :]) for Hk in out["iterates"]]


def kstar(errors, tau):
    """Smallest K (1-based) with errors[K-1] <= tau, else None."""
    for k, e in enumerate(errors, start=1):
        if e <= tau:
            return k
    return None


def k_table(kstars: dict) -> dict:
    """{T: K*} measured at increasing T -> the per-T table of the FAQs'
    newton_iters_by_t form, made monotone (a longer sequence never gets a
    smaller K than a shorter one measured below it)."""
    out, run = {}, 0
    for T in sorted(kstars):
        run = max(run, int(kstars[T]))
        out[int(T)] = run
    return out
