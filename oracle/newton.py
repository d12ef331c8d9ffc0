"""Sequential unroll and K-iteration parallel Newton, written out plainly (float64).

Sources on the pararnn-torch pages:
  * FAQs, "Does parallel Newton match sequential unroll?" and the Numerics
    contract, "Invariant": the Newton forward must agree with an honest
    sequential unroll within tau (1e-4 in fp32) at the measured depth K*(T).
  * FAQs, "train() vs eval()": train runs parallel Newton + scan, eval the
    sequential step.
  * FAQs, "How many Newton iterations should I use?": K pinned (3 for
    GRU/LSTM-style cells) or taken from a per-T table.
  * Numerics contract, "Two thresholds" and "1. Runtime": the residual
    max|F(H)| is read after K steps and gated (warn 1e-3, fail 1.0).
  * Shapes/layout page, ragged packs: x is one row of N tokens plus
    cu_seqlens (S+1 offsets); every segment head uses J = 0 on the scan.

The Newton method (the pages name it without equations; this is the standard
Newton iteration on the stacked system F(H) = 0, F_t = h_t - f(h_{t-1}, x_t)):
  H^(0) = 0 for every step; at iteration k = 1..K
    prev_t = H^(k-1)_{t-1}, replaced by the segment's initial state at a head
    f_t = f(prev_t, x_t),  J_t = df/ds (prev_t, x_t)
    J_t := 0 at a head
    b_t = f_t - J_t prev_t
    H^(k)_t = J_t H^(k)_{t-1} + b_t        (serial affine recurrence)
  and H^(k) is stored in the storage dtype before it becomes the next
  linearisation point.  r_k = max |H^(k)_t - f(prev^(k)_t, x_t)| over batch,
  time, state component and channel, with NaN counted as +Inf.

Readings where the pages are silent (each one listed in the design notes):
  * the initial guess is zero at every step t >= 1; the initial state h0 is
    fixed, not an unknown;
  * a head's previous state is its own segment's h0 (zero when none is given);
  * the residual is that of the stored (storage-dtype) trajectory;
  * max-abs is the agreement norm (AgreementReport.max_abs; the strided-view
    example on the shapes/layout page prints (y_n - y_s).abs().max()).
"""
from __future__ import annotations

import numpy as np

from .cells import cell_fns
from .rounding import store


# ------------------------------------------------------------ layout ----

def head_segments(B: int, T: int, cu_seqlens=None) -> np.ndarray:
    """(B, T) int array: the segment index starting at (b, t), else -1.

    Rectangular batch: one segment per row, starting at t = 0 (index b).
    Ragged pack (B = 1): segment j starts at cu[j]; an empty segment starts
    nowhere (its final state is its initial state).
    """
    hs = np.full((B, T), -1, dtype=np.int64)
    if cu_seqlens is None:
        if T > 0:                      # a zero-length row has no step, so no head
            hs[:, 0] = np.arange(B)
        return hs
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    for j in range(len(cu) - 1):
        if cu[j + 1] > cu[j]:
            hs[0, cu[j]] = j
    return hs


def n_rows(B: int, cu_seqlens) -> int:
    return B if cu_seqlens is None else len(cu_seqlens) - 1


def initial_states(B, S, d, cu_seqlens, h0) -> np.ndarray:
    rows = n_rows(B, cu_seqlens)
    if h0 is None:
        return np.zeros((rows, S, d))
    h0 = np.asarray(h0, dtype=np.float64)
    assert h0.shape == (rows, S, d)
    return h0


def previous_states(H: np.ndarray, heads: np.ndarray, H0: np.ndarray) -> np.ndarray:
    """prev[b, t] = H[b, t-1], or the segment's initial state at a head."""
    prev = np.zeros_like(H)
    prev[:, 1:] = H[:, :-1]
    bi, ti = np.nonzero(heads >= 0)
    prev[bi, ti] = H0[heads[bi, ti]]
    return prev


def last_states(H: np.ndarray, cu_seqlens, H0: np.ndarray) -> np.ndarray:
    """Final state of every sequence (row or segment); h0 for an empty one."""
    if cu_seqlens is None:
        return H[:, -1].copy()
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = H0.copy()
    for j in range(len(cu) - 1):
        if cu[j + 1] > cu[j]:
            out[j] = H[0, cu[j + 1] - 1]
    return out


def max_abs(x) -> float:
    """max |x| with NaN counted as +Inf (a non-finite residual must trip the gate)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    if x.size == 0:
        return 0.0
    x = np.where(np.isnan(x), np.inf, x)
    return float(x.max())


# -------------------------------------------------------- sequential ----

def sequential(cell, xp, a, h0=None, cu_seqlens=None):
    """The plain for-loop unroll s_t = f(s_{t-1}, x_t) (the truth).

    xp (B,T,G,d) float64, a (G,d).  Returns (states (B,T,S,d), last (rows,S,d)).
    """
    G, S, f, _ = cell_fns(cell)
    xp = np.asarray(xp, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    B, T, _, d = xp.shape
    heads = head_segments(B, T, cu_seqlens)
    H0 = initial_states(B, S, d, cu_seqlens, h0)
    out = np.zeros((B, T, S, d))
    s = np.zeros((B, S, d))
    for t in range(T):
        hb = heads[:, t]
        m = hb >= 0
        if m.any():
            s[m] = H0[hb[m]]
        s = f(s, xp[:, t], a)
        out[:, t] = s
    return out, last_states(out, cu_seqlens, H0)


# ------------------------------------------------------------ newton ----

def affine_recurrence(J: np.ndarray, b: np.ndarray) -> np.ndarray:
    """s_t = J_t s_{t-1} + b_t serially from s_{-1} = 0 (J at t=0 is 0 anyway).

    J (B,T,S,S,d), b (B,T,S,d) -> (B,T,S,d).
    """
    B, T, S, d = b.shape
    out = np.zeros_like(b)
    s = np.zeros((B, S, d))
    for t in range(T):
        s = np.einsum("bpqd,bqd->bpd", J[:, t], s) + b[:, t]
        out[:, t] = s
    return out


def residual(cell, H, xp, a, heads, H0) -> float:
    """max |F(H)|, F_t = H_t - f(prev_t, x_t)."""
    _, _, f, _ = cell_fns(cell)
    return max_abs(H - f(previous_states(H, heads, H0), xp, a))


def newton(cell, xp, a, K, h0=None, cu_seqlens=None, dtype="f64", jacobian=True,
           keep_iterates=False, picard=0):
    """K Newton iterations from H^(0) = 0, or from P = picard Picard sweeps.

    Picard warm-start (FAQs, "How many Newton iterations should I use?":
    try picard_iters before raising the iteration budget).  Reading: a sweep
    is the Jacobi step H <- f(shift(H), x) over all steps at once (the
    previous step's value of the current guess, h0 at a head), stored in the
    storage dtype; P sweeps from 0 give the guess the Newton iterations
    start from, and r_0 is the residual of that guess.

    xp (B,T,G,d) float64 (already the stored projection, upcast), a (G,d).
    dtype: storage dtype of the iterates ('f64', 'f32', 'bf16').
    jacobian=False replaces J by 0 (a Picard / Jacobi sweep H <- f(shift(H))),
    used only as a comparison.
    Returns dict(H = H^(K) (B,T,S,d) as stored, residuals = [r_0..r_K],
    last = final state per sequence, iterates = [H^(1)..H^(K)] if asked).
    """
    G, S, f, jac = cell_fns(cell)
    xp = np.asarray(xp, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    B, T, _, d = xp.shape
    heads = head_segments(B, T, cu_seqlens)
    H0 = initial_states(B, S, d, cu_seqlens, h0)
    head_mask = heads >= 0
    H = np.zeros((B, T, S, d))
    for _p in range(picard):
        H = store(f(previous_states(H, heads, H0), xp, a), dtype)
    res = []
    iterates = []
    for _k in range(K):
        prev = previous_states(H, heads, H0)
        fv = f(prev, xp, a)
        res.append(max_abs(H - fv))
        if jacobian:
            J = jac(prev, xp, a)
        else:
            J = np.zeros((B, T, S, S, d))
        J[head_mask] = 0.0
        b = fv - np.einsum("btpqd,btqd->btpd", J, prev)
        H = store(affine_recurrence(J, b), dtype)
        if keep_iterates:
            iterates.append(H.copy())
    res.append(residual(cell, H, xp, a, heads, H0))
    out = {"H": H, "residuals": res, "last": last_states(H, cu_seqlens, H0)}
    if keep_iterates:
        out["iterates"] = iterates
    return out


# --------------------------------------------------------- K schedule ---

def resolve_k(T: int, table: dict) -> int:
    """K for length T from a per-T table {T_key: K}.

    Reading of newton_iters_by_t={64: 2, 1024: 3, ...} (FAQs, "How many Newton
    iterations should I use?"): the entry with the smallest key >= T; above
    the largest key, the largest key's entry.
    """
    keys = sorted(int(k) for k in table)
    for k in keys:
        if T <= k:
            return int(table[k])
    return int(table[keys[-1]])
