"""Head-mix GRU: the GRU with a block-diagonal recurrent matrix (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name GRU cells with mix='head' beside the diagonal ones (shapes/
layout page, support table: head-mix is a fused path for rectangular
batches; with a ragged pack the fused path raises and the eager one runs),
and the FAQs' memory notes speak of heads and d_head.  They print no
equations.  Reading (the plainest one the diagonal cell supports): the
hidden width d_h splits into n_heads = d_h / d_head heads of d_head
consecutive channels, and each gate's per-channel recurrent term a_g * h
becomes, head by head, a dense d_head x d_head matrix times that head's
part of h:

    z = sig(x_z + A_z h)      r = sig(x_r + A_r h)
    c = tanh(x_c + A_c (r * h))
    h' = (1 - z) * h + z * c

A_g has shape (n_heads, d_head, d_head); (A_g h) for head k is
A_g[k] @ h[k*d_head:(k+1)*d_head].  With d_head = 1, or with diagonal
blocks, this is the diagonal GRU of cells.py.

Jacobian of one step, per head a dense d_head x d_head block (product and
chain rules applied to f):
    dz/dh = diag(z(1-z)) A_z          dr/dh = diag(r(1-r)) A_r
    d(r*h)/dh = diag(r) + diag(h) dr/dh
    dc/dh = diag(1 - c^2) A_c d(r*h)/dh
    J = diag(1 - z) + diag(c - h) dz/dh + diag(z) dc/dh

Newton is the method of newton.py with these dense blocks: at iteration k,
prev_t = H^(k-1)_{t-1} (h0 at t = 0), f_t = f(prev_t, x_t), J_t = df/dh at
prev_t (J_0 := 0), b_t = f_t - J_t prev_t, and H^(k)_t = J_t H^(k)_{t-1}
+ b_t serially, stored in the storage dtype.  Rectangular batches only.
Arrays: xp (B, T, 3, d_h); states (B, T, d_h); h0 (B, d_h).
"""
from __future__ import annotations

import numpy as np

from .newton import max_abs
from .rounding import store


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def heads_of(v, d_head):
    """(..., d_h) -> (..., n_heads, d_head)."""
    return v.reshape(*v.shape[:-1], v.shape[-1] // d_head, d_head)


def block_matvec(Ag, v):
    """Ag (n_heads, d_head, d_head), v (..., d_h) -> (..., d_h): each head's block times its slice."""
    d_head = Ag.shape[-1]
    out = np.einsum("kij,...kj->...ki", Ag, heads_of(v, d_head))
    return out.reshape(v.shape)


def gates(h, xp, A):
    z = sigmoid(xp[..., 0, :] + block_matvec(A[0], h))
    r = sigmoid(xp[..., 1, :] + block_matvec(A[1], h))
    c = np.tanh(xp[..., 2, :] + block_matvec(A[2], r * h))
    return z, r, c


def f(h, xp, A):
    z, r, c = gates(h, xp, A)
    return (1.0 - z) * h + z * c


def jac(h, xp, A):
    """(..., n_heads, d_head, d_head): J[..., k, i, j] = d h'_(k,i) / d h_(k,j)."""
    d_head = A.shape[-1]
    z, r, c = (heads_of(v, d_head) for v in gates(h, xp, A))
    hh = heads_of(h, d_head)
    eye = np.eye(d_head)
    dz = (z * (1.0 - z))[..., :, None] * A[0]                     # diag(z(1-z)) A_z
    dr = (r * (1.0 - r))[..., :, None] * A[1]                     # diag(r(1-r)) A_r
    drh = r[..., :, None] * eye + hh[..., :, None] * dr           # diag(r) + diag(h) dr/dh
    dc = (1.0 - c * c)[..., :, None] * np.einsum("kim,...kmj->...kij", A[2], drh)
    return (1.0 - z)[..., :, None] * eye + (c - hh)[..., :, None] * dz + z[..., :, None] * dc


def block_apply(J, v):
    """J (..., n_heads, d_head, d_head), v (..., d_h) -> (..., d_h)."""
    d_head = J.shape[-1]
    return np.einsum("...kij,...kj->...ki", J, heads_of(v, d_head)).reshape(v.shape)


def sequential(xp, A, h0=None):
    """The for-loop unroll h_t = f(h_{t-1}, x_t).  Returns (H (B,T,d_h), last (B,d_h))."""
    xp = np.asarray(xp, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B, T, _, d = xp.shape
    h = np.zeros((B, d)) if h0 is None else np.asarray(h0, dtype=np.float64).copy()
    last = h.copy()
    H = np.zeros((B, T, d))
    for t in range(T):
        h = f(h, xp[:, t], A)
        H[:, t] = h
    if T > 0:
        last = H[:, T - 1].copy()
    return H, last


def affine_recurrence(J, b):
    """h_t = J_t h_{t-1} + b_t serially from h_{-1} = 0; J (B,T,n_heads,d_head,d_head), b (B,T,d_h)."""
    B, T, d = b.shape
    out = np.zeros_like(b)
    h = np.zeros((B, d))
    for t in range(T):
        h = block_apply(J[:, t], h) + b[:, t]
        out[:, t] = h
    return out


def previous(H, h0):
    """prev_t = H_{t-1}, h0 (or 0) at t = 0."""
    B, T, d = H.shape
    prev = np.zeros_like(H)
    if T > 0:
        prev[:, 0] = 0.0 if h0 is None else h0
        prev[:, 1:] = H[:, :-1]
    return prev


def newton(xp, A, K, h0=None, dtype="f64", keep_iterates=False):
    """K Newton iterations from H^(0) = 0.  Returns dict(H, residuals [r_0..r_K], iterates)."""
    xp = np.asarray(xp, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    h0 = None if h0 is None else np.asarray(h0, dtype=np.float64)
    B, T, _, d = xp.shape
    H = np.zeros((B, T, d))
    res, iterates = [], []
    for _k in range(K):
        prev = previous(H, h0)
        fv = f(prev, xp, A)
        res.append(max_abs(H - fv))
        J = jac(prev, xp, A)
        J[:, 0] = 0.0
        b = fv - block_apply(J, prev)
        H = store(affine_recurrence(J, b), dtype)
        if keep_iterates:
            iterates.append(H.copy())
    res.append(max_abs(H - f(previous(H, h0), xp, A)))
    out = {"H": H, "residuals": res}
    if keep_iterates:
        out["iterates"] = iterates
    return out
