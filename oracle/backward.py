"""Gradients through the recurrence: the adjoint (reverse-time) recurrence,
written out plainly (float64).  TEST INFRASTRUCTURE ONLY, like the rest of
this package.

Sources on the pararnn-torch pages: the FAQs ("train() vs eval()": training
runs the parallel Newton forward and backpropagates through it; the OOM
cheat sheet's recompute option for long sequences) and the shapes/layout
page (the train forward+backward surface of the diagonal GRU/LSTM, ragged
packs with J = 0 at segment heads).  The pages do not print the backward
equations.  Reading taken (listed in the design notes): the backward of the
Newton forward is the gradient of the sequential recurrence
s_t = f(s_{t-1}, x_t) at the trajectory the forward returned, i.e. the
solution of the adjoint (transposed) linear recurrence

    lam_t = g_t + J_{t+1}^T lam_{t+1}          (0 past a sequence's end)

with g_t = dL/ds_t the gradient arriving directly at step t (dL/dh_t in the
h component, plus dL/d(final state) at the last step of a sequence) and
J_{t+1} = d f / d s at step t+1, which is cut (0) where step t+1 is a
segment head: the state before a head is the segment's h0, not step t.
Then, per step,
    dL/dx_t  = (d s_t/d x_t)^T lam_t           (the projected inputs)
    dL/da   += (d s_t/d a)^T lam_t             (summed over rows and steps)
    dL/dh0_j = J_t^T lam_t at the head t of segment j
and an empty segment or a zero-length row (final state = its h0, as in the
forward) passes its final-state gradient to its h0 unchanged.
"""
from __future__ import annotations

import numpy as np

from .cells import cell_fns, cell_partials
from .newton import head_segments, initial_states, previous_states


def adjoint(cell, xp, a, states, dH, h0=None, cu_seqlens=None, dstate_last=None):
    """Gradients at a given trajectory.

    xp (B,T,G,d), a (G,d), states (B,T,S,d) the trajectory s_1..s_T (its
    h component is the forward's output), dH (B,T,d) = dL/dh_t, dstate_last
    (rows,S,d) = dL/d(final state of each sequence) or None.
    Returns (dxp (B,T,G,d), da (G,d), dh0 (rows,S,d)).
    """
    G, S, _, jac = cell_fns(cell)
    dxf, daf = cell_partials(cell)
    xp = np.asarray(xp, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    states = np.asarray(states, dtype=np.float64)
    B, T, _, d = xp.shape
    heads = head_segments(B, T, cu_seqlens)
    H0 = initial_states(B, S, d, cu_seqlens, h0)
    rows = H0.shape[0]
    prev = previous_states(states, heads, H0)   # the state each step starts from
    J = jac(prev, xp, a)                        # (B,T,S,S,d): J[..., p, q, :] = d s'_p / d s_q
    DX = dxf(prev, xp, a)                       # (B,T,S,G,d)
    DA = daf(prev, xp, a)

    g = np.zeros((B, T, S, d))
    g[:, :, S - 1, :] = np.asarray(dH, dtype=np.float64)
    dh0 = np.zeros((rows, S, d))
    if dstate_last is not None:
        dsl = np.asarray(dstate_last, dtype=np.float64)
        if cu_seqlens is None:
            if T > 0:
                g[:, T - 1] += dsl
            else:                    # a zero-length row ends in its h0
                dh0 += dsl
        else:
            cu = np.asarray(cu_seqlens, dtype=np.int64)
            for j in range(rows):
                if cu[j + 1] > cu[j]:
                    g[0, cu[j + 1] - 1] += dsl[j]
                else:
                    dh0[j] += dsl[j]

    dxp = np.zeros((B, T, G, d))
    da = np.zeros((G, d))
    nxt = np.zeros((B, S, d))                   # J_{t+1}^T lam_{t+1}, already cut at heads
    for t in range(T - 1, -1, -1):
        lam = g[:, t] + nxt
        dxp[:, t] = np.einsum("bpgd,bpd->bgd", DX[:, t], lam)
        da += np.einsum("bpgd,bpd->gd", DA[:, t], lam)
        mu = np.einsum("bpqd,bpd->bqd", J[:, t], lam)
        hb = heads[:, t]
        for b in np.nonzero(hb >= 0)[0]:
            dh0[hb[b]] += mu[b]
        nxt = np.where((hb >= 0)[:, None, None], 0.0, mu)
    return dxp, da, dh0
