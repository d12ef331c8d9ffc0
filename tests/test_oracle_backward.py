"""Pins of the oracle's backward (adjoint) pass.

Nothing here re-types the adjoint formulas: every gradient is checked against
central finite differences of the forward functions in float64 (the cell f,
and the plain sequential for-loop unroll), which share no code with the
closed-form partials or the reverse recurrence.  Central differences with
step 1e-6 in float64 are accurate to about 1e-9 on these smooth functions.
"""
import zlib

import numpy as np
import pytest

from oracle import backward, cells, newton

EPS = 1e-6
CELLS = [("gru", 3, 1), ("lstm", 4, 2)]


def fd(fun, x, idx):
    xp_, xm_ = x.copy(), x.copy()
    xp_[idx] += EPS
    xm_[idx] -= EPS
    return (fun(xp_) - fun(xm_)) / (2 * EPS)


@pytest.mark.parametrize("cell,G,S", CELLS)
def test_input_and_weight_partials_match_finite_differences(cell, G, S):
    rng = np.random.default_rng(11)
    d = 5
    s = rng.standard_normal((S, d)) * 0.7
    xp = rng.standard_normal((G, d)) * 1.5
    a = rng.uniform(-0.9, 0.9, (G, d))
    _, _, f, _ = cells.cell_fns(cell)
    dxf, daf = cells.cell_partials(cell)
    DX, DA = dxf(s, xp, a), daf(s, xp, a)
    assert DX.shape == DA.shape == (S, G, d)
    for p in range(S):
        for g in range(G):
            for c in range(d):
                ex = fd(lambda v: f(s, v, a)[p, c], xp, (g, c))
                ea = fd(lambda v: f(s, xp, v)[p, c], a, (g, c))
                assert abs(DX[p, g, c] - ex) <= 1e-8, (p, g, c)
                assert abs(DA[p, g, c] - ea) <= 1e-8, (p, g, c)


def loss_fn(cell, S, dH, dsl, cu=None):
    """L = sum_t <dH_t, h_t> + sum_j <dsl_j, final state_j> through the unroll."""
    def L(xp, a, h0):
        st, last = newton.sequential(cell, xp, a, h0=h0, cu_seqlens=cu)
        return float((st[..., S - 1, :] * dH).sum() + (last * dsl).sum())
    return L


CASES = [
    ("rect", 2, 5, None),
    ("ragged", 1, 9, [0, 3, 3, 7, 9]),     # includes an empty segment
    ("ragged-tail", 1, 7, [0, 6, 7]),      # a one-step last segment
    ("single-step", 3, 1, None),
]


@pytest.mark.parametrize("cell,G,S", CELLS)
@pytest.mark.parametrize("name,B,T,cu", CASES)
def test_adjoint_matches_finite_differences_of_the_unroll(cell, G, S, name, B, T, cu):
    rng = np.random.default_rng(zlib.crc32(f"{cell}/{name}".encode()))
    d = 2
    rows = B if cu is None else len(cu) - 1
    xp = rng.standard_normal((B, T, G, d))
    a = rng.uniform(-0.8, 0.8, (G, d))
    h0 = rng.standard_normal((rows, S, d)) * 0.5
    dH = rng.standard_normal((B, T, d))
    dsl = rng.standard_normal((rows, S, d))
    states, _ = newton.sequential(cell, xp, a, h0=h0, cu_seqlens=cu)
    dxp, da, dh0 = backward.adjoint(cell, xp, a, states, dH, h0=h0, cu_seqlens=cu, dstate_last=dsl)
    L = loss_fn(cell, S, dH, dsl, cu)
    for idx in np.ndindex(*xp.shape):
        assert abs(dxp[idx] - fd(lambda v: L(v, a, h0), xp, idx)) <= 1e-7, idx
    for idx in np.ndindex(*a.shape):
        assert abs(da[idx] - fd(lambda v: L(xp, v, h0), a, idx)) <= 1e-7, idx
    for idx in np.ndindex(*h0.shape):
        assert abs(dh0[idx] - fd(lambda v: L(xp, a, v), h0, idx)) <= 1e-7, idx


@pytest.mark.parametrize("cell,G,S", CELLS)
def test_adjoint_without_final_state_gradient_and_h0(cell, G, S):
    """dstate_last and h0 omitted: the same as passing zeros."""
    rng = np.random.default_rng(5)
    B, T, d = 2, 6, 3
    xp = rng.standard_normal((B, T, G, d))
    a = rng.uniform(-0.5, 0.5, (G, d))
    dH = rng.standard_normal((B, T, d))
    states, _ = newton.sequential(cell, xp, a)
    r1 = backward.adjoint(cell, xp, a, states, dH)
    r2 = backward.adjoint(cell, xp, a, states, dH, h0=np.zeros((B, S, d)), dstate_last=np.zeros((B, S, d)))
    for u, v in zip(r1, r2):
        assert np.array_equal(u, v)


def test_gradient_of_a_cut_sequence_does_not_cross_a_head():
    """Two segments: the loss on the second segment gives no gradient to the
    first segment's inputs (J = 0 across the head)."""
    rng = np.random.default_rng(2)
    T, d, cu = 8, 3, [0, 4, 8]
    xp = rng.standard_normal((1, T, 3, d))
    a = rng.uniform(-0.5, 0.5, (3, d))
    h0 = rng.standard_normal((2, 1, d)) * 0.5   # nonzero: the reset gate's gradient carries a factor h
    states, _ = newton.sequential("gru", xp, a, h0=h0, cu_seqlens=cu)
    dH = np.zeros((1, T, d))
    dH[0, 4:] = rng.standard_normal((4, d))
    dxp, _, dh0 = backward.adjoint("gru", xp, a, states, dH, h0=h0, cu_seqlens=cu)
    assert np.all(dxp[0, :4] == 0.0) and np.all(dh0[0] == 0.0)
    assert np.all(dxp[0, 4:] != 0.0) and np.all(dh0[1] != 0.0)


@pytest.mark.parametrize("cell,G,S", CELLS)
def test_zero_length_rows_pass_final_state_gradient_to_h0(cell, G, S):
    """A zero-length row (or an all-empty pack) ends in its h0."""
    d = 3
    dsl = np.arange(2 * S * d, dtype=np.float64).reshape(2, S, d)
    for B_, cu in ((2, None), (1, [0, 0, 0])):
        dxp, da, dh0 = backward.adjoint(cell, np.zeros((B_, 0, G, d)), np.zeros((G, d)), np.zeros((B_, 0, S, d)),
                                        np.zeros((B_, 0, d)), cu_seqlens=cu, dstate_last=dsl)
        assert dxp.shape == (B_, 0, G, d) and np.all(da == 0.0) and np.array_equal(dh0, dsl)
