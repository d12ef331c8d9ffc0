"""Pins for the oracle's cells and Jacobians (CPU only).

The cells are pinned against PyTorch's own GRUCell / LSTMCell (a library
routine) on the special case where the recurrent matrices are diagonal and
the input weights only route the projected gates; gate roles are pinned by
saturating limits; the closed-form Jacobians by central finite differences.
"""
import numpy as np
import pytest
import torch

from oracle import cells

RNG = np.random.default_rng(123)


def _rand(shape, scale=1.0):
    return scale * RNG.standard_normal(shape)


def test_gru_matches_torch_grucell_with_diagonal_recurrence():
    d, n = 7, 5
    xp = _rand((n, 3, d))
    h = _rand((n, 1, d), 0.7)
    a = RNG.uniform(-0.5, 0.5, (3, d))
    cellt = torch.nn.GRUCell(3 * d, d, bias=False).double()
    I = torch.eye(d, dtype=torch.float64)
    Z = torch.zeros(d, d, dtype=torch.float64)
    # torch gate order (r, z, n); torch keeps z*h, so its z is 1 - ours:
    # sigma(-u) = 1 - sigma(u) -> negate the z input and its recurrent weight.
    w_ih = torch.cat([torch.cat([Z, I, Z], 1), torch.cat([-I, Z, Z], 1), torch.cat([Z, Z, I], 1)], 0)
    a_t = torch.from_numpy(a)
    w_hh = torch.cat([torch.diag(a_t[1]), torch.diag(-a_t[0]), torch.diag(a_t[2])], 0)
    with torch.no_grad():
        cellt.weight_ih.copy_(w_ih)
        cellt.weight_hh.copy_(w_hh)
        ref = cellt(torch.from_numpy(xp.reshape(n, 3 * d)), torch.from_numpy(h[:, 0])).numpy()
    got = cells.gru_f(h, xp, a)[:, 0]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_lstm_matches_torch_lstmcell_with_diagonal_recurrence():
    d, n = 6, 4
    xp = _rand((n, 4, d))
    s = _rand((n, 2, d), 0.8)
    a = RNG.uniform(-0.5, 0.5, (4, d))
    cellt = torch.nn.LSTMCell(4 * d, d, bias=False).double()
    I = torch.eye(d, dtype=torch.float64)
    Z = torch.zeros(d, d, dtype=torch.float64)

    def sel(k):  # rows that pick gate block k of [i|f|o|g]
        return torch.cat([I if j == k else Z for j in range(4)], 1)

    # torch gate order (i, f, g, o)
    w_ih = torch.cat([sel(0), sel(1), sel(3), sel(2)], 0)
    a_t = torch.from_numpy(a)
    w_hh = torch.cat([torch.diag(a_t[0]), torch.diag(a_t[1]), torch.diag(a_t[3]), torch.diag(a_t[2])], 0)
    with torch.no_grad():
        cellt.weight_ih.copy_(w_ih)
        cellt.weight_hh.copy_(w_hh)
        h1, c1 = cellt(torch.from_numpy(xp.reshape(n, 4 * d)),
                       (torch.from_numpy(s[:, 1]), torch.from_numpy(s[:, 0])))
    got = cells.lstm_f(s, xp, a)
    np.testing.assert_allclose(got[:, 0], c1.numpy(), rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[:, 1], h1.numpy(), rtol=0, atol=1e-14)


def test_gru_gate_roles_by_saturation():
    d = 5
    h = _rand((1, d), 0.6)
    a = RNG.uniform(-0.5, 0.5, (3, d))
    xp = _rand((3, d))
    xp[0] = -80.0                     # update gate shut: state carried over unchanged
    np.testing.assert_allclose(cells.gru_f(h, xp, a)[0], h[0], atol=1e-30)
    xp[0] = 80.0
    xp[2] = 80.0                      # gate open, candidate saturated at +1
    np.testing.assert_allclose(cells.gru_f(h, xp, a)[0], 1.0, atol=1e-15)
    xp[2] = -80.0
    np.testing.assert_allclose(cells.gru_f(h, xp, a)[0], -1.0, atol=1e-15)
    # reset gate shut: candidate sees no state, tanh(x_c)
    xp[1] = -80.0
    xp[2] = 0.3
    np.testing.assert_allclose(cells.gru_f(h, xp, a)[0], np.tanh(0.3), atol=1e-15)


def test_lstm_gate_roles_by_saturation():
    d = 5
    s = _rand((2, d), 0.6)
    a = RNG.uniform(-0.5, 0.5, (4, d))
    xp = _rand((4, d))
    xp[0], xp[1], xp[2] = -80.0, 80.0, 80.0   # input shut, forget open, output open
    out = cells.lstm_f(s, xp, a)
    np.testing.assert_allclose(out[0], s[0], atol=1e-15)
    np.testing.assert_allclose(out[1], np.tanh(s[0]), atol=1e-15)
    xp[2] = -80.0                              # output shut -> h' = 0
    np.testing.assert_allclose(cells.lstm_f(s, xp, a)[1], 0.0, atol=1e-30)
    xp[0], xp[1], xp[2], xp[3] = 80.0, -80.0, 80.0, 80.0   # write g=1, forget all
    out = cells.lstm_f(s, xp, a)
    np.testing.assert_allclose(out[0], 1.0, atol=1e-15)
    np.testing.assert_allclose(out[1], np.tanh(1.0), atol=1e-15)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_jacobian_matches_central_differences(cell):
    G, S, f, jac = cells.cell_fns(cell)
    d, n = 9, 6
    xp = _rand((n, G, d))
    s = _rand((n, S, d), 0.9)
    a = RNG.uniform(-0.5, 0.5, (G, d))
    J = jac(s, xp, a)
    eps = 1e-6
    for q in range(S):
        e = np.zeros_like(s)
        e[:, q, :] = eps
        fd = (f(s + e, xp, a) - f(s - e, xp, a)) / (2 * eps)   # (n, S, d): column q
        np.testing.assert_allclose(J[:, :, q, :], fd, rtol=0, atol=1e-8)
    # the Jacobian does depend on every recurrent weight: a = 0 kills the state
    # dependence of the gates, leaving the GRU's 1 - z and the LSTM's forget gate
    J0 = jac(s, xp, np.zeros_like(a))
    if cell == "gru":
        z = cells.sigmoid(xp[:, 0])
        np.testing.assert_allclose(J0[:, 0, 0], 1 - z, atol=1e-15)
    else:
        fg = cells.sigmoid(xp[:, 1])
        np.testing.assert_allclose(J0[:, 0, 0], fg, atol=1e-15)
        np.testing.assert_allclose(J0[:, 0, 1], 0.0, atol=1e-15)
