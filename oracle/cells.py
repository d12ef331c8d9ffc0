"""Diagonal GRU and LSTM cells and their exact per-channel Jacobians (float64).

The pages do not print the cell equations; they name diagonal ("mix='diag'")
GRU and LSTM cells (shapes/layout page, support table) whose recurrent
weight is a per-channel vector a instead of a matrix.  The forms used here:

GRU (gates z, r, c; state h):
    z = sig(x_z + a_z h)      r = sig(x_r + a_r h)
    c = tanh(x_c + a_c (r h)) h' = (1 - z) h + z c

LSTM (gates i, f, o, g; state s = (c, h)); the textbook LSTM without
peepholes, recurrent matrix replaced by diag(a):
    i = sig(x_i + a_i h)  f = sig(x_f + a_f h)  o = sig(x_o + a_o h)
    g = tanh(x_g + a_g h) c' = f c + i g        h' = o tanh(c')

x_* are the projected inputs (bias included).  Array conventions: a state is
(..., S, d) with S = 1 (GRU: h) or 2 (LSTM: c, h); projected inputs are
(..., G, d); a is (G, d).  Jacobians are (..., S, S, d) with
J[..., p, q, :] = d s'_p / d s_q.  Channels never interact, so the Jacobian
of the whole state is block diagonal with one S x S block per channel; the
LSTM block is the full 2 x 2 (dropping its off-diagonal terms would turn
Newton into a quasi-Newton method).
"""
from __future__ import annotations

import numpy as np


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


# ---------------------------------------------------------------- GRU ---

def gru_gates(s, xp, a):
    h = s[..., 0, :]
    z = sigmoid(xp[..., 0, :] + a[0] * h)
    r = sigmoid(xp[..., 1, :] + a[1] * h)
    c = np.tanh(xp[..., 2, :] + a[2] * (r * h))
    return h, z, r, c


def gru_f(s, xp, a):
    h, z, r, c = gru_gates(s, xp, a)
    return ((1.0 - z) * h + z * c)[..., None, :]


def gru_jac(s, xp, a):
    """d h'/d h by the product and chain rules applied to gru_f."""
    h, z, r, c = gru_gates(s, xp, a)
    dz = z * (1.0 - z) * a[0]
    dr = r * (1.0 - r) * a[1]
    dc = (1.0 - c * c) * a[2] * (r + h * dr)
    J = (1.0 - z) + (c - h) * dz + z * dc
    return J[..., None, None, :]


# --------------------------------------------------------------- LSTM ---

def lstm_gates(s, xp, a):
    c, h = s[..., 0, :], s[..., 1, :]
    i = sigmoid(xp[..., 0, :] + a[0] * h)
    f = sigmoid(xp[..., 1, :] + a[1] * h)
    o = sigmoid(xp[..., 2, :] + a[2] * h)
    g = np.tanh(xp[..., 3, :] + a[3] * h)
    return c, h, i, f, o, g


def lstm_f(s, xp, a):
    c, h, i, f, o, g = lstm_gates(s, xp, a)
    c1 = f * c + i * g
    h1 = o * np.tanh(c1)
    return np.stack([c1, h1], axis=-2)


def lstm_jac(s, xp, a):
    """2x2 per-channel block d(c', h')/d(c, h)."""
    c, h, i, f, o, g = lstm_gates(s, xp, a)
    c1 = f * c + i * g
    tc = np.tanh(c1)
    di = i * (1.0 - i) * a[0]
    df = f * (1.0 - f) * a[1]
    do = o * (1.0 - o) * a[2]
    dg = (1.0 - g * g) * a[3]
    dc1_dc = f
    dc1_dh = c * df + g * di + i * dg
    dtc = 1.0 - tc * tc
    dh1_dc = o * dtc * dc1_dc
    dh1_dh = tc * do + o * dtc * dc1_dh
    J = np.empty(c.shape[:-1] + (2, 2) + c.shape[-1:], dtype=np.float64)
    J[..., 0, 0, :] = dc1_dc
    J[..., 0, 1, :] = dc1_dh
    J[..., 1, 0, :] = dh1_dc
    J[..., 1, 1, :] = dh1_dh
    return J


# ---------------------------------------- input and weight partials ---
# For the backward pass: d s'/d x_g and d s'/d a_g, per channel, as arrays
# (..., S, G, d) with [..., p, g, :] = d s'_p / d x_g (resp. d a_g).  Every
# gate is a function of its pre-activation u_g = x_g + a_g * m_g, where the
# multiplier m_g is h for every gate except the GRU candidate (m_c = r h);
# so d/d x_g = d/d u_g and d/d a_g = m_g d/d u_g.

def gru_dx(s, xp, a):
    """d h'/d x_g for g = z, r, c (chain rule through the pre-activations)."""
    h, z, r, c = gru_gates(s, xp, a)
    du_z = (c - h) * z * (1.0 - z)
    du_c = z * (1.0 - c * c)
    du_r = du_c * a[2] * h * r * (1.0 - r)
    return np.stack([du_z, du_r, du_c], axis=-2)[..., None, :, :]


def gru_da(s, xp, a):
    h, z, r, c = gru_gates(s, xp, a)
    d = gru_dx(s, xp, a)
    m = np.stack([h, h, r * h], axis=-2)[..., None, :, :]
    return d * m


def lstm_dx(s, xp, a):
    """d (c', h')/d x_g for g = i, f, o, g."""
    c, h, i, f, o, g = lstm_gates(s, xp, a)
    c1 = f * c + i * g
    tc = np.tanh(c1)
    dc = np.stack([g * i * (1.0 - i), c * f * (1.0 - f), np.zeros_like(c), i * (1.0 - g * g)], axis=-2)
    dh = o[..., None, :] * (1.0 - tc * tc)[..., None, :] * dc
    dh[..., 2, :] = tc * o * (1.0 - o)
    return np.stack([dc, dh], axis=-3)


def lstm_da(s, xp, a):
    c, h = s[..., 0, :], s[..., 1, :]
    return lstm_dx(s, xp, a) * h[..., None, None, :]


CELLS = {
    "gru": (3, 1, gru_f, gru_jac),
    "lstm": (4, 2, lstm_f, lstm_jac),
}
PARTIALS = {
    "gru": (gru_dx, gru_da),
    "lstm": (lstm_dx, lstm_da),
}


def cell_fns(cell: str):
    """(G, S, f, jac) for a cell name."""
    return CELLS[cell]


def cell_partials(cell: str):
    """(dx, da) for a cell name: d s'/d x and d s'/d a, shaped (..., S, G, d)."""
    return PARTIALS[cell]
