"""Pins of the oracle's K*(T) definition against what the mathematics fixes."""
import numpy as np
import pytest

from oracle import kstar, newton

RNG = np.random.default_rng(21)


def inputs(cell, B, T, d, a_scale=0.5):
    G = 3 if cell == "gru" else 4
    return RNG.standard_normal((B, T, G, d)), RNG.uniform(-a_scale, a_scale, (G, d))


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_newton_is_exact_after_T_iterations(cell):
    """Newton's k-th iterate is exact on the first k steps, so K = T agrees
    to rounding and K* <= T for any tau above rounding."""
    xp, a = inputs(cell, 2, 6, 3)
    errs = kstar.agreement_errors(cell, xp, a, 6)
    assert errs[-1] <= 1e-13
    assert kstar.kstar(errs, 1e-10) <= 6


def test_gru_with_zero_recurrent_weight_needs_one_iteration():
    """a = 0: the GRU's gates do not depend on h, the map is affine in h, and
    one Newton step is exact (K* = 1 for every tau above rounding)."""
    xp, _ = inputs("gru", 2, 50, 4)
    errs = kstar.agreement_errors("gru", xp, np.zeros((3, 4)), 3)
    assert errs[0] <= 1e-12 and kstar.kstar(errs, 1e-10) == 1


def test_lstm_with_zero_recurrent_weight_needs_two_iterations():
    """a = 0: h' depends on c nonlinearly (tanh) but c' is affine in c, so the
    first iterate gets c exact and the second gets h exact."""
    xp, _ = inputs("lstm", 1, 40, 3)
    errs = kstar.agreement_errors("lstm", xp, np.zeros((4, 3)), 3)
    assert errs[0] > 1e-6 and errs[1] <= 1e-12
    assert kstar.kstar(errs, 1e-10) == 2


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_errors_fall_with_K_and_kstar_is_the_first_under_tau(cell):
    xp, a = inputs(cell, 2, 300, 4)
    errs = kstar.agreement_errors(cell, xp, a, 6)
    k = kstar.kstar(errs, 1e-4)
    assert k is not None and errs[k - 1] <= 1e-4 and all(e > 1e-4 for e in errs[:k - 1])
    assert errs[-1] <= errs[0]


def test_kstar_none_and_table_monotone():
    assert kstar.kstar([1.0, 0.5], 1e-4) is None
    assert kstar.k_table({64: 2, 1024: 3, 256: 2, 4096: 2}) == {64: 2, 256: 2, 1024: 3, 4096: 3}


def test_table_is_resolved_like_the_pages_table():
    """The table feeds resolve_k (smallest key >= T, else the largest)."""
    tab = kstar.k_table({64: 2, 1024: 3})
    assert newton.resolve_k(64, tab) == 2 and newton.resolve_k(65, tab) == 3 and newton.resolve_k(10 ** 6, tab) == 3
