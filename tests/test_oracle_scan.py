"""Pins for the exact affine scan and the oracle's float recurrence (CPU only)."""
from fractions import Fraction
import random

import numpy as np
import pytest

from oracle import scan
from oracle.newton import affine_recurrence

R = random.Random(7)


def rand_map(S, head=False):
    def q():
        return Fraction(R.randint(-9, 9), R.randint(1, 5))
    A = [[Fraction(0) if head else q() for _ in range(S)] for _ in range(S)]
    b = [q() for _ in range(S)]
    return (A, b)


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 6])
def test_every_bracketing_gives_the_serial_result(S, T):
    maps = [rand_map(S) for _ in range(T)]
    s0 = [Fraction(R.randint(-5, 5), 3) for _ in range(S)]
    total = scan.all_bracketings(maps)
    assert len(total) == 1                      # associativity: one composite
    (comp,) = total
    serial = scan.serial_states(maps, s0)[-1]
    assert scan.apply((list(map(list, comp[0])), list(comp[1])), s0) == serial
    assert scan.count_bracketings(T) == [1, 1, 2, 5, 14, 42][T - 1 if T <= 6 else 0]


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("T", [1, 4, 7, 9])
def test_three_phase_equals_serial_for_every_chunk_length(S, T):
    maps = [rand_map(S, head=(t in (0, 3, 4))) for t in range(T)]
    s0 = [Fraction(R.randint(-5, 5), 7) for _ in range(S)]
    ref = scan.serial_states(maps, s0)
    for L in range(1, T + 1):
        assert scan.three_phase(maps, s0, L) == ref


def test_head_map_annihilates_the_carry():
    h = rand_map(2, head=True)
    m = rand_map(2)
    c = scan.compose(h, m)
    assert all(v == 0 for row in c[0] for v in row)
    assert scan.apply(c, [Fraction(123), Fraction(-7)]) == h[1]


@pytest.mark.parametrize("S", [1, 2])
def test_float_recurrence_is_exact_on_dyadic_data(S):
    """The oracle's float64 serial recurrence equals the rational serial loop.

    Entries are small dyadic numbers with few bits, so every float operation
    is exact; a transposed 2x2 block or a wrong time index would show up.
    """
    T, d = 6, 3
    rng = np.random.default_rng(3)
    J = rng.integers(-4, 5, (1, T, S, S, d)) / 4.0
    b = rng.integers(-8, 9, (1, T, S, d)) / 8.0
    J[:, 0] = 0.0
    got = affine_recurrence(J, b)
    for ch in range(d):
        maps = [([[Fraction(J[0, t, p, q, ch]) for q in range(S)] for p in range(S)],
                 [Fraction(b[0, t, p, ch]) for p in range(S)]) for t in range(T)]
        ref = scan.serial_states(maps, [Fraction(0)] * S)
        for t in range(T):
            for p in range(S):
                assert Fraction(got[0, t, p, ch]) == ref[t][p]
