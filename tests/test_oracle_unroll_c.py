"""The C unroll (oracle/c/unroll.c) against the NumPy oracle's unroll: two
independent float64 implementations of the same recurrence, rectangular
batches and a ragged pack with empty segments and h0."""
import numpy as np
import pytest

from oracle import newton as onewton
from oracle import unroll_c


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_c_unroll_equals_numpy_unroll(cell):
    G, S = (3, 1) if cell == "gru" else (4, 2)
    rng = np.random.default_rng(5)
    xp = rng.standard_normal((3, 300, G, 37)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (G, 37))
    h0 = 0.5 * rng.standard_normal((3, S, 37))
    ref, _ = onewton.sequential(cell, xp.astype(np.float64), a, h0=h0)
    got = unroll_c.unroll(cell, xp, a, h0=h0)
    assert np.abs(got - ref[..., -1, :]).max() <= 1e-12


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_c_unroll_ragged_pack(cell):
    G, S = (3, 1) if cell == "gru" else (4, 2)
    rng = np.random.default_rng(6)
    cu = np.array([0, 0, 17, 17, 18, 250, 400], dtype=np.int32)
    xp = rng.standard_normal((1, 400, G, 20)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (G, 20))
    h0 = 0.5 * rng.standard_normal((len(cu) - 1, S, 20))
    ref, _ = onewton.sequential(cell, xp.astype(np.float64), a, h0=h0, cu_seqlens=cu)
    got = unroll_c.unroll(cell, xp, a, h0=h0, cu_seqlens=cu)
    assert np.abs(got - ref[..., -1, :]).max() <= 1e-12
