"""Pins for the oracle's sequential unroll, Newton iteration and residual (CPU only).

What the pages and the mathematics fix, independent of the code under test:
  * after k Newton iterations from a fixed h0 the first k steps of every
    sequence are exact, so K = T reproduces the unroll (holds for any J, pins
    indexing and segment heads);
  * with a = 0 the GRU is affine in h (K = 1 is exact, and equals the closed
    cumulative-product solution) and the LSTM's cell state is affine (K = 2
    is exact): the parallel scan solves a linear recurrence exactly;
  * Newton converges quadratically when J is the true Jacobian, and a Picard
    sweep (J := 0) is far worse at the same K (this pins J inside Newton);
  * fp32 agreement with the unroll at K = 3 within tau = 1e-4 on the small
    GRU workload (FAQs "Does parallel Newton match sequential unroll?");
  * a ragged pack equals its segments run one by one (J = 0 at heads);
  * the residual of the exact trajectory is zero, a single perturbation is
    read back exactly, and non-finite values trip the gate.
"""
import numpy as np
import pytest

from oracle import cells, newton, rounding
from workloads import WORKLOADS, make_inputs, random_state, segment_lengths
from oracle.proj import input_proj


def small_problem(cell, B=2, T=40, d=5, seed=0, scale=1.0):
    G = cells.cell_fns(cell)[0]
    rng = np.random.default_rng(seed)
    xp = scale * rng.standard_normal((B, T, G, d))
    if cell == "lstm":
        xp[:, :, 1] += 1.0
    a = rng.uniform(-0.5, 0.5, (G, d))
    return xp, a


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_first_k_steps_exact_and_K_equals_T(cell):
    xp, a = small_problem(cell, B=2, T=12, d=4)
    S = cells.cell_fns(cell)[1]
    h0 = np.random.default_rng(1).standard_normal((2, S, 4)) * 0.5
    seq, _ = newton.sequential(cell, xp, a, h0=h0)
    for k in range(1, 13):
        out = newton.newton(cell, xp, a, k, h0=h0)
        np.testing.assert_allclose(out["H"][:, :k], seq[:, :k], rtol=0, atol=1e-13)
        if k < 3:   # later steps are not yet converged (this also checks the test bites)
            assert np.abs(out["H"][:, k:] - seq[:, k:]).max() > 1e-9
    np.testing.assert_allclose(out["H"], seq, rtol=0, atol=1e-13)
    assert out["residuals"][-1] < 1e-13


def test_first_k_steps_exact_in_every_segment_of_a_pack():
    cell = "gru"
    xp, a = small_problem(cell, B=1, T=30, d=3, seed=4)
    cu = np.array([0, 7, 7, 19, 30])          # includes an empty segment
    h0 = np.random.default_rng(2).standard_normal((4, 1, 3)) * 0.5
    seq, last = newton.sequential(cell, xp, a, h0=h0, cu_seqlens=cu)
    for k in (1, 2, 3):
        out = newton.newton(cell, xp, a, k, h0=h0, cu_seqlens=cu)
        for j in range(4):
            lo, hi = cu[j], min(cu[j] + k, cu[j + 1])
            np.testing.assert_allclose(out["H"][0, lo:hi], seq[0, lo:hi], atol=1e-13)
    np.testing.assert_array_equal(last[1], h0[1])   # empty segment keeps its h0


def test_gru_linear_case_exact_at_K1_and_matches_closed_form():
    xp, a = small_problem("gru", B=1, T=9, d=3, seed=5)
    a0 = np.zeros_like(a)
    h0 = np.array([[[0.3, -0.2, 0.7]]])
    seq, _ = newton.sequential("gru", xp, a0, h0=h0)
    out = newton.newton("gru", xp, a0, 1, h0=h0)
    np.testing.assert_allclose(out["H"], seq, atol=1e-15)
    # closed form of h_t = (1 - z_t) h_{t-1} + z_t c_t with constant gates
    z = cells.sigmoid(xp[0, :, 0])
    c = np.tanh(xp[0, :, 2])
    for t in range(9):
        acc = np.prod(1 - z[:t + 1], axis=0) * h0[0, 0]
        for j in range(t + 1):
            acc = acc + np.prod(1 - z[j + 1:t + 1], axis=0) * z[j] * c[j]
        np.testing.assert_allclose(out["H"][0, t, 0], acc, atol=1e-15)


def test_lstm_linear_case_exact_at_K2_not_K1():
    xp, a = small_problem("lstm", B=2, T=20, d=4, seed=6)
    a0 = np.zeros_like(a)
    seq, _ = newton.sequential("lstm", xp, a0)
    o1 = newton.newton("lstm", xp, a0, 1)
    o2 = newton.newton("lstm", xp, a0, 2)
    np.testing.assert_allclose(o1["H"][..., 0, :], seq[..., 0, :], atol=1e-14)  # c is affine
    assert np.abs(o1["H"][..., 1, :] - seq[..., 1, :]).max() > 1e-3
    np.testing.assert_allclose(o2["H"], seq, atol=1e-14)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_quadratic_convergence_and_picard_is_worse(cell):
    xp, a = small_problem(cell, B=1, T=512, d=16, seed=7)
    seq, _ = newton.sequential(cell, xp, a)
    errs = [np.abs(newton.newton(cell, xp, a, k)["H"] - seq).max() for k in range(1, 6)]
    # strictly decreasing, and each step roughly squares the error while it is
    # well above round-off: log e_{k+1} / log e_k >= 1.5
    for k in range(len(errs) - 1):
        if errs[k] < 1e-7:
            break
        assert errs[k + 1] < errs[k]
        if errs[k] < 0.2:
            assert np.log(errs[k + 1]) / np.log(errs[k]) > 1.5, errs
    pic = np.abs(newton.newton(cell, xp, a, 3, jacobian=False)["H"] - seq).max()
    assert pic > 100 * errs[2]


def test_tau_claim_small_gru_workload_fp32_storage():
    w = WORKLOADS["gru_tiny"]
    inp = make_inputs(w)
    xp = input_proj(inp["x"].astype(np.float64), inp["W"].astype(np.float64),
                    inp["bias"].astype(np.float64), w.G)
    xp = rounding.store(xp, "f32")
    seq, _ = newton.sequential("gru", xp, inp["a"])
    out = newton.newton("gru", xp, inp["a"], w.K, dtype="f32")
    assert np.abs(out["H"] - seq).max() <= 1e-4
    # and two iterations are not enough: the claim is not vacuous
    out2 = newton.newton("gru", xp, inp["a"], 2, dtype="f32")
    assert np.abs(out2["H"] - seq).max() > 1e-4


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_ragged_pack_equals_segments_run_alone(cell):
    xp, a = small_problem(cell, B=1, T=50, d=3, seed=8)
    S = cells.cell_fns(cell)[1]
    cu = np.array([0, 11, 11, 30, 31, 50])
    h0 = np.random.default_rng(9).standard_normal((5, S, 3)) * 0.4
    for K in (1, 2, 3):
        pk = newton.newton(cell, xp, a, K, h0=h0, cu_seqlens=cu)
        res = []
        for j in range(5):
            lo, hi = cu[j], cu[j + 1]
            if hi == lo:
                np.testing.assert_array_equal(pk["last"][j], h0[j])
                continue
            one = newton.newton(cell, xp[:, lo:hi], a, K, h0=h0[j:j + 1])
            np.testing.assert_array_equal(pk["H"][0, lo:hi], one["H"][0])
            np.testing.assert_array_equal(pk["last"][j], one["last"][0])
            res.append(one["residuals"])
        np.testing.assert_allclose(pk["residuals"], np.max(res, axis=0), rtol=0, atol=0)
    seq, last = newton.sequential(cell, xp, a, h0=h0, cu_seqlens=cu)
    for j in range(5):
        lo, hi = cu[j], cu[j + 1]
        if hi > lo:
            s1, l1 = newton.sequential(cell, xp[:, lo:hi], a, h0=h0[j:j + 1])
            np.testing.assert_array_equal(seq[0, lo:hi], s1[0])
            np.testing.assert_array_equal(last[j], l1[0])


def test_residual_properties():
    cell = "lstm"
    xp, a = small_problem(cell, B=1, T=30, d=4, seed=10)
    heads = newton.head_segments(1, 30)
    H0 = np.zeros((1, 2, 4))
    seq, _ = newton.sequential(cell, xp, a)
    assert newton.residual(cell, seq, xp, a, heads, H0) < 1e-15
    # r_0 is the size of f at the zero state
    r0 = newton.newton(cell, xp, a, 1)["residuals"][0]
    assert r0 == pytest.approx(np.abs(cells.lstm_f(np.zeros((1, 30, 2, 4)), xp, a)).max(), abs=0)
    # a single perturbation at the last step is read back exactly
    P = seq.copy()
    P[0, -1, 1, 2] += 0.125
    assert newton.residual(cell, P, xp, a, heads, H0) == pytest.approx(0.125, abs=1e-15)
    # non-finite inputs give +Inf, never NaN or a silently small number
    xq = xp.copy()
    xq[0, 5, 0, 1] = np.nan
    out = newton.newton(cell, xq, a, 2)
    assert out["residuals"][-1] == np.inf


def test_storage_rounding_of_iterates():
    xp, a = small_problem("gru", B=1, T=64, d=8, seed=11)
    o64 = newton.newton("gru", xp, a, 3, dtype="f64")
    o16 = newton.newton("gru", xp, a, 3, dtype="bf16")
    np.testing.assert_array_equal(o16["H"], rounding.bf16_round(o16["H"]))
    diff = np.abs(o16["H"] - o64["H"]).max()
    assert 0 < diff < 2e-2


def test_resolve_k_table():
    tab = {64: 2, 1024: 3, 8192: 4}
    assert newton.resolve_k(1, tab) == 2
    assert newton.resolve_k(64, tab) == 2
    assert newton.resolve_k(65, tab) == 3
    assert newton.resolve_k(1024, tab) == 3
    assert newton.resolve_k(5000, tab) == 4
    assert newton.resolve_k(10 ** 6, tab) == 4


def test_workload_generator_shapes_and_determinism():
    for name, w in WORKLOADS.items():
        if w.tokens * w.d_in > 2 ** 22:
            continue
        i1, i2 = make_inputs(w), make_inputs(w)
        assert i1["x"].shape == (w.B, w.T, w.d_in)
        assert i1["W"].shape == (w.G * w.d_h, w.d_in)
        np.testing.assert_array_equal(i1["x"], i2["x"])
    rng = np.random.default_rng(0)
    L = segment_lengths(rng, 64, 65536, 64, 2048)
    assert L.sum() == 65536 and L.min() > 0
    st = random_state(WORKLOADS["lstm_t131k"], 3, seed=1)
    assert st.shape == (3, 2, 256)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_picard_warm_start(cell):
    """P Jacobi sweeps from 0 are exact on the first P steps; k Newton
    iterations from that guess are exact on the first P + k steps; P = T
    sweeps alone are the unroll; and r_0 is the residual of the guess."""
    from oracle import newton as on
    rng = np.random.default_rng(17)
    G = 3 if cell == "gru" else 4
    S = 1 if cell == "gru" else 2
    B, T, d = 2, 12, 3
    xp = rng.standard_normal((B, T, G, d))
    a = rng.uniform(-0.5, 0.5, (G, d))
    h0 = rng.standard_normal((B, S, d)) * 0.3
    seq, _ = on.sequential(cell, xp, a, h0=h0)
    for P in (1, 2, 3):
        out = on.newton(cell, xp, a, 2, h0=h0, picard=P, keep_iterates=True)
        for k, Hk in enumerate(out["iterates"], start=1):
            assert np.abs(Hk[:, :P + k] - seq[:, :P + k]).max() <= 1e-13
    full = on.newton(cell, xp, a, 1, h0=h0, picard=T)
    assert np.abs(full["H"] - seq).max() <= 1e-13 and full["residuals"][0] <= 1e-13
    # in a ragged pack the guess restarts at every head: after P sweeps and
    # k iterations the first P + k steps of every segment are exact, also in
    # segments shorter than P
    cu = np.array([0, 1, 4, 12, 13, 24], dtype=np.int32)
    xq = xp[:1].reshape(1, T, G, d).repeat(2, axis=1)
    hq = rng.standard_normal((len(cu) - 1, S, d)) * 0.3
    sq, _ = on.sequential(cell, xq, a, h0=hq, cu_seqlens=cu)
    for P in (2, 5):
        out = on.newton(cell, xq, a, 1, h0=hq, cu_seqlens=cu, picard=P, keep_iterates=True)
        for lo, hi in zip(cu[:-1], cu[1:]):
            m = min(hi, lo + P + 1)
            assert np.abs(out["H"][:, lo:m] - sq[:, lo:m]).max() <= 1e-13
        if P == 2:   # and not beyond: the segment of 11 steps is not solved at step 3
            assert np.abs(out["H"][:, 4:12] - sq[:, 4:12]).max() > 1e-8
    g1 = on.newton(cell, xp, a, 1, h0=h0, picard=1)
    _, _, f, _ = cells.cell_fns(cell)
    guess = f(np.concatenate([h0[:, None], np.zeros((B, T - 1, S, d))], axis=1), xp, a)  # one sweep from 0
    heads = on.head_segments(B, T)
    assert g1["residuals"][0] == on.residual(cell, guess, xp, a, heads, h0)


def test_oracle_reproduces_the_recorded_convergence_of_the_tiny_gru():
    """The oracle, fed by the workload generator, reproduces the errors and
    residuals an independent float64 script recorded for the 1 x 1024 GRU
    workload (tests/golden/gru_tiny_newton_convergence.txt).  This pins the
    input recipe (draw order, float64 draws cast to float32, W scaling) and
    the oracle's Newton and residual together."""
    import os

    from oracle import proj as oproj
    from oracle import rounding as oround
    from workloads import WORKLOADS, make_inputs

    path = os.path.join(os.path.dirname(__file__), "golden", "gru_tiny_newton_convergence.txt")
    rows = [list(map(float, ln.split())) for ln in open(path) if ln.strip() and not ln.startswith("#")]
    w = WORKLOADS["gru_tiny"]
    inp = make_inputs(w, seed=0)
    xp = oproj.input_proj(oround.load(inp["x"], "f32"), oround.load(inp["W"], "f32"),
                          inp["bias"].astype(np.float64), w.G)
    a = inp["a"].astype(np.float64)
    seq, _ = newton.sequential("gru", xp, a)
    for K, err_want, r_want in rows:
        out = newton.newton("gru", xp, a, int(K))
        err = np.abs(out["H"][..., 0, :] - seq[..., 0, :]).max()
        assert abs(err - err_want) <= 5e-3 * err_want, (K, err, err_want)
        r = out["residuals"][int(K) - 1]
        assert abs(r - r_want) <= 5e-3 * r_want, (K, r, r_want)
