"""Pins of the head-mix GRU oracle (dense d_head x d_head recurrent blocks).

Each pin checks the oracle against something other than itself:
  * the Jacobian blocks against central finite differences of f (every
    entry, float64, step 1e-6);
  * diagonal blocks against the diagonal GRU of cells.py / newton.py, which
    is written independently (per-channel formulas, no matrices);
  * the dense affine recurrence against an explicit product of the step
    maps composed right to left;
  * the Newton invariants the pages' method fixes: after k iterations from
    zero the first k steps are exact, K = T reproduces the unroll, and
    convergence near the solution is quadratic;
  * head independence: a block-diagonal recurrence never couples heads.
"""
import numpy as np
import pytest

from oracle import cells, headmix, newton

EPS = 1e-6


def inputs(B, T, d_h, d_head, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    xp = rng.standard_normal((B, T, 3, d_h))
    A = rng.uniform(-scale, scale, (3, d_h // d_head, d_head, d_head)) / np.sqrt(d_head)
    h0 = 0.5 * rng.standard_normal((B, d_h))
    return xp, A, h0


@pytest.mark.parametrize("d_head", [1, 2, 4, 16])
def test_jacobian_blocks_match_finite_differences(d_head):
    d_h = 16
    xp, A, h0 = inputs(2, 1, d_h, d_head, seed=d_head, scale=1.5)
    x, h = xp[:, 0], h0
    J = headmix.jac(h, x, A)
    assert J.shape == (2, d_h // d_head, d_head, d_head)
    for b in range(2):
        for col in range(d_h):
            hp, hm = h.copy(), h.copy()
            hp[b, col] += EPS
            hm[b, col] -= EPS
            fd = (headmix.f(hp, x, A) - headmix.f(hm, x, A))[b] / (2 * EPS)
            k, j = divmod(col, d_head)
            for row in range(d_h):
                k2, i = divmod(row, d_head)
                want = J[b, k, i, j] if k2 == k else 0.0   # no coupling across heads
                assert abs(fd[row] - want) <= 1e-8, (b, row, col)


@pytest.mark.parametrize("d_head", [1, 4])
def test_diagonal_blocks_are_the_diagonal_gru(d_head):
    """A_g with diagonal blocks diag(a_g) gives the per-channel diagonal GRU:
    same step, same Jacobian, same unroll, same Newton iterates."""
    rng = np.random.default_rng(7)
    B, T, d_h = 2, 40, 8
    xp = rng.standard_normal((B, T, 3, d_h))
    a = rng.uniform(-0.5, 0.5, (3, d_h))
    A = np.zeros((3, d_h // d_head, d_head, d_head))
    for g in range(3):
        for k in range(d_h // d_head):
            A[g, k] = np.diag(a[g, k * d_head:(k + 1) * d_head])
    h = rng.standard_normal((B, d_h))
    s = h[:, None, :]
    assert np.allclose(headmix.f(h, xp[:, 0], A), cells.gru_f(s, xp[:, 0], a)[:, 0], rtol=0, atol=1e-15)
    Jd = cells.gru_jac(s, xp[:, 0], a)[:, 0, 0]                   # (B, d_h)
    Jh = headmix.jac(h, xp[:, 0], A)
    diag = np.stack([np.diagonal(Jh[:, k], axis1=-2, axis2=-1) for k in range(d_h // d_head)], 1).reshape(B, d_h)
    assert np.allclose(diag, Jd, rtol=0, atol=1e-15)
    off = Jh.copy()
    for k in range(d_h // d_head):
        off[:, k] -= np.einsum("bi,ij->bij", diag.reshape(B, -1, d_head)[:, k], np.eye(d_head))
    assert np.abs(off).max() <= 1e-15
    H, last = headmix.sequential(xp, A, h0=h)
    Hd, lastd = newton.sequential("gru", xp, a, h0=s)
    assert np.allclose(H, Hd[:, :, 0], rtol=0, atol=1e-13)
    nh = headmix.newton(xp, A, 3, h0=h)
    nd = newton.newton("gru", xp, a, 3, h0=s)
    assert np.allclose(nh["H"], nd["H"][:, :, 0], rtol=0, atol=1e-12)
    assert np.allclose(nh["residuals"], nd["residuals"], rtol=1e-10, atol=1e-14)


def test_dense_affine_recurrence_equals_the_composed_maps():
    """h_T from the serial recurrence equals the product of the step maps
    composed right to left (M = J_T ... J_1, v accumulated) applied to 0."""
    rng = np.random.default_rng(3)
    B, T, nh, dhd = 1, 7, 2, 3
    J = rng.standard_normal((B, T, nh, dhd, dhd)) * 0.7
    b = rng.standard_normal((B, T, nh * dhd))
    out = headmix.affine_recurrence(J, b)
    for k in range(nh):
        M = np.eye(dhd)
        v = np.zeros(dhd)
        for t in range(T):   # (J_t, b_t) o (M, v) = (J_t M, J_t v + b_t)
            M = J[0, t, k] @ M
            v = J[0, t, k] @ v + b[0, t, k * dhd:(k + 1) * dhd]
        assert np.allclose(out[0, T - 1, k * dhd:(k + 1) * dhd], v, rtol=0, atol=1e-12)
        assert np.allclose(out[0, T - 1, k * dhd:(k + 1) * dhd], M @ np.zeros(dhd) + v, rtol=0, atol=1e-12)


def test_first_k_steps_exact_and_k_equals_t():
    xp, A, h0 = inputs(2, 9, 8, 4, seed=11, scale=1.0)
    seq, _ = headmix.sequential(xp, A, h0=h0)
    res = headmix.newton(xp, A, 9, h0=h0, keep_iterates=True)
    for k, Hk in enumerate(res["iterates"], start=1):
        assert np.abs(Hk[:, :k] - seq[:, :k]).max() <= 1e-13, k
    assert np.abs(res["H"] - seq).max() <= 1e-12
    assert res["residuals"][-1] <= 1e-12


def test_quadratic_convergence():
    xp, A, h0 = inputs(1, 64, 16, 16, seed=5, scale=0.5)
    seq, _ = headmix.sequential(xp, A, h0=h0)
    res = headmix.newton(xp, A, 5, keep_iterates=True, h0=h0)
    errs = [np.abs(Hk - seq).max() for Hk in res["iterates"]]
    assert errs[-1] <= 1e-12
    for e0, e1 in zip(errs, errs[1:]):
        if e1 > 1e-12 and e0 < 0.1:
            assert np.log(e1) / np.log(e0) > 1.5, errs


def test_heads_do_not_interact():
    """Changing the inputs of one head leaves every other head's trajectory
    unchanged, in the unroll and in every Newton iterate."""
    xp, A, h0 = inputs(1, 20, 16, 4, seed=9)
    xp2 = xp.copy()
    xp2[:, :, :, 4:8] += 1.0                       # head 1 only
    for run in (lambda x: headmix.sequential(x, A, h0=h0)[0], lambda x: headmix.newton(x, A, 3, h0=h0)["H"]):
        u, v = run(xp), run(xp2)
        assert np.array_equal(np.delete(u, np.s_[4:8], axis=-1), np.delete(v, np.s_[4:8], axis=-1))
        assert np.abs(u[..., 4:8] - v[..., 4:8]).max() > 1e-3


def test_fp32_storage_rounds_every_iterate():
    xp, A, h0 = inputs(1, 30, 16, 16, seed=2)
    res = headmix.newton(xp, A, 3, dtype="f32", keep_iterates=True)
    for Hk in res["iterates"]:
        assert np.array_equal(Hk, Hk.astype(np.float32).astype(np.float64))
