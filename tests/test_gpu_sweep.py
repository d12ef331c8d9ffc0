"""Seeded shape sweep: the forward paths against the oracle on shapes drawn
at random rather than picked by hand.

Each case draws the cell, the storage dtype, a rectangular batch or a ragged
pack (segment boundaries drawn freely, empty segments included), T, d_h,
d_in, K and whether h0 is given, all from one seeded generator, so that a
failure names a reproducible case.  Every case runs
  - the projection + Newton forward (two calls) against the oracle at equal K,
  - the fused forward (projection inside the Newton kernel) against the same,
    and its stored projection bitwise against the stand-alone one,
  - the sequential unroll against the oracle's unroll.
Tolerances are the parity tests' own: 1e-5 (fp32) and 2e-2 (bf16) on H and
the final state at equal K; residuals to 1e-3 relative (fp32) or 2e-2
(bf16) plus an absolute floor.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (gpu_run, gpu_run_fused, gpu_sequential, oracle_newton, oracle_sequential, say, to_f64,
                         tol)
from workloads import Workload, make_inputs, random_state

pytestmark = pytest.mark.gpu

N_CASES = 64
TOKENS_X_CH = 250_000   # cap on rows * T * d_h, keeps the oracle at about a second per case
T_MAX = 3000


def draw_case(i: int):
    rng = np.random.default_rng(1000 + i)
    cell = ("gru", "lstm")[int(rng.integers(2))]
    dtype = ("f32", "bf16")[int(rng.integers(2))]
    kvec = 4 if dtype == "f32" else 8
    d_in = kvec * int(rng.integers(1, 41))
    d_h = int(rng.choice([int(rng.integers(1, 64)), 64, int(rng.integers(65, 200))]))
    K = int(rng.integers(1, 7))
    ragged = bool(rng.integers(2))
    if ragged:
        n_seqs = int(rng.integers(1, 10))
        B = 1
        T = int(rng.integers(0, min(T_MAX, TOKENS_X_CH // d_h) + 1))
        cuts = np.sort(rng.integers(0, T + 1, size=n_seqs - 1))
        if n_seqs > 1 and rng.integers(3) == 0:   # an empty segment: repeat a boundary (0, T or a cut)
            j = int(rng.integers(n_seqs - 1))
            cuts[j] = (0, T, cuts[-1 - j])[int(rng.integers(3))]
            cuts = np.sort(cuts)
        cu = np.concatenate([[0], cuts, [T]]).astype(np.int32)
        rows = n_seqs
    else:
        B = int(rng.integers(1, 6))
        T = int(rng.integers(0, min(T_MAX, TOKENS_X_CH // (B * d_h)) + 1))
        cu = None
        rows = B
    if rng.integers(12) == 0:
        T = 0
        if cu is not None:
            cu[:] = 0
    with_h0 = bool(rng.integers(2))
    w = Workload(f"sweep{i}", cell, B, T, d_in, d_h, dtype, K, n_seqs=0 if cu is None else len(cu) - 1)
    return w, cu, rows, with_h0


def case_id(i):
    w, cu, rows, with_h0 = draw_case(i)
    pack = f"pack{len(cu) - 1}" if cu is not None else f"B{w.B}"
    return f"{i}-{w.cell}-{w.dtype}-{pack}-T{w.T}-dh{w.d_h}-din{w.d_in}-K{w.K}" + ("-h0" if with_h0 else "")


def res_lim(w, rs):
    return (2e-5 + 1e-3 * rs) if w.dtype == "f32" else (2e-2 + 2e-2 * rs)


@pytest.mark.parametrize("i", range(N_CASES), ids=case_id)
def test_sweep_forward_paths_against_the_oracle(i):
    w, cu, rows, with_h0 = draw_case(i)
    say(f"[case] sweep {case_id(i)} cu={None if cu is None else cu.tolist()}")
    base = w.scaled(n_seqs=0)
    inp = make_inputs(base, seed=2000 + i)
    h0 = random_state(w, rows, seed=3000 + i) if with_h0 else None

    two = gpu_run(w, inp, w.K, h0=h0, cu=cu)
    fused = gpu_run_fused(w, inp, w.K, h0=h0, cu=cu)
    assert torch.equal(fused["xproj"], two["xproj"])
    if w.T == 0:
        # every row (segment) is empty: the final state is h0, else zero
        want = np.zeros((rows, w.S, w.d_h)) if h0 is None else to_f64(torch.from_numpy(h0).to(two["last"].dtype))
        for out in (two, fused):
            assert np.array_equal(out["res"], np.zeros(w.K + 1))
            assert np.array_equal(to_f64(out["last"]), want)
        return

    xp = to_f64(two["xproj"])
    ref = oracle_newton(w, xp, inp["a"], w.K, h0=h0, cu=cu)
    rs = np.array(ref["residuals"])
    for name, out in (("two-call", two), ("fused", fused)):
        err = np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max()
        err_last = np.abs(to_f64(out["last"]) - ref["last"]).max()
        say(f"  {name}: max|H - oracle| {err:.3e}, last {err_last:.3e}; residuals {out['res']} oracle {rs}")
        assert err <= tol(w, 1e-5) and err_last <= tol(w, 1e-5)
        assert np.all(np.abs(out["res"] - rs) <= res_lim(w, rs))

    Hs, last_s = gpu_sequential(w, inp, two["xproj"], h0=h0, cu=cu)
    seq, seq_last = oracle_sequential(w, xp, inp["a"], h0=h0, cu=cu)
    err = np.abs(to_f64(Hs) - seq[..., -1, :]).max()
    say(f"  unroll: max|H - oracle unroll| {err:.3e}")
    assert err <= tol(w, 1e-5)
    assert np.abs(to_f64(last_s) - seq_last).max() <= tol(w, 1e-5)
