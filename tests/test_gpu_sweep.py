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
(bf16) plus an absolute floor.  The backward (both schedules) and the
head-mix GRU get sweeps of their own, drawn the same way.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (TORCH_DT, gpu_backward, gpu_forward_states, gpu_run, gpu_run_fused, gpu_sequential, hm_inputs,
                         hm_newton, hm_sequential, oracle_backward, oracle_newton, oracle_sequential, random_grads,
                         rel_err, say, state_err, to_f64, tols)
from gpu_helpers import BF16_ABS
from oracle import headmix as ohm
from oracle.rounding import bf16_round
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
        assert state_err(w, to_f64(out["H"]), ref["H"][..., -1, :], 1e-5) <= 1
        assert state_err(w, to_f64(out["last"]), ref["last"], 1e-5) <= 1
        assert np.all(np.abs(out["res"] - rs) <= res_lim(w, rs))

    Hs, last_s = gpu_sequential(w, inp, two["xproj"], h0=h0, cu=cu)
    seq, seq_last = oracle_sequential(w, xp, inp["a"], h0=h0, cu=cu)
    err = np.abs(to_f64(Hs) - seq[..., -1, :]).max()
    say(f"  unroll: max|H - oracle unroll| {err:.3e}")
    assert state_err(w, to_f64(Hs), seq[..., -1, :], 1e-5) <= 1
    assert state_err(w, to_f64(last_s), seq_last, 1e-5) <= 1


@pytest.mark.parametrize("algo", ["sp", "tp"])
@pytest.mark.parametrize("i", range(N_CASES // 2), ids=lambda i: case_id(N_CASES + i))
def test_sweep_backward_against_the_oracle_adjoint(i, algo, monkeypatch):
    """The backward on the forward's own trajectory, both schedules (the
    library reads PRN_ALGO at every call); tolerances of the backward parity
    tests, relative to 1 + max|reference|."""
    monkeypatch.setenv("PRN_ALGO", algo)
    w, cu, rows, with_h0 = draw_case(N_CASES + i)
    say(f"[case] sweep backward {algo} {case_id(N_CASES + i)} cu={None if cu is None else cu.tolist()}")
    inp = dict(make_inputs(w.scaled(n_seqs=0), seed=4000 + i), cu_seqlens=cu)
    h0 = random_state(w, rows, seed=5000 + i) if with_h0 else None
    if w.T == 0:
        xproj = torch.empty((w.B, 0, w.G, w.d_h), dtype=TORCH_DT[w.dtype], device="cuda")
        states = torch.empty((w.B, 0, w.S, w.d_h), dtype=TORCH_DT[w.dtype], device="cuda")
    else:
        xproj, _, states, _ = gpu_forward_states(w, inp, w.K, h0=h0)
    dH, dsl = random_grads(w, rows, seed=6000 + i)
    dx, da, dh0 = gpu_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
    rdx, rda, rdh0 = oracle_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
    e_dx, e_da, e_dh0 = rel_err(to_f64(dx), rdx), rel_err(to_f64(da), rda), rel_err(to_f64(dh0), rdh0)
    say(f"  dxproj {e_dx:.2e}  da {e_da:.2e}  dh0 {e_dh0:.2e}")
    t_x, t_a = tols(w)
    assert e_dx <= t_x and e_dh0 <= t_x and e_da <= t_a


def draw_head_case(i: int):
    rng = np.random.default_rng(7000 + i)
    Bn = int(rng.integers(1, 4))
    d_h = 16 * int(rng.integers(1, 9))
    T = int(rng.integers(1, 1501)) if rng.integers(12) else 0
    K = int(rng.integers(1, 6))
    return Bn, T, d_h, K, bool(rng.integers(2))


@pytest.mark.parametrize("i", range(8), ids=lambda i: "{}-B{}-T{}-dh{}-K{}-h0{}".format(i, *draw_head_case(100 + i)))
def test_sweep_head_mix_bf16_against_the_oracle(i):
    """Head-mix GRU with bf16 storage (inputs rounded once to bf16): Newton at
    equal K against the oracle's Newton with bf16 stores (BF16_ABS on h;
    residuals 2e-2 + 2e-2 r), the sequential kernel against the float64
    unroll (BF16_ABS)."""
    Bn, T, d_h, K, with_h0 = draw_head_case(100 + i)
    say(f"[case] sweep head-mix bf16 B={Bn} T={T} d_h={d_h} K={K} h0={with_h0}")
    xp, A, h0 = hm_inputs(Bn, T, d_h, seed=9000 + i, with_h0=with_h0)
    xp = bf16_round(xp)
    h0 = None if h0 is None else bf16_round(h0)
    H, res, last = hm_newton(xp, A, K, h0, want_last=True, dtype="bf16")
    if T == 0:
        assert np.array_equal(res, np.zeros(K + 1))
        assert np.array_equal(last, np.zeros((Bn, d_h)) if h0 is None else h0)
        return
    ref = ohm.newton(xp, A, K, h0=h0, dtype="bf16")
    r = np.asarray(ref["residuals"])
    e = np.abs(H - ref["H"]).max()
    say(f"  newton max err {e:.2e}")
    assert e <= BF16_ABS
    assert np.array_equal(last, H[:, -1])
    assert np.all(np.abs(res - r) <= 2e-2 + 2e-2 * r)
    Hs, _ = hm_sequential(xp, A, h0, dtype="bf16")
    seq, _ = ohm.sequential(xp, A, h0=h0)
    assert np.abs(Hs - seq).max() <= BF16_ABS


@pytest.mark.parametrize("i", range(16), ids=lambda i: "{}-B{}-T{}-dh{}-K{}-h0{}".format(i, *draw_head_case(i)))
def test_sweep_head_mix_against_the_oracle(i):
    """Head-mix GRU (dense 16 x 16 blocks per head): Newton at equal K and
    the sequential kernel against the oracle, tolerances of the head-mix
    parity tests (1e-5; residuals 2e-5 + 1e-3 r)."""
    Bn, T, d_h, K, with_h0 = draw_head_case(i)
    say(f"[case] sweep head-mix B={Bn} T={T} d_h={d_h} K={K} h0={with_h0}")
    xp, A, h0 = hm_inputs(Bn, T, d_h, seed=8000 + i, with_h0=with_h0)
    H, res, last = hm_newton(xp, A, K, h0, want_last=True)
    if T == 0:
        assert np.array_equal(res, np.zeros(K + 1))
        assert np.array_equal(last, np.zeros((Bn, d_h)) if h0 is None else h0)
        return
    ref = ohm.newton(xp, A, K, h0=h0, dtype="f32")
    r = np.asarray(ref["residuals"])
    e = np.abs(H - ref["H"]).max()
    say(f"  newton H err {e:.2e}; residuals gpu {np.round(res, 6)} oracle {np.round(r, 6)}")
    assert e <= 1e-5 and np.array_equal(last, H[:, T - 1])
    assert np.all(np.abs(res - r) <= 2e-5 + 1e-3 * r)
    Hs, last_s = hm_sequential(xp, A, h0)
    seq, seq_last = ohm.sequential(xp, A, h0=h0)
    assert np.abs(Hs - seq).max() <= 1e-5 and np.abs(last_s - seq_last).max() <= 1e-5
