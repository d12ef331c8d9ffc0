"""GPU parity of the backward pass (prn_newton_backward) against the oracle's
adjoint recurrence, on the same stored numbers: the GPU forward's trajectory
(states_out), the projected inputs, h0, dL/dH and dL/d(final state), all
upcast to float64 for the oracle.

Tolerances (max-abs, relative to 1 + max|reference| of the output):
  * fp32 storage: dxproj and dh0 1e-5, da 1e-4 (da sums B*T products in
    fp32: about sqrt(B*T) roundings of 2^-24 of terms up to the size of the
    result);
  * bf16 storage: dxproj and dh0 are stored in bf16 (one rounding, 2^-9
    relative) plus the fp32 arithmetic: 1e-2; da stays fp32: 1e-4.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (TORCH_DT, gpu_backward, gpu_forward_states, oracle_backward, random_grads, rel_err, say,
                         small_inputs, to_dev, to_f64, tols)
from oracle import backward as obackward
from workloads import Workload, WORKLOADS, random_state

pytestmark = pytest.mark.gpu

SMALL = [
    Workload("gru_small", "gru", 3, 1000, 24, 80, "f32", 3),
    Workload("lstm_small", "lstm", 2, 777, 16, 72, "f32", 2),
    Workload("gru_bf16_small", "gru", 2, 600, 32, 64, "bf16", 3),
    Workload("lstm_bf16_small", "lstm", 2, 300, 16, 130, "bf16", 3),
    Workload("gru_ragged_small", "gru", 1, 1500, 16, 40, "f32", 3, n_seqs=7),
    Workload("lstm_ragged_small", "lstm", 1, 900, 16, 64, "f32", 3, n_seqs=5, seg_lo=1, seg_hi=400),
    WORKLOADS["gru_tiny"],
]
IDS = [w.name for w in SMALL]


@pytest.fixture(params=["sp", "tp"])
def algo(request, monkeypatch):
    """Backward schedule: 'sp' single-pass look-back kernel (default), 'tp'
    three-phase kernels.  The library reads PRN_ALGO at every call."""
    monkeypatch.setenv("PRN_ALGO", request.param)
    return request.param


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_states_out_is_the_trajectory(w):
    """states_out holds every state: its h component is H_out, and at a
    sequence end it is the final state."""
    say(f"[case] states_out {w}")
    inp = small_inputs(w)
    rows = w.B if inp["cu_seqlens"] is None else w.n_seqs
    h0 = random_state(w, seed=3, rows=rows)
    xproj, H, states, last = gpu_forward_states(w, inp, w.K, h0=h0)
    assert torch.equal(states[..., w.S - 1, :], H)
    cu = inp["cu_seqlens"]
    if cu is None:
        assert torch.equal(states[:, -1], last)
    else:
        for j in range(len(cu) - 1):
            if cu[j + 1] > cu[j]:
                assert torch.equal(states[0, cu[j + 1] - 1], last[j])


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_backward_matches_oracle_adjoint(w, algo):
    say(f"[case] backward {algo} {w}")
    inp = small_inputs(w)
    cu = inp["cu_seqlens"]
    rows = w.B if cu is None else w.n_seqs
    h0 = random_state(w, seed=4, rows=rows)
    xproj, H, states, last = gpu_forward_states(w, inp, w.K, h0=h0)
    dH, dsl = random_grads(w, rows, seed=7)
    dx, da, dh0 = gpu_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
    rdx, rda, rdh0 = oracle_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
    e_dx, e_da, e_dh0 = rel_err(to_f64(dx), rdx), rel_err(to_f64(da), rda), rel_err(to_f64(dh0), rdh0)
    say(f"  {w.name} {algo}: dxproj {e_dx:.2e}  da {e_da:.2e}  dh0 {e_dh0:.2e}  (max|dxproj| {np.abs(rdx).max():.3g}, "
        f"max|da| {np.abs(rda).max():.3g})")
    t_x, t_a = tols(w)
    assert e_dx <= t_x and e_dh0 <= t_x and e_da <= t_a


@pytest.mark.parametrize("w", [SMALL[1], SMALL[4]], ids=[SMALL[1].name, SMALL[4].name])
def test_backward_optional_arguments(w):
    """No h0, no dstate_last, no dh0_out: the same as zeros / not written."""
    inp = small_inputs(w)
    cu = inp["cu_seqlens"]
    rows = w.B if cu is None else w.n_seqs
    xproj, H, states, last = gpu_forward_states(w, inp, w.K)
    dH, _ = random_grads(w, rows, seed=8)
    dx, da, _ = gpu_backward(w, inp, xproj, states, dH, want_dh0=False)
    dx2, da2, dh0 = gpu_backward(w, inp, xproj, states, dH, dsl=torch.zeros((rows, w.S, w.d_h),
                                 dtype=TORCH_DT[w.dtype], device="cuda"))
    # a zero dstate_last adds exact zeros: the same bits as none at all
    assert torch.equal(dx, dx2) and torch.equal(da, da2)
    rdx, rda, rdh0 = oracle_backward(w, inp, xproj, states, dH)
    assert rel_err(to_f64(dx), rdx) <= tols(w)[0] and rel_err(to_f64(dh0), rdh0) <= tols(w)[0]


@pytest.mark.parametrize("w", [SMALL[1], SMALL[2], SMALL[4]], ids=lambda w: w.name)
def test_backward_is_deterministic(w, algo):
    """Both schedules combine the chunk carries in an order fixed by the chunk
    index and reduce dL/da in a fixed order: repeated backward passes (and
    the forwards that give their trajectories) are bitwise identical."""
    inp = small_inputs(w)
    rows = w.B if inp["cu_seqlens"] is None else w.n_seqs
    xproj, H, states, last = gpu_forward_states(w, inp, w.K)
    _, H2, states2, last2 = gpu_forward_states(w, inp, w.K)
    assert torch.equal(H, H2) and torch.equal(states, states2) and torch.equal(last, last2)
    dH, dsl = random_grads(w, rows, seed=9)
    r1 = gpu_backward(w, inp, xproj, states, dH, dsl=dsl)
    for _ in range(2):
        r2 = gpu_backward(w, inp, xproj, states, dH, dsl=dsl)
        for u, v in zip(r1, r2):
            assert torch.equal(u, v)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_backward_edge_shapes(cell, algo):
    """T = 0 (da = 0, dh0 = dstate_last), T = 1, empty and one-step segments,
    and T at and just past whole chunks of the single-pass schedule (128 steps
    for the LSTM, 256 for the GRU with few chains), with segment heads on the
    chunk boundaries."""
    G, S = (3, 1) if cell == "gru" else (4, 2)
    d = 70
    for name, B_, T, cu in [("T0", 2, 0, None), ("T1", 3, 1, None), ("one-chunk", 1, 5, None),
                            ("ragged-empty", 1, 70, [0, 0, 33, 33, 69, 70]), ("ragged-T0", 1, 0, [0, 0, 0]),
                            ("T128", 1, 128, None), ("T129", 2, 129, None), ("T256", 1, 256, None),
                            ("T257", 1, 257, None), ("ragged-at-chunks", 1, 300, [0, 128, 256, 300])]:
        n_seqs = 0 if cu is None else len(cu) - 1
        w = Workload(f"{cell}_{name}", cell, B_, T, 8, d, "f32", 2, n_seqs=n_seqs)
        say(f"[case] backward edge {w}")
        rng = np.random.default_rng(12)
        inp = {"a": rng.uniform(-0.5, 0.5, (G, d)).astype(np.float32),
               "cu_seqlens": None if cu is None else np.asarray(cu, dtype=np.int32)}
        rows = B_ if cu is None else n_seqs
        h0 = random_state(w, seed=5, rows=rows)
        xproj = to_dev(rng.standard_normal((B_, T, G, d)), "f32")
        if T == 0:
            states = torch.empty((B_, 0, S, d), dtype=torch.float32, device="cuda")
        else:
            xproj, H, states, last = gpu_forward_states(w, inp, 2, h0=h0, xproj=xproj)
        dH, dsl = random_grads(w, rows, seed=6)
        dx, da, dh0 = gpu_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
        rdx, rda, rdh0 = oracle_backward(w, inp, xproj, states, dH, h0=h0, dsl=dsl)
        assert rel_err(to_f64(dx), rdx) <= 1e-5 and rel_err(to_f64(da), rda) <= 1e-4, name
        assert rel_err(to_f64(dh0), rdh0) <= 1e-5, name


SAMPLE = {"lstm_t131k": ([0, 1], [0, 130, 255]), "gru_ragged": ([0], [0, 77, 255]), "gru_bf16": ([15], [3, 511])}


@pytest.mark.parametrize("name", list(SAMPLE))
def test_backward_full_size_sampled(name):
    """At the full workload sizes: sampled channels (channels never interact,
    so a channel subset of the adjoint is an exact sub-problem)."""
    w = WORKLOADS[name]
    say(f"[case] backward full size {w}")
    inp = small_inputs(w)
    cu = inp["cu_seqlens"]
    rows = w.B if cu is None else w.n_seqs
    xproj, H, states, last = gpu_forward_states(w, inp, w.K)
    dH, dsl = random_grads(w, rows, seed=10)
    dx, da, dh0 = gpu_backward(w, inp, xproj, states, dH, dsl=dsl)
    rws, chs = SAMPLE[name]
    if cu is not None:
        rws = [0]
    sel = lambda t, ax: t[rws][..., chs] if ax else t[..., chs]
    sub_inp = dict(inp, a=inp["a"][:, chs])
    sw = Workload(w.name, w.cell, len(rws), w.T, w.d_in, len(chs), w.dtype, w.K, n_seqs=w.n_seqs)
    sub_dsl = dsl[:, :, chs] if cu is not None else dsl[rws][:, :, chs]
    rdx, rda, rdh0 = obackward.adjoint(w.cell, to_f64(sel(xproj, 1)), sub_inp["a"].astype(np.float64),
                                       to_f64(sel(states, 1)), to_f64(sel(dH, 1)), cu_seqlens=cu,
                                       dstate_last=to_f64(sub_dsl))
    got_dh0 = dh0[:, :, chs] if cu is not None else dh0[rws][:, :, chs]
    e_dx, e_dh0 = rel_err(to_f64(sel(dx, 1)), rdx), rel_err(to_f64(got_dh0), rdh0)
    say(f"  {name}: dxproj {e_dx:.2e} dh0 {e_dh0:.2e}")
    t_x, t_a = tols(sw)
    assert e_dx <= t_x and e_dh0 <= t_x
    if cu is not None or len(rws) == w.B:   # da sums over all rows: comparable only when all rows are sampled
        e_da = rel_err(to_f64(da[:, chs]), rda)
        say(f"  {name}: da {e_da:.2e}")
        assert e_da <= t_a
