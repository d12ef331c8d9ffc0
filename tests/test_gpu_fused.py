"""GPU parity of the fused forward (prn_newton_forward_fused: the input
projection computed inside the Newton kernel) against the oracle and
against the two-call path (prn_input_proj + prn_newton_forward).

The fused tile uses the stand-alone projection's instruction and summation
order, so the projected inputs it stores are bitwise the stand-alone ones;
its Newton part is the single-pass kernel with the same, timing-independent
carry arithmetic.  So wherever both take the same chunk length (every LSTM,
and the GRU below 64 (row, 64-channel) chains) the fused forward equals the
two-call forward bit for bit; the many-chain GRU takes longer chunks fused
than unfused, and the two then agree to rounding (1e-6 in fp32, one bf16
step in bf16).  Oracle tolerances as in test_gpu_parity: 1e-5 (fp32) / 2e-2
(bf16) at equal K, tau = 1e-4 against the unroll.
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import (gpu_run, gpu_run_fused, oracle_newton, oracle_sequential, say, small_inputs, state_err, to_dev,
                         to_f64, tol, TORCH_DT)
from nonlinear_rnn_amd import binding as B
from oracle import proj as oproj
from oracle import rounding as oround
from workloads import Workload, WORKLOADS, make_inputs, random_state

pytestmark = pytest.mark.gpu

CASES = [
    Workload("gru_small", "gru", 3, 1000, 24, 80, "f32", 3),
    Workload("lstm_small", "lstm", 2, 777, 16, 72, "f32", 2),
    Workload("gru_bf16_small", "gru", 2, 600, 32, 64, "bf16", 3),
    Workload("lstm_bf16_small", "lstm", 2, 300, 40, 130, "bf16", 3),
    Workload("gru_ragged_small", "gru", 1, 1500, 16, 40, "f32", 3, n_seqs=7),
    Workload("lstm_ragged_small", "lstm", 1, 900, 20, 64, "f32", 3, n_seqs=5, seg_lo=1, seg_hi=400),
    Workload("gru_many_chains", "gru", 64, 100, 12, 70, "f32", 3),          # >= 64 chains
    Workload("gru_many_chains_bf16", "gru", 40, 90, 48, 100, "bf16", 3),
    WORKLOADS["gru_tiny"],
]
IDS = [w.name for w in CASES]


def same_chunking(w) -> bool:
    """Do the fused and two-call forwards take the same chunks?  Only the
    LSTM: the fused GRU takes 64-step chunks of four waves, the unfused one
    96-step chunks of eight waves below 64 (row, 64-channel) chains and
    48-step chunks from 64 on."""
    return w.cell == "lstm"


def lim_rr(w):
    return 1e-6 if w.dtype == "f32" else 1e-2


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_fused_projection_is_the_standalone_projection(w):
    say(f"[case] fused projection {w}")
    inp = small_inputs(w)
    ref = gpu_run(w, inp, w.K)
    got = gpu_run_fused(w, inp, w.K)
    assert torch.equal(got["xproj"], ref["xproj"])
    o = oproj.input_proj(oround.load(inp["x"], w.dtype), oround.load(inp["W"], w.dtype),
                         inp["bias"].astype(np.float64), w.G)
    if w.dtype == "f32":
        assert np.abs(to_f64(got["xproj"]) - o).max() <= 1e-5
    else:
        assert np.all(np.abs(to_f64(got["xproj"]) - o) <= 2 ** -8 * np.abs(o) + 1e-4)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_fused_matches_oracle_at_equal_K(w):
    say(f"[case] fused newton equal-K {w}")
    inp = small_inputs(w)
    out = gpu_run_fused(w, inp, w.K)
    ref = oracle_newton(w, to_f64(out["xproj"]), inp["a"], w.K, cu=inp["cu_seqlens"])
    err = np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max()
    err_last = np.abs(to_f64(out["last"]) - ref["last"]).max()
    rs = np.array(ref["residuals"])
    say(f"  max|H - oracle| {err:.3e}, last {err_last:.3e}; residuals gpu {out['res']} oracle {rs}")
    assert state_err(w, out["H"].float().cpu(), ref["H"][..., -1, :], 1e-5) <= 1
    assert state_err(w, out["last"].float().cpu(), ref["last"], 1e-5) <= 1
    lim = (2e-5 + 1e-3 * rs) if w.dtype == "f32" else (2e-2 + 2e-2 * rs)
    assert np.all(np.abs(out["res"] - rs) <= lim)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_fused_matches_two_call_path(w):
    say(f"[case] fused vs projection + newton {w}")
    inp = small_inputs(w)
    ref = gpu_run(w, inp, w.K)
    for with_xproj in (True, False):
        got = gpu_run_fused(w, inp, w.K, with_xproj=with_xproj)
        if same_chunking(w):
            assert torch.equal(got["H"], ref["H"]) and torch.equal(got["last"], ref["last"])
            assert np.array_equal(got["res"], ref["res"])
        else:
            assert (got["H"].float() - ref["H"].float()).abs().max().item() <= lim_rr(w)
            assert (got["last"].float() - ref["last"].float()).abs().max().item() <= lim_rr(w)
            assert np.all(np.abs(got["res"] - ref["res"]) <= lim_rr(w) + 1e-5 * ref["res"])


@pytest.mark.parametrize("w", [CASES[0], CASES[4], CASES[6]], ids=lambda w: w.name)
def test_fused_gru_within_tau_of_sequential(w):
    say(f"[case] fused vs unroll {w}")
    inp = small_inputs(w)
    out = gpu_run_fused(w, inp, 3)
    seq, _ = oracle_sequential(w, to_f64(out["xproj"]), inp["a"], cu=inp["cu_seqlens"])
    err = np.abs(to_f64(out["H"]) - seq[..., -1, :]).max()
    say(f"  max|H - sequential| {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_fused_nonzero_h0_and_packed_segments(cell):
    w = Workload(f"{cell}_pack", cell, 1, 700, 16, 40, "f32", 3)
    cu = np.array([0, 0, 64, 64, 65, 300, 700, 700], dtype=np.int32)
    wp = w.scaled(n_seqs=len(cu) - 1)
    say(f"[case] fused pack with h0 {wp}")
    inp = small_inputs(w)
    h0 = random_state(w, len(cu) - 1, seed=5)
    out = gpu_run_fused(wp, inp, w.K, h0=h0, cu=cu)
    ref = oracle_newton(wp, to_f64(out["xproj"]), inp["a"], w.K, h0=h0, cu=cu)
    assert np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max() <= 1e-5
    assert np.abs(to_f64(out["last"]) - ref["last"]).max() <= 1e-5
    for j in range(len(cu) - 1):   # empty segments end in their h0
        if cu[j] == cu[j + 1]:
            assert torch.equal(out["last"][j].cpu(), torch.from_numpy(h0[j]))


@pytest.mark.parametrize("T,d_h,d_in,K", [(1, 16, 4, 3), (31, 64, 12, 2), (32, 64, 8, 3), (33, 65, 20, 3),
                                          (70, 1, 4, 1), (45, 63, 36, 50), (0, 16, 8, 3)])
@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_fused_edge_shapes(cell, T, d_h, d_in, K):
    w = Workload(f"{cell}_edge", cell, 2, T, d_in, d_h, "f32", K)
    say(f"[case] fused edge {w}")
    inp = small_inputs(w)
    h0 = random_state(w, w.B, seed=9)
    out = gpu_run_fused(w, inp, K, h0=h0)
    if T == 0:
        assert np.array_equal(out["res"], np.zeros(K + 1))
        assert np.abs(to_f64(out["last"]) - h0).max() == 0
        return
    ref = oracle_newton(w, to_f64(out["xproj"]), inp["a"], K, h0=h0)
    assert np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max() <= 1e-5
    assert np.abs(to_f64(out["last"]) - ref["last"]).max() <= 1e-5
    two = gpu_run(w, inp, K, h0=h0)
    assert torch.equal(out["xproj"], two["xproj"])


def test_fused_rejections():
    w = Workload("lstm_rej", "lstm", 1, 64, 8, 16, "f32", 2)
    inp = small_inputs(w)
    dev = "cuda"
    x = torch.from_numpy(inp["x"]).to(dev)
    W = torch.from_numpy(inp["W"]).to(dev)
    a = torch.from_numpy(inp["a"]).to(dev)
    H = torch.empty((1, 64, 16), device=dev)
    ws = torch.empty(B.prn_workspace_bytes("lstm", torch.float32, 1, 64, 16, 2), dtype=torch.uint8, device=dev)
    # Picard warm-start is not part of the fused path
    p = B.make_params("lstm", torch.float32, 1, 64, 16, d_in=8, a=a, workspace=ws, picard_iters=1)
    st = B.lib().prn_newton_forward_fused(x.data_ptr(), W.data_ptr(), None, ctypes.byref(p), None, 2, None,
                                          H.data_ptr(), None, None)
    assert st == B.PRN_ERR_UNSUPPORTED and "Picard" in B.prn_last_error()
    # d_in not a multiple of 4 (fp32)
    x6 = torch.zeros((1, 64, 6), device=dev)
    W6 = torch.zeros((64, 6), device=dev)
    with pytest.raises(B.PrnError):
        B.prn_newton_forward_fused(x6, W6, None, a, 2, H, cell="lstm", workspace=ws)
    # workspace too small
    with pytest.raises(B.PrnError):
        B.prn_newton_forward_fused(x, W, None, a, 2, H, cell="lstm", workspace=ws[:16])
    # shape mismatch is caught by the binding
    with pytest.raises(ValueError):
        B.prn_newton_forward_fused(x, W[:32], None, a, 2, H, cell="lstm", workspace=ws)


SAMPLE = {  # rows, channels
    "gru_d256": ([0, 7], [0, 63, 64, 200, 255]),
    "gru_bf16": ([0, 15], [0, 255, 511]),
    "lstm_t131k": ([0, 1], [0, 130, 255]),
    "gru_ragged": ([0], [0, 77, 255]),
}


@pytest.mark.parametrize("name", list(SAMPLE))
def test_fused_full_size_sampled_parity(name):
    """Full size, the bench's launch configuration: sampled channels against
    the oracle (channels never interact), every output against the two-call
    path."""
    w = WORKLOADS[name]
    say(f"[case] fused full size {w}")
    inp = make_inputs(w, seed=0)
    out = gpu_run_fused(w, inp, w.K)
    two = gpu_run(w, inp, w.K)
    assert torch.equal(out["xproj"], two["xproj"])
    d = (out["H"].float() - two["H"].float()).abs().max().item()
    rows, chans = SAMPLE[name]
    xp = out["xproj"][rows][:, :, :, chans].float().cpu().numpy().astype(np.float64)
    ref = oracle_newton(w, xp, inp["a"][:, chans], w.K, cu=inp["cu_seqlens"])
    err = np.abs(to_f64(out["H"][rows][:, :, chans]) - ref["H"][..., -1, :]).max()
    say(f"  {name}: max|fused - two-call| {d:.3e}; sampled max|H - oracle| {err:.3e}; residuals {out['res']}")
    if same_chunking(w):   # the same chunks: the same bits
        assert d == 0
    else:
        assert state_err(w, out["H"].float().cpu(), two["H"].float().cpu(), 1e-5) <= 1
    assert state_err(w, out["H"][rows][:, :, chans].float().cpu(), ref["H"][..., -1, :], 1e-5) <= 1
    assert np.all(np.abs(out["res"] - two["res"]) <= tol(w, 1e-5) + 1e-4 * two["res"])


def test_api_forward_fused_matches_two_calls_and_gates():
    """The Python-level contract around the fused entry point: same results as
    the two-call forward, the final state and stored xproj on request, K from
    a per-T table, strided inputs copied, and the divergence gate."""
    from nonlinear_rnn_amd import api
    w = Workload("lstm_api", "lstm", 2, 500, 24, 70, "f32", 3)
    say(f"[case] api fused forward {w}")
    inp = small_inputs(w)
    x = torch.from_numpy(inp["x"]).cuda()
    W = torch.from_numpy(inp["W"]).cuda()
    bias = torch.from_numpy(inp["bias"]).cuda()
    a = torch.from_numpy(inp["a"]).cuda()
    H2, r2, st2 = api.forward(x, W, bias, a, 3, cell="lstm", return_state=True)
    H1, r1, st1, xp = api.forward(x, W, bias, a, 3, cell="lstm", fused=True, return_state=True, return_xproj=True)
    assert torch.equal(H1, H2) and torch.equal(st1, st2) and r1 == r2   # LSTM: same chunking
    assert torch.equal(xp, api.input_proj(x, W, bias, cell="lstm"))
    Ht, rt = api.forward(x, W, bias, a, None, cell="lstm", fused=True, k_table={64: 2, 1024: 4})
    assert len(rt) == 5   # T = 500 -> K = 4
    # a strided view of x (every other feature of a wider tensor) is copied first
    xw = torch.zeros((2, 500, 48), device="cuda")
    xw[:, :, ::2] = x
    Hs, _ = api.forward(xw[:, :, ::2], W, bias, a, 3, cell="lstm", fused=True)
    assert torch.equal(Hs, H1)
    # non-finite input: the residual gate raises
    xn = x.clone()
    xn[1, 100, 3] = float("nan")
    with pytest.raises(api.NewtonDivergenceError):
        api.forward(xn, W, bias, a, 3, cell="lstm", fused=True)


@pytest.mark.parametrize("cell,dtype", [("lstm", "f32"), ("gru", "f32"), ("lstm", "bf16")])
def test_fused_states_out_matches_two_call_trajectory(cell, dtype):
    """The fused instance that also writes every state (the trajectory the
    backward pass takes) against prn_newton_forward's states_out, ragged pack
    with h0 included."""
    w = Workload(f"{cell}_states", cell, 1, 900, 16, 72, dtype, 3)
    cu = np.array([0, 100, 100, 433, 900], dtype=np.int32)
    wp = w.scaled(n_seqs=len(cu) - 1)
    say(f"[case] fused states_out {wp}")
    inp = small_inputs(w)
    dt = TORCH_DT[dtype]
    x = to_dev(inp["x"], dtype)
    W = to_dev(inp["W"], dtype)
    bias = torch.from_numpy(inp["bias"]).cuda()
    a = torch.from_numpy(inp["a"]).cuda()
    h0 = to_dev(random_state(w, len(cu) - 1, seed=2), dtype)
    cu_d = torch.from_numpy(cu).cuda()
    ws = torch.empty(B.prn_workspace_bytes(cell, dt, 1, w.T, w.d_h, 3, n_seqs=len(cu) - 1), dtype=torch.uint8,
                     device="cuda")
    xp = torch.empty((1, w.T, w.G, w.d_h), dtype=dt, device="cuda")
    B.prn_input_proj(x, W, bias, xp, cell=cell)
    outs = []
    for fused in (False, True):
        H = torch.empty((1, w.T, w.d_h), dtype=dt, device="cuda")
        st = torch.empty((1, w.T, w.S, w.d_h), dtype=dt, device="cuda")
        if fused:
            B.prn_newton_forward_fused(x, W, bias, a, 3, H, cell=cell, h0=h0, cu_seqlens=cu_d, states_out=st,
                                       workspace=ws)
        else:
            B.prn_newton_forward(xp, a, 3, H, cell=cell, h0=h0, cu_seqlens=cu_d, states_out=st, workspace=ws)
        torch.cuda.synchronize()
        outs.append((H, st))
    if same_chunking(w):   # the same chunks: the same bits
        assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][0], outs[1][0])
    else:
        assert (outs[0][1].float() - outs[1][1].float()).abs().max().item() <= lim_rr(w)
        assert (outs[0][0].float() - outs[1][0].float()).abs().max().item() <= lim_rr(w)
    assert torch.equal(outs[1][1][..., w.S - 1, :], outs[1][0])   # h part of the states is H_out
