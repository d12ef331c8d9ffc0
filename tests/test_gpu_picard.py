"""GPU parity of the Picard warm-start (picard_iters = P sweeps) against the
oracle at equal K, on the GPU's own projected inputs; tolerances as in
test_gpu_parity (1e-5 fp32 max-abs on h, bf16 within the bf16 band;
residuals 2e-5 + 1e-3 r fp32, 2e-2 + 2e-2 r bf16).  P runs from one sweep to
more than a sub-chunk's steps (the guess's window then reaches into earlier
sub-chunks and chunks) and past the segment lengths of the packs."""
import numpy as np
import pytest
import torch

from gpu_helpers import TORCH_DT, gpu_run, oracle_h0, say, small_inputs, state_err, to_dev, to_f64, tol
from nonlinear_rnn_amd import binding as B
from oracle import newton as onewton
from workloads import Workload, WORKLOADS, random_state

pytestmark = pytest.mark.gpu

CASES = [
    Workload("gru_small", "gru", 3, 1000, 24, 80, "f32", 3),
    Workload("lstm_small", "lstm", 2, 777, 16, 72, "f32", 3),
    Workload("lstm_bf16_small", "lstm", 2, 300, 16, 130, "bf16", 3),
    Workload("gru_ragged_small", "gru", 1, 1500, 16, 40, "f32", 3, n_seqs=7),
    Workload("lstm_ragged_small", "lstm", 1, 900, 16, 64, "f32", 3, n_seqs=5, seg_lo=1, seg_hi=400),
]


def picard_forward(w, inp, xproj, K, h0=None, P=1):
    dt = TORCH_DT[w.dtype]
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"]
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    n_seqs = 0 if cu is None else len(cu) - 1
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    res = torch.full((K + 1,), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, K, n_seqs=n_seqs, picard_iters=P), 1),
                     dtype=torch.uint8, device="cuda")
    B.prn_newton_forward(xproj, a, K, H, cell=w.cell, h0=None if h0 is None else to_dev(h0, w.dtype),
                         cu_seqlens=cu_d, residual_out=res, workspace=ws, picard_iters=P)
    torch.cuda.synchronize()
    return H, res.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
@pytest.mark.parametrize("K", [1, 3])
@pytest.mark.parametrize("P", [1, 2, 5, 23])
def test_picard_matches_oracle(w, K, P):
    say(f"[case] picard P={P} K={K} {w}")
    inp = small_inputs(w)
    rows = w.B if inp["cu_seqlens"] is None else w.n_seqs
    h0 = random_state(w, seed=2, rows=rows)
    xproj = gpu_run(w, inp, 1)["xproj"]
    H, res = picard_forward(w, inp, xproj, K, h0=h0, P=P)
    ref = onewton.newton(w.cell, to_f64(xproj), inp["a"].astype(np.float64), K, h0=oracle_h0(w, h0),
                         cu_seqlens=inp["cu_seqlens"], dtype=w.dtype, picard=P)
    err = np.abs(to_f64(H) - ref["H"][..., -1, :]).max()
    rr = np.array(ref["residuals"])
    say(f"  {w.name}: max|H - oracle| {err:.2e}; residuals gpu {res} oracle {rr}")
    assert state_err(w, to_f64(H), ref["H"][..., -1, :], 1e-5) <= 1
    assert np.all(np.abs(res - rr) <= tol(w, 2e-5) + (1e-3 if w.dtype == "f32" else 2e-2) * rr)


def test_picard_lowers_the_lstm_agreement_error_at_K3():
    """The campaign's point: one Picard sweep before Newton brings the LSTM
    under tau at K = 3 where plain Newton needs K = 4 (measured K* 4)."""
    w = Workload("lstm_k", "lstm", 2, 4096, 64, 128, "f32", 3)
    inp = small_inputs(w)
    xproj = gpu_run(w, inp, 1)["xproj"]
    a = torch.from_numpy(inp["a"]).cuda()
    Hs = torch.empty((w.B, w.T, w.d_h), device="cuda")
    B.prn_sequential_forward(xproj, a, Hs, cell="lstm")
    H0 = gpu_run(w, inp, 3, xproj=xproj)["H"]
    H1, _ = picard_forward(w, inp, xproj, 3)
    e0, e1 = float((H0 - Hs).abs().max()), float((H1 - Hs).abs().max())
    say(f"  LSTM K=3 agreement: plain {e0:.2e}, Picard {e1:.2e}")
    assert e1 < e0


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_picard_with_at_least_T_sweeps_is_the_unroll(cell):
    """P >= T sweeps give the unroll itself (every step's window reaches its
    head), so K = 1 Newton iteration from that guess stays on it, r_0 is zero
    up to rounding, and any P above T returns the bits of P = T."""
    w = Workload("picard_full", cell, 2, 70, 16, 96, "f32", 1)
    inp = small_inputs(w)
    xproj = gpu_run(w, inp, 1)["xproj"]
    a = torch.from_numpy(inp["a"]).cuda()
    Hs = torch.empty((w.B, w.T, w.d_h), device="cuda")
    B.prn_sequential_forward(xproj, a, Hs, cell=cell)
    HT, rT = picard_forward(w, inp, xproj, 1, P=w.T)
    Hb, rb = picard_forward(w, inp, xproj, 1, P=w.T + 57)
    say(f"  {cell}: max|H(P=T) - unroll| {float((HT - Hs).abs().max()):.2e}; r = {rT}")
    assert torch.equal(HT, Hb) and np.array_equal(rT, rb)
    assert float((HT - Hs).abs().max()) <= 1e-5
    assert rT[0] <= 1e-5


def test_picard_rejections(monkeypatch):
    w = CASES[0]
    inp = small_inputs(w)
    xproj = gpu_run(w, inp, 1)["xproj"]
    a = torch.from_numpy(inp["a"]).cuda()
    H = torch.empty((w.B, w.T, w.d_h), device="cuda")
    ws = torch.empty(B.prn_workspace_bytes("gru", torch.float32, w.B, w.T, w.d_h, 3), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(B.PrnError, match="INVALID"):
        B.prn_newton_forward(xproj, a, 3, H, cell="gru", workspace=ws, picard_iters=-1)
    monkeypatch.setenv("PRN_ALGO", "tp")
    ws = torch.empty(B.prn_workspace_bytes("gru", torch.float32, w.B, w.T, w.d_h, 3), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(B.PrnError, match="UNSUPPORTED"):
        B.prn_newton_forward(xproj, a, 3, H, cell="gru", workspace=ws, picard_iters=1)
