"""A look-back wait that gives up is reported, never silent.

The single-pass kernels (forward and backward) wait for records of earlier
chunks with a bounded number of polls.  PRN_SPIN_LIMIT=0, read by the host
at every call, makes every such wait give up at once (each chunk but the
first of every chain), so the error path runs with no fault and no hang:
the kernels poison the carries with NaN, set bit PRN_FAULT_LOOKBACK of the
caller's error word, and exit normally.  The Numerics contract page opens on
the risk this guards against: a silent wrong answer.
"""
import numpy as np
import pytest
import torch

import nonlinear_rnn_amd as prn
from gpu_helpers import TORCH_DT, say, small_inputs, to_dev
from nonlinear_rnn_amd import binding as B
from workloads import Workload

pytestmark = pytest.mark.gpu

W_GRU = Workload("gru_small", "gru", 3, 1000, 24, 80, "f32", 3)
W_LSTM = Workload("lstm_small", "lstm", 2, 777, 16, 72, "f32", 2)


def _run(w, err, states=None):
    inp = small_inputs(w)
    dt = TORCH_DT[w.dtype]
    xp = torch.empty((w.B, w.T, w.G, w.d_h), dtype=dt, device="cuda")
    B.prn_input_proj(to_dev(inp["x"], w.dtype), to_dev(inp["W"], w.dtype), torch.from_numpy(inp["bias"]).cuda(),
                     xp, cell=w.cell)
    a = torch.from_numpy(inp["a"]).cuda()
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    res = torch.zeros(w.K + 1, device="cuda")
    ws = torch.empty(B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, w.K), dtype=torch.uint8, device="cuda")
    B.prn_newton_forward(xp, a, w.K, H, cell=w.cell, residual_out=res, states_out=states, workspace=ws,
                         error_out=err)
    torch.cuda.synchronize()
    return xp, a, H, res


@pytest.mark.parametrize("w", [W_GRU, W_LSTM], ids=lambda w: w.name)
def test_forward_reports_a_given_up_wait(w, monkeypatch):
    say(f"[case] forward look-back give-up {w}")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, _, H, res = _run(w, err)
    assert int(err.item()) == 0 and torch.isfinite(H).all()
    monkeypatch.setenv("PRN_SPIN_LIMIT", "0")
    _, _, H, res = _run(w, err)
    assert int(err.item()) & B.PRN_FAULT_LOOKBACK
    assert float(res[-1]) == float("inf")
    assert torch.isnan(H).any()
    # the API raises instead of returning the poisoned trajectory
    inp = small_inputs(w)
    xp = torch.randn((w.B, w.T, w.G, w.d_h), device="cuda")
    with pytest.raises(prn.LookbackTimeoutError):
        prn.newton_forward(xp, torch.from_numpy(inp["a"]).cuda(), w.K, cell=w.cell)
    monkeypatch.delenv("PRN_SPIN_LIMIT")
    err.zero_()
    _, _, H, res = _run(w, err)
    assert int(err.item()) == 0 and torch.isfinite(H).all() and np.isfinite(float(res[-1]))


@pytest.mark.parametrize("w", [W_GRU, W_LSTM], ids=lambda w: w.name)
def test_backward_reports_a_given_up_wait(w, monkeypatch):
    say(f"[case] backward look-back give-up {w}")
    dt = TORCH_DT[w.dtype]
    states = torch.empty((w.B, w.T, w.S, w.d_h), dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    xp, a, H, _ = _run(w, err, states)
    assert int(err.item()) == 0
    dH = torch.randn((w.B, w.T, w.d_h), device="cuda").to(dt)
    dxp = torch.empty_like(xp)
    da = torch.empty((w.G, w.d_h), device="cuda")
    ws = torch.empty(B.prn_backward_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h), dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("PRN_SPIN_LIMIT", "0")
    B.prn_newton_backward(xp, a, states, dH, dxp, da, cell=w.cell, workspace=ws, error_out=err)
    torch.cuda.synchronize()
    assert int(err.item()) & B.PRN_FAULT_LOOKBACK
    assert torch.isnan(dxp).any()
    # through autograd: the backward raises rather than hand NaN gradients on
    monkeypatch.delenv("PRN_SPIN_LIMIT")
    xq = xp.detach().clone().requires_grad_()
    Hq = prn.newton_apply(xq, a, w.K, cell=w.cell)
    monkeypatch.setenv("PRN_SPIN_LIMIT", "0")
    with pytest.raises(prn.LookbackTimeoutError):
        Hq.sum().backward()
    monkeypatch.delenv("PRN_SPIN_LIMIT")
    err.zero_()
    B.prn_newton_backward(xp, a, states, dH, dxp, da, cell=w.cell, workspace=ws, error_out=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and torch.isfinite(dxp).all()
