"""The allocation-free forward (prn_newton_forward_noalloc) against
prn_newton_forward with a caller workspace: the same kernels on the same
inputs, so the same bits.  Two calls in a row share the library's static
scratch, the second with a smaller input (its status words must be cleared
again, its records overwritten); then the ragged 65536-token GRU pack at full
size, the largest workload the scratch holds."""
import numpy as np
import pytest
import torch

from gpu_helpers import TORCH_DT, say, small_inputs, to_dev
from nonlinear_rnn_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs, random_state

pytestmark = pytest.mark.gpu


def _inputs(w, inp, h0=None):
    dt = TORCH_DT[w.dtype]
    xp = torch.empty((w.B, w.T, w.G, w.d_h), dtype=dt, device="cuda")
    B.prn_input_proj(to_dev(inp["x"], w.dtype), to_dev(inp["W"], w.dtype), torch.from_numpy(inp["bias"]).cuda(),
                     xp, cell=w.cell)
    a = torch.from_numpy(inp["a"]).cuda()
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).cuda()
    return xp, a, cu, (None if h0 is None else to_dev(h0, w.dtype))


def _both(w, inp, h0=None):
    """(with workspace, allocation-free) outputs: H, residuals, final states."""
    dt = TORCH_DT[w.dtype]
    xp, a, cu, h0d = _inputs(w, inp, h0)
    n_seqs = 0 if cu is None else cu.numel() - 1
    rows = w.B if cu is None else n_seqs
    outs = []
    for noalloc in (False, True):
        H = torch.full((w.B, w.T, w.d_h), float("nan"), dtype=dt, device="cuda")
        res = torch.full((w.K + 1,), -1.0, device="cuda")
        last = torch.full((rows, w.S, w.d_h), float("nan"), dtype=dt, device="cuda")
        if noalloc:
            B.prn_newton_forward_noalloc(xp, a, w.K, H, cell=w.cell, h0=h0d, cu_seqlens=cu, residual_out=res,
                                         state_last_out=last)
        else:
            n = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, w.K, n_seqs=n_seqs)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            B.prn_newton_forward(xp, a, w.K, H, cell=w.cell, h0=h0d, cu_seqlens=cu, residual_out=res,
                                 state_last_out=last, workspace=ws)
        torch.cuda.synchronize()
        outs.append((H, res, last))
    return outs


def _same(outs):
    (H1, r1, l1), (H2, r2, l2) = outs
    assert torch.equal(H1, H2) and torch.equal(r1, r2) and torch.equal(l1, l2)
    assert torch.isfinite(r2).all() and float(r2.min()) >= 0.0


def test_noalloc_matches_the_workspace_forward_on_two_calls_in_a_row():
    big = Workload("lstm_noalloc", "lstm", 3, 3000, 16, 200, "f32", 3)
    small = Workload("gru_noalloc", "gru", 1, 700, 16, 40, "bf16", 2)
    for w, h0 in ((big, None), (small, random_state(small, 1, seed=4))):
        say(f"[case] noalloc vs workspace forward {w}")
        _same(_both(w, small_inputs(w), h0))


def test_noalloc_full_size_ragged_pack():
    w = WORKLOADS["gru_ragged"]
    say(f"[case] noalloc full size {w}")
    _same(_both(w, make_inputs(w, seed=0)))


def test_noalloc_rejects_a_call_larger_than_its_scratch():
    w = WORKLOADS["lstm_t131k"].scaled(T=16384, B=8)   # 8 x 16384 LSTM: more records than the scratch holds
    dt = TORCH_DT[w.dtype]
    need = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, w.K)
    assert need > B.NOALLOC_SCRATCH_BYTES
    xp = torch.zeros((w.B, w.T, w.G, w.d_h), device="cuda")
    a = torch.zeros((w.G, w.d_h), device="cuda")
    H = torch.empty((w.B, w.T, w.d_h), device="cuda")
    with pytest.raises(B.PrnError, match="scratch"):
        B.prn_newton_forward_noalloc(xp, a, w.K, H, cell=w.cell)
