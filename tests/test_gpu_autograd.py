"""The differentiable training surface (newton_apply + input_proj_apply):
autograd gradients of a loss through projection and Newton against the
oracle's adjoint at the same trajectory, chained through the projection in
float64.  Tolerances relative to 1 + max|reference|: 1e-5 for per-token
gradients (x, h0), 1e-4 for gradients summed over all tokens (W, bias, a)."""
import numpy as np
import pytest
import torch

import nonlinear_rnn_amd as prn
from gpu_helpers import say, to_f64
from nonlinear_rnn_amd import binding as B
from oracle import backward as obackward

pytestmark = pytest.mark.gpu


def rel(got, ref):
    return float(np.abs(got - ref).max() / (1.0 + np.abs(ref).max()))


@pytest.mark.parametrize("cell,K,cu", [("gru", 3, None), ("lstm", 4, None), ("gru", 3, [0, 300, 300, 800, 1000]),
                                       ("lstm", 4, [0, 1, 517, 1000])])
def test_autograd_matches_oracle(cell, K, cu):
    g = torch.Generator(device="cuda").manual_seed(5)
    G, S = (3, 1) if cell == "gru" else (4, 2)
    Bn = 2 if cu is None else 1
    T, d_in, d_h = 1000, 24, 72
    rows = Bn if cu is None else len(cu) - 1
    x = torch.randn((Bn, T, d_in), generator=g, device="cuda").requires_grad_()
    W = (torch.randn((G * d_h, d_in), generator=g, device="cuda") / d_in ** 0.5).requires_grad_()
    bias = (0.1 * torch.randn(G * d_h, generator=g, device="cuda")).requires_grad_()
    a = (torch.rand((G, d_h), generator=g, device="cuda") - 0.5).requires_grad_()
    h0 = (0.5 * torch.randn((rows, S, d_h), generator=g, device="cuda")).requires_grad_()
    wgt = torch.randn((Bn, T, d_h), generator=g, device="cuda")
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32)
    xproj = prn.input_proj_apply(x, W, bias, cell=cell)
    H = prn.newton_apply(xproj, a, K, cell=cell, h0=h0, cu_seqlens=cu_t)
    (H * wgt).sum().backward()

    # the trajectory the gradient is taken at, and the oracle's adjoint there
    with torch.no_grad():
        xp = xproj.detach().contiguous()
        states = torch.empty((Bn, T, S, d_h), device="cuda")
        Hn = torch.empty((Bn, T, d_h), device="cuda")
        ws = torch.empty(B.prn_workspace_bytes(cell, torch.float32, Bn, T, d_h, K, n_seqs=rows if cu else 0),
                         dtype=torch.uint8, device="cuda")
        B.prn_newton_forward(xp, a.detach(), K, Hn, cell=cell, h0=h0.detach(),
                             cu_seqlens=None if cu is None else cu_t.cuda(), states_out=states, workspace=ws)
    dxp, da, dh0 = obackward.adjoint(cell, to_f64(xp), to_f64(a), to_f64(states), to_f64(wgt), h0=to_f64(h0),
                                     cu_seqlens=cu)
    gtok = dxp.reshape(Bn * T, G * d_h)
    dx = (gtok @ to_f64(W)).reshape(Bn, T, d_in)
    dW = gtok.T @ to_f64(x).reshape(Bn * T, d_in)
    db = gtok.sum(0)
    errs = {"x": rel(to_f64(x.grad), dx), "W": rel(to_f64(W.grad), dW), "bias": rel(to_f64(bias.grad), db),
            "a": rel(to_f64(a.grad), da), "h0": rel(to_f64(h0.grad), dh0)}
    say(f"[case] autograd {cell} K={K} cu={cu}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert errs["x"] <= 1e-5 and errs["h0"] <= 1e-5
    assert errs["W"] <= 1e-4 and errs["bias"] <= 1e-4 and errs["a"] <= 1e-4


def test_autograd_gradient_is_the_unrolls_at_kstar():
    """At K = K*, the gradient through Newton equals the gradient of the
    sequential unroll (the oracle's adjoint at the unroll's trajectory) to
    about the agreement tolerance."""
    from oracle import newton as onewton
    g = torch.Generator(device="cuda").manual_seed(9)
    T, d_h = 800, 64
    xproj = torch.randn((2, T, 4, d_h), generator=g, device="cuda").requires_grad_()
    a = (torch.rand((4, d_h), generator=g, device="cuda") - 0.5).requires_grad_()
    wgt = torch.randn((2, T, d_h), generator=g, device="cuda")
    H = prn.newton_apply(xproj, a, None, cell="lstm")      # K from the measured K*(T) table
    (H * wgt).sum().backward()
    seq, _ = onewton.sequential("lstm", to_f64(xproj), to_f64(a))
    dxp, da, _ = obackward.adjoint("lstm", to_f64(xproj), to_f64(a), seq, to_f64(wgt))
    e = rel(to_f64(xproj.grad), dxp)
    say(f"  gradient vs the unroll's: {e:.1e}")
    assert e <= 1e-3


@pytest.mark.parametrize("cell,cu", [("lstm", None), ("gru", [0, 200, 200, 700, 900])])
def test_recompute_gives_the_stored_trajectory_gradients(cell, cu):
    """recompute=True rebuilds the trajectory in the backward: the same
    kernels on the same inputs give the same trajectory bit for bit, so the
    gradients equal those of the stored-trajectory backward exactly."""
    g = torch.Generator(device="cuda").manual_seed(3)
    G, S = (3, 1) if cell == "gru" else (4, 2)
    Bn = 2 if cu is None else 1
    T, d_h = 900, 80
    rows = Bn if cu is None else len(cu) - 1
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32)
    xp0 = torch.randn((Bn, T, G, d_h), generator=g, device="cuda")
    a0 = torch.rand((G, d_h), generator=g, device="cuda") - 0.5
    h00 = 0.5 * torch.randn((rows, S, d_h), generator=g, device="cuda")
    wgt = torch.randn((Bn, T, d_h), generator=g, device="cuda")
    grads = []
    for rc in (False, True):
        xp, a, h0 = (t.clone().requires_grad_() for t in (xp0, a0, h00))
        H = prn.newton_apply(xp, a, 3, cell=cell, h0=h0, cu_seqlens=cu_t, recompute=rc)
        (H * wgt).sum().backward()
        grads.append([to_f64(t.grad) for t in (xp, a, h0)])
    for name, u, v in zip(("xproj", "a", "h0"), *grads):
        say(f"  recompute vs stored, {cell} {name}: {rel(u, v):.1e}")
        assert np.array_equal(u, v)
