"""The T = 1 decode step (projection and cell fused, one launch per token):
against the oracle's projection + one sequential step, against the library's
own projection + sequential kernels, chained after a Newton prefill, and
captured in a CUDA graph.

Tolerances (max-abs): fp32 1e-5 (the projection's fp32 sum against fp64,
carried through one cell step whose derivative is at most about 1); bf16
2e-2, as for the other bf16 paths (the projected value and the stored state
each take one bf16 rounding).  The prefill + decode chain against the
oracle's unroll uses tau = 1e-4, the Newton prefill's agreement bound.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say, to_dev, to_f64, TORCH_DT
from nonlinear_rnn_amd import binding as B
from oracle import newton as onewton
from oracle import proj as oproj
from oracle import rounding as oround

pytestmark = pytest.mark.gpu

GS = {"gru": (3, 1), "lstm": (4, 2)}


def inputs(cell, dtype, slots, d_in, d_h, seed):
    rng = np.random.default_rng(seed)
    G, S = GS[cell]
    x = oround.store(rng.standard_normal((slots, d_in)), dtype)
    W = oround.store(rng.standard_normal((G * d_h, d_in)) / np.sqrt(d_in), dtype)
    bias = (0.1 * rng.standard_normal(G * d_h)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (G, d_h)).astype(np.float32)
    s0 = oround.store(0.5 * rng.standard_normal((slots, S, d_h)), dtype)
    return x, W, bias, a, s0


def run_decode(cell, dtype, x, W, bias, a, s0, with_h=True):
    G, S = GS[cell]
    dt = TORCH_DT[dtype]
    slots, d_h = x.shape[0], W.shape[0] // G
    xd, Wd = to_dev(x, dtype), to_dev(W, dtype)
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    ad = torch.from_numpy(a).cuda()
    sin = None if s0 is None else to_dev(s0, dtype)
    sout = torch.empty((slots, S, d_h), dtype=dt, device="cuda")
    h = torch.empty((slots, d_h), dtype=dt, device="cuda") if with_h else None
    B.prn_decode_step(xd, Wd, bd, ad, sout, cell=cell, state_in=sin, h_out=h)
    torch.cuda.synchronize()
    return sout, h


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("dtype,slots,d_in,d_h", [("f32", 5, 36, 130), ("bf16", 5, 40, 130), ("f32", 16, 4, 64),
                                                  ("bf16", 37, 512, 1000), ("f32", 3, 1024, 257),
                                                  ("f32", 33, 7, 6), ("bf16", 17, 13, 70), ("f32", 1, 1, 1),
                                                  ("f32", 64, 256, 256)])
@pytest.mark.parametrize("with_state", [True, False])
def test_decode_step_matches_oracle(cell, dtype, slots, d_in, d_h, with_state):
    """Slot counts around the 16-slot group (1, 3, 5, 16, 17, 33, 37, 64),
    channel counts around the 4-channel workgroup, d_in around the 64-lane
    row piece (1, 4, 7, 13, 36, 40, 256, 512, 1024)."""
    say(f"[case] decode {cell} {dtype} slots={slots} d_in={d_in} d_h={d_h} state={with_state}")
    G, S = GS[cell]
    x, W, bias, a, s0 = inputs(cell, dtype, slots, d_in, d_h, seed=d_in * 7 + d_h)
    s0 = s0 if with_state else None
    sout, h = run_decode(cell, dtype, x, W, bias, a, s0)
    # x, W and s0 hold values the storage dtype represents exactly (oracle rounding.store)
    xp = oproj.input_proj(x[:, None], W, bias.astype(np.float64), G)
    st, last = onewton.sequential(cell, xp, a.astype(np.float64), h0=s0)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.abs(to_f64(sout) - last).max() <= tol
    assert np.array_equal(to_f64(h), to_f64(sout)[:, S - 1])


@pytest.mark.parametrize("cell,dtype", [("gru", "f32"), ("lstm", "f32"), ("lstm", "bf16")])
def test_decode_step_equals_projection_then_sequential_kernel(cell, dtype):
    """Same token through prn_input_proj + prn_sequential_forward (T = 1)."""
    G, S = GS[cell]
    dt = TORCH_DT[dtype]
    x, W, bias, a, s0 = inputs(cell, dtype, 4, 64, 200, seed=3)
    sout, h = run_decode(cell, dtype, x, W, bias, a, s0)
    xd, Wd = to_dev(x, dtype)[:, None].contiguous(), to_dev(W, dtype)
    xp = torch.empty((4, 1, G, 200), dtype=dt, device="cuda")
    B.prn_input_proj(xd, Wd, torch.from_numpy(bias).cuda(), xp, cell=cell)
    H = torch.empty((4, 1, 200), dtype=dt, device="cuda")
    last = torch.empty((4, S, 200), dtype=dt, device="cuda")
    B.prn_sequential_forward(xp, torch.from_numpy(a).cuda(), H, cell=cell, h0=to_dev(s0, dtype), state_last_out=last)
    torch.cuda.synchronize()
    e = np.abs(to_f64(sout) - to_f64(last)).max()
    say(f"  decode vs proj + sequential: {e:.2e}")
    assert e <= (1e-5 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("cell,K", [("gru", 3), ("lstm", 4)])
def test_prefill_with_newton_then_decode_chain(cell, K):
    """Prefill T0 tokens with Newton (final carry out), then N decode steps on
    ping-pong carries: the outputs follow the oracle's unroll over T0 + N."""
    G, S = GS[cell]
    rng = np.random.default_rng(17)
    slots, T0, N, d_in, d_h = 3, 700, 12, 32, 96
    x = rng.standard_normal((slots, T0 + N, d_in)).astype(np.float32)
    W = (rng.standard_normal((G * d_h, d_in)) / np.sqrt(d_in)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(G * d_h)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (G, d_h)).astype(np.float32)
    xd, Wd = torch.from_numpy(x).cuda(), torch.from_numpy(W).cuda()
    bd, ad = torch.from_numpy(bias).cuda(), torch.from_numpy(a).cuda()
    xp = torch.empty((slots, T0, G, d_h), device="cuda")
    B.prn_input_proj(xd[:, :T0].contiguous(), Wd, bd, xp, cell=cell)
    H = torch.empty((slots, T0, d_h), device="cuda")
    carry = [torch.empty((slots, S, d_h), device="cuda") for _ in range(2)]
    ws = torch.empty(B.prn_workspace_bytes(cell, torch.float32, slots, T0, d_h, K), dtype=torch.uint8, device="cuda")
    B.prn_newton_forward(xp, ad, K, H, cell=cell, state_last_out=carry[0], workspace=ws)
    hs = torch.empty((N, slots, d_h), device="cuda")
    for i in range(N):
        B.prn_decode_step(xd[:, T0 + i].contiguous(), Wd, bd, ad, carry[(i + 1) % 2], cell=cell,
                          state_in=carry[i % 2], h_out=hs[i])
    torch.cuda.synchronize()
    xp64 = oproj.input_proj(x.astype(np.float64), W.astype(np.float64), bias.astype(np.float64), G)
    st, last = onewton.sequential(cell, xp64, a.astype(np.float64))
    ref = st[:, T0:, S - 1].transpose(1, 0, 2)
    e = np.abs(to_f64(hs) - ref).max()
    el = np.abs(to_f64(carry[N % 2]) - last).max()
    say(f"[case] prefill+decode {cell}: h {e:.2e} carry {el:.2e}")
    assert e <= 1e-4 and el <= 1e-4


@pytest.mark.parametrize("cell,dtype", [("lstm", "f32"), ("gru", "bf16")])
def test_decode_steps_captured_in_a_graph(cell, dtype):
    """Four decode steps captured once and replayed three times on new tokens;
    every replay equals the same steps run eagerly."""
    G, S = GS[cell]
    dt = TORCH_DT[dtype]
    slots, d_in, d_h, steps = 6, 64, 160, 4
    x, W, bias, a, s0 = inputs(cell, dtype, slots, d_in, d_h, seed=23)
    Wd, bd, ad = to_dev(W, dtype), torch.from_numpy(bias).cuda(), torch.from_numpy(a).cuda()
    xs = torch.zeros((steps, slots, d_in), dtype=dt, device="cuda")
    carry = [torch.zeros((slots, S, d_h), dtype=dt, device="cuda") for _ in range(2)]
    hs = torch.zeros((steps, slots, d_h), dtype=dt, device="cuda")

    def run_steps():
        for i in range(steps):
            B.prn_decode_step(xs[i], Wd, bd, ad, carry[(i + 1) % 2], cell=cell, state_in=carry[i % 2], h_out=hs[i])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_steps()                           # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps()
    rng = np.random.default_rng(5)
    for rep in range(3):
        tok = to_dev(rng.standard_normal((steps, slots, d_in)), dtype)
        init = to_dev(0.5 * rng.standard_normal((slots, S, d_h)), dtype)
        xs.copy_(tok)
        carry[0].copy_(init)
        graph.replay()
        torch.cuda.synchronize()
        got_h, got_c = hs.clone(), carry[steps % 2].clone()
        xs.copy_(tok)
        carry[0].copy_(init)
        run_steps()                           # the same steps, eagerly
        torch.cuda.synchronize()
        assert torch.equal(got_h, hs) and torch.equal(got_c, carry[steps % 2]), rep
        say(f"  replay {rep}: equal to eager")
