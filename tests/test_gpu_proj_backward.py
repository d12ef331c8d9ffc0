"""GPU parity of the projection's backward (prn_input_proj_backward: dx, dW,
dbias) against the oracle's float64 products (oracle.proj.input_proj_backward,
pinned by finite differences), element by element.

Bands, with ref_abs the same sums taken over absolute values (the scale
floating-point summation errors are measured against):
  fp32 storage: |got - ref| <= 1e-5 ref_abs
  bf16 storage: |got - ref| <= 2^-8 |ref| + 2e-5 ref_abs  (one rounding of the
                result to 8 significant bits, fp32 accumulation)
Shapes cover ragged tiles, rows of dxproj that are not whole 16-byte chunks
(the padded-copy path), the weight gradient read along the operand rows
(G d_h and d_in multiples of 256) and through transposed copies, a
misaligned dxproj (rejected) and a misaligned x where the rows are read
directly (rejected), T = 0, optional outputs, and the long LSTM workload at
full size on sampled entries."""
import numpy as np
import pytest
import torch

from gpu_helpers import TORCH_DT, say, to_f64
from nonlinear_rnn_amd import binding as B
from oracle import proj as oproj

pytestmark = pytest.mark.gpu


def _inputs(cell, dtype, Bn, T, d_in, d_h, seed):
    G = B.GATES[cell]
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = TORCH_DT[dtype]
    dxp = torch.randn((Bn, T, G, d_h), generator=g, device="cuda").to(dt)
    x = torch.randn((Bn, T, d_in), generator=g, device="cuda").to(dt)
    W = (torch.randn((G * d_h, d_in), generator=g, device="cuda") / d_in ** 0.5).to(dt)
    return dxp, x, W


def _run(cell, dxp, x, W, *, dx=True, dW=True, db=True):
    Bn, T, G, d_h = dxp.shape
    d_in = x.shape[-1]
    n = B.prn_input_proj_backward_workspace_bytes(cell, dxp.dtype, Bn, T, d_in, d_h)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    out_dx = torch.full_like(x, float("nan")) if dx else None
    out_dW = torch.full_like(W, float("nan")) if dW else None
    out_db = torch.full((G * d_h,), float("nan"), device="cuda") if db else None
    B.prn_input_proj_backward(dxp, x, W, cell=cell, dx_out=out_dx, dW_out=out_dW, dbias_out=out_db, workspace=ws)
    torch.cuda.synchronize()
    return out_dx, out_dW, out_db


def _check(dtype, got, ref, ref_abs, what):
    got = to_f64(got)
    band = 1e-5 * ref_abs if dtype == "f32" else 2.0 ** -8 * np.abs(ref) + 2e-5 * ref_abs
    worst = float((np.abs(got - ref) / np.maximum(band, 1e-30)).max()) if got.size else 0.0
    say(f"  {what}: max|got - ref| {np.abs(got - ref).max() if got.size else 0:.2e}, worst / band {worst:.2f}")
    assert worst <= 1.0, what


CASES = [
    ("gru", "f32", 3, 1000, 24, 80),
    ("lstm", "f32", 2, 777, 40, 72),
    ("gru", "f32", 2, 300, 16, 70),     # dxproj rows of 840 bytes: padded copy
    ("gru", "bf16", 2, 600, 32, 64),
    ("lstm", "bf16", 2, 300, 40, 130),
    ("gru", "bf16", 1, 513, 24, 42),    # rows of 252 bytes: padded copy
    ("lstm", "f32", 1, 1, 4, 16),
    ("gru", "f32", 4, 2048, 256, 256),  # G d_h and d_in multiples of 256: dW along the rows, no transposes
    ("gru", "f32", 1, 1234, 512, 256),  # the same with a ragged last slice of tokens
    ("lstm", "bf16", 2, 1500, 256, 128),
    ("gru", "f32", 1, 700, 512, 256),   # two column tiles of dW: only the first takes the dbias sums
    ("gru", "bf16", 1, 700, 512, 256),
]


@pytest.mark.parametrize("cell,dtype,Bn,T,d_in,d_h", CASES)
def test_projection_backward_matches_oracle(cell, dtype, Bn, T, d_in, d_h):
    say(f"[case] projection backward {cell} {dtype} B={Bn} T={T} d_in={d_in} d_h={d_h}")
    dxp, x, W = _inputs(cell, dtype, Bn, T, d_in, d_h, seed=T + d_h)
    dx, dW, db = _run(cell, dxp, x, W)
    g64, x64, W64 = to_f64(dxp), to_f64(x), to_f64(W)
    rdx, rdW, rdb = oproj.input_proj_backward(g64, x64, W64)
    adx, adW, adb = oproj.input_proj_backward(np.abs(g64), np.abs(x64), np.abs(W64))
    _check(dtype, dx, rdx, adx, "dx")
    _check(dtype, dW, rdW, adW, "dW")
    _check("f32", db, rdb, adb, "dbias")
    # bitwise reproducible
    dx2, dW2, db2 = _run(cell, dxp, x, W)
    assert torch.equal(dx, dx2) and torch.equal(dW, dW2) and torch.equal(db, db2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dbias_with_and_without_the_weight_gradient(dtype):
    """Where dW reads the operand rows (G d_h and d_in multiples of 256) the
    dW tiles also take dbias's column sums (one per token slice); asked for
    alone, dbias comes from 64-token column sums.  Both against the oracle,
    and each bitwise reproducible."""
    cell = "gru"
    dxp, x, W = _inputs(cell, dtype, 2, 1500, 256, 256, seed=11)
    _, _, db_all = _run(cell, dxp, x, W)
    _, _, db_alone = _run(cell, dxp, x, W, dx=False, dW=False)
    g64 = to_f64(dxp).reshape(-1, dxp.shape[-2] * dxp.shape[-1])
    ref, ref_abs = g64.sum(0), np.abs(g64).sum(0)
    _check("f32", db_all, ref, ref_abs, "dbias with dW")
    _check("f32", db_alone, ref, ref_abs, "dbias alone")
    assert torch.equal(db_all, _run(cell, dxp, x, W)[2])
    assert torch.equal(db_alone, _run(cell, dxp, x, W, dx=False, dW=False)[2])


def test_projection_backward_optional_outputs_misaligned_input_and_empty():
    cell, dtype = "lstm", "f32"
    dxp, x, W = _inputs(cell, dtype, 2, 500, 24, 40, seed=3)
    full = _run(cell, dxp, x, W)
    for flags in ((True, False, False), (False, True, False), (False, False, True), (False, True, True)):
        part = _run(cell, dxp, x, W, dx=flags[0], dW=flags[1], db=flags[2])
        for f, a, b in zip(flags, full, part):
            assert (b is None) if not f else torch.equal(a, b)
    # dxproj at an address that is not 16-byte aligned (one element into a larger buffer): rejected
    buf = torch.empty(dxp.numel() + 1, device="cuda")
    dxm = buf[1:].view(dxp.shape)
    with pytest.raises(B.PrnError, match="16-byte"):
        _run(cell, dxm, x, W)
    # x not 16-byte aligned where dW reads the operand rows directly (G d_h, d_in multiples of 256): rejected
    dxq, xq, Wq = _inputs("gru", dtype, 1, 300, 256, 256, seed=4)
    xbuf = torch.empty(xq.numel() + 1, device="cuda")
    xm = xbuf[1:].view(xq.shape)
    xm.copy_(xq)
    with pytest.raises(B.PrnError, match="16-byte"):
        _run("gru", dxq, xm, Wq)
    dxo, _, _ = _run("gru", dxq, xm, Wq, dW=False)   # dx and dbias alone do not read x
    assert torch.equal(dxo, _run("gru", dxq, xq, Wq, dW=False)[0])
    # T = 0: dW = 0, dbias = 0, dx empty
    e = _run(cell, dxp[:, :0].contiguous(), x[:, :0].contiguous(), W)
    assert e[0].numel() == 0 and float(e[1].abs().max()) == 0.0 and float(e[2].abs().max()) == 0.0


def test_projection_backward_full_size_sampled():
    """The long LSTM workload's shapes (262144 tokens, 1024 gate channels,
    d_in 256): every entry against the bands where the oracle takes it
    cheaply (dx on sampled tokens, dW and dbias on sampled gate channels)."""
    cell, dtype, Bn, T, d_in, d_h = "lstm", "f32", 2, 131072, 256, 256
    say(f"[case] projection backward full size {cell} {dtype} {Bn}x{T} d_in={d_in} d_h={d_h}")
    dxp, x, W = _inputs(cell, dtype, Bn, T, d_in, d_h, seed=7)
    dx, dW, db = _run(cell, dxp, x, W)
    G = 4
    g2 = dxp.reshape(Bn * T, G * d_h)
    x2 = x.reshape(Bn * T, d_in)
    rows = torch.tensor([0, 1, 4095, 131071, 131072, 262143], device="cuda")
    cols = torch.tensor([0, 5, 255, 256, 700, 1023], device="cuda")
    gm, W64 = to_f64(g2[rows]), to_f64(W)
    _check(dtype, dx.reshape(Bn * T, d_in)[rows], gm @ W64, np.abs(gm) @ np.abs(W64), "dx (sampled tokens)")
    gc, x64 = to_f64(g2[:, cols]), to_f64(x2)
    _check(dtype, dW[cols], gc.T @ x64, np.abs(gc).T @ np.abs(x64), "dW (sampled gate channels)")
    _check("f32", db[cols], gc.sum(0), np.abs(gc).sum(0), "dbias (sampled gate channels)")
