"""Shared plumbing for the GPU parity tests: moving seeded inputs to the
device, running the HIP path through the C ABI, and running the oracle on
the very same stored numbers (float64 upcast of the GPU's own projected
inputs, so the Newton comparison isolates the Newton engine)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import nonlinear_rnn_amd as prn
from nonlinear_rnn_amd import binding as B
from oracle import backward as obackward
from oracle import newton as onewton
from oracle import rounding as oround
from workloads import Workload, make_inputs

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype: str) -> torch.Tensor:
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_run(w: Workload, inp: dict, K: int, *, h0=None, xproj=None, with_state=True, cu=None):
    """Projection (unless xproj is given) + Newton through the C ABI.

    Returns dict(xproj, H, res (K+1), last)."""
    dt = TORCH_DT[w.dtype]
    if xproj is None:
        x = to_dev(inp["x"], w.dtype)
        W = to_dev(inp["W"], w.dtype)
        bias = torch.from_numpy(inp["bias"]).cuda()
        xproj = torch.empty((w.B, w.T, w.G, w.d_h), dtype=dt, device="cuda")
        B.prn_input_proj(x, W, bias, xproj, cell=w.cell)
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"] if cu is None else cu
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    n_seqs = 0 if cu is None else len(cu) - 1
    rows = w.B if cu is None else n_seqs
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    res = torch.full((K + 1,), -1.0, dtype=torch.float32, device="cuda")
    last = torch.empty((rows, w.S, w.d_h), dtype=dt, device="cuda") if with_state else None
    h0_d = None if h0 is None else to_dev(h0, w.dtype)
    ws_n = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, K, n_seqs=n_seqs)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    B.prn_newton_forward(xproj, a, K, H, cell=w.cell, h0=h0_d, cu_seqlens=cu_d, residual_out=res,
                         state_last_out=last, workspace=ws)
    torch.cuda.synchronize()
    return {"xproj": xproj, "H": H, "res": res.cpu().numpy().astype(np.float64), "last": last}


def gpu_sequential(w: Workload, inp: dict, xproj, *, h0=None, cu=None):
    dt = TORCH_DT[w.dtype]
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"] if cu is None else cu
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    rows = w.B if cu is None else len(cu) - 1
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    last = torch.empty((rows, w.S, w.d_h), dtype=dt, device="cuda")
    h0_d = None if h0 is None else to_dev(h0, w.dtype)
    B.prn_sequential_forward(xproj, a, H, cell=w.cell, h0=h0_d, cu_seqlens=cu_d, state_last_out=last)
    torch.cuda.synchronize()
    return H, last


def oracle_h0(w, h0):
    return None if h0 is None else oround.store(h0, w.dtype)


def oracle_newton(w: Workload, xp64, a, K, *, h0=None, cu=None):
    return onewton.newton(w.cell, xp64, np.asarray(a, np.float64), K, h0=oracle_h0(w, h0), cu_seqlens=cu,
                          dtype=w.dtype)


def oracle_sequential(w: Workload, xp64, a, *, h0=None, cu=None):
    return onewton.sequential(w.cell, xp64, np.asarray(a, np.float64), h0=oracle_h0(w, h0), cu_seqlens=cu)


def tol(w: Workload, f32: float, bf16: float = 2e-2) -> float:
    """A scalar band: f32 for fp32 storage, bf16 for bf16 storage (used for
    residuals, whose bf16 floor is about 2^-9 max|h|)."""
    return f32 if w.dtype == "f32" else bf16


BF16_ABS = 4e-3   # twice the largest bf16 error seen on h (1.95e-3, one rounding of |h| < 1)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers (8 significant bits) at |x|."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def state_err(w: Workload, got, ref, f32: float) -> float:
    """Largest |got - ref| as a fraction of the allowed band (<= 1 passes).
    fp32 storage: the fixed f32.  bf16 storage: BF16_ABS, or one bf16 ulp of
    the reference where that is larger (an LSTM cell state above 1); every
    stored value carries one rounding to 8 significant bits."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    band = f32 if w.dtype == "f32" else np.maximum(BF16_ABS, bf16_ulp(ref))
    return float((np.abs(got - ref) / band).max())


def small_inputs(w: Workload, seed: int = 0) -> dict:
    return make_inputs(w, seed=seed)




def gpu_run_fused(w: Workload, inp: dict, K: int, *, h0=None, cu=None, with_xproj=True, with_state=True):
    """prn_newton_forward_fused through the C ABI (projection inside the Newton
    kernel).  Returns dict(xproj (or None), H, res (K+1), last)."""
    dt = TORCH_DT[w.dtype]
    x = to_dev(inp["x"], w.dtype)
    W = to_dev(inp["W"], w.dtype)
    bias = torch.from_numpy(inp["bias"]).cuda()
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"] if cu is None else cu
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    n_seqs = 0 if cu is None else len(cu) - 1
    rows = w.B if cu is None else n_seqs
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    res = torch.full((K + 1,), -1.0, dtype=torch.float32, device="cuda")
    last = torch.empty((rows, w.S, w.d_h), dtype=dt, device="cuda") if with_state else None
    xproj = torch.empty((w.B, w.T, w.G, w.d_h), dtype=dt, device="cuda") if with_xproj else None
    h0_d = None if h0 is None else to_dev(h0, w.dtype)
    ws_n = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, K, n_seqs=n_seqs)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    B.prn_newton_forward_fused(x, W, bias, a, K, H, cell=w.cell, h0=h0_d, cu_seqlens=cu_d, residual_out=res,
                               xproj_out=xproj, state_last_out=last, workspace=ws)
    torch.cuda.synchronize()
    return {"xproj": xproj, "H": H, "res": res.cpu().numpy().astype(np.float64), "last": last}


# backward: the forward's trajectory through states_out, the backward through
# the C ABI, and the oracle's adjoint on the same stored numbers


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / (1.0 + np.abs(ref).max())) if ref.size else 0.0


def tols(w):
    return (1e-5, 1e-4) if w.dtype == "f32" else (1e-2, 1e-4)


def gpu_forward_states(w, inp, K, h0=None, cu=None, xproj=None):
    """Newton forward with states_out; returns (xproj, H, states, last)."""
    dt = TORCH_DT[w.dtype]
    out = gpu_run(w, inp, K, h0=h0, cu=cu, xproj=xproj)
    xproj = out["xproj"]
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"] if cu is None else cu
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    n_seqs = 0 if cu is None else len(cu) - 1
    rows = w.B if cu is None else n_seqs
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device="cuda")
    states = torch.full((w.B, w.T, w.S, w.d_h), float("nan"), dtype=dt, device="cuda")
    last = torch.empty((rows, w.S, w.d_h), dtype=dt, device="cuda")
    ws_n = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, K, n_seqs=n_seqs)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    h0_d = None if h0 is None else to_dev(h0, w.dtype)
    B.prn_newton_forward(xproj, a, K, H, cell=w.cell, h0=h0_d, cu_seqlens=cu_d, state_last_out=last,
                         states_out=states, workspace=ws)
    torch.cuda.synchronize()
    return xproj, H, states, last


def gpu_backward(w, inp, xproj, states, dH, *, h0=None, cu=None, dsl=None, want_dh0=True):
    dt = TORCH_DT[w.dtype]
    a = torch.from_numpy(inp["a"]).cuda()
    cu = inp["cu_seqlens"] if cu is None else cu
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    n_seqs = 0 if cu is None else len(cu) - 1
    rows = w.B if cu is None else n_seqs
    dx = torch.full_like(xproj, float("nan"))
    da = torch.full((w.G, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    dh0 = torch.full((rows, w.S, w.d_h), float("nan"), dtype=dt, device="cuda") if want_dh0 else None
    ws_n = B.prn_backward_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, n_seqs=n_seqs)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    h0_d = None if h0 is None else to_dev(h0, w.dtype)
    B.prn_newton_backward(xproj, a, states, dH, dx, da, cell=w.cell, h0=h0_d, cu_seqlens=cu_d, dstate_last=dsl,
                          dh0_out=dh0, workspace=ws)
    torch.cuda.synchronize()
    return dx, da, dh0


def oracle_backward(w, inp, xproj, states, dH, *, h0=None, cu=None, dsl=None):
    cu = inp["cu_seqlens"] if cu is None else cu
    return obackward.adjoint(w.cell, to_f64(xproj), inp["a"].astype(np.float64), to_f64(states), to_f64(dH),
                             h0=None if h0 is None else oround.store(h0, w.dtype), cu_seqlens=cu,
                             dstate_last=None if dsl is None else to_f64(dsl))


def random_grads(w, rows, seed):
    rng = np.random.default_rng(seed)
    dH = to_dev(rng.standard_normal((w.B, w.T, w.d_h)), w.dtype)
    dsl = to_dev(rng.standard_normal((rows, w.S, w.d_h)), w.dtype)
    return dH, dsl


# head-mix GRU (dense 16 x 16 blocks per head), fp32 storage


def hm_inputs(Bn, T, d_h, seed, scale=0.5, with_h0=True):
    rng = np.random.default_rng(seed)
    xp = rng.standard_normal((Bn, T, 3, d_h)).astype(np.float32).astype(np.float64)
    A = (rng.uniform(-scale, scale, (3, d_h // 16, 16, 16)) / 4.0).astype(np.float32).astype(np.float64)
    h0 = (0.5 * rng.standard_normal((Bn, d_h))).astype(np.float32).astype(np.float64) if with_h0 else None
    return xp, A, h0


def hm_dev(a, dtype="f32"):
    """A device tensor of a (float64 values exactly representable in dtype)."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t if dtype == "f32" else t.to(torch.bfloat16)


def hm_newton(xp, A, K, h0=None, want_last=False, dtype="f32"):
    """Head-mix Newton forward on the GPU; xp and h0 must hold values of the storage dtype."""
    Bn, T, _, d_h = xp.shape
    dt = TORCH_DT[dtype]
    H = torch.empty((Bn, T, d_h), dtype=dt, device="cuda")
    res = torch.full((K + 1,), -1.0, device="cuda")
    last = torch.empty((Bn, d_h), dtype=dt, device="cuda") if want_last else None
    ws = torch.empty(max(B.prn_head_workspace_bytes(Bn, T, d_h, K, dtype=dt), 1), dtype=torch.uint8, device="cuda")
    B.prn_head_newton_forward(hm_dev(xp, dtype), hm_dev(A), K, H, h0=hm_dev(h0, dtype), residual_out=res,
                              state_last_out=last, workspace=ws)
    torch.cuda.synchronize()
    return to_f64(H), res.cpu().numpy().astype(np.float64), (None if last is None else to_f64(last))


def hm_sequential(xp, A, h0=None, dtype="f32"):
    Bn, T, _, d_h = xp.shape
    dt = TORCH_DT[dtype]
    H = torch.empty((Bn, T, d_h), dtype=dt, device="cuda")
    last = torch.empty((Bn, d_h), dtype=dt, device="cuda")
    B.prn_head_sequential_forward(hm_dev(xp, dtype), hm_dev(A), H, h0=hm_dev(h0, dtype), state_last_out=last)
    torch.cuda.synchronize()
    return to_f64(H), to_f64(last)


__all__ = ["prn", "say", "to_dev", "to_f64", "gpu_run", "gpu_run_fused", "gpu_sequential", "oracle_newton", "oracle_sequential",
           "tol", "state_err", "bf16_ulp", "BF16_ABS", "small_inputs", "TORCH_DT", "rel_err", "tols", "gpu_forward_states", "gpu_backward", "oracle_backward",
           "random_grads", "hm_inputs", "hm_dev", "hm_newton", "hm_sequential"]
