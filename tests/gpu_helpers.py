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
    return f32 if w.dtype == "f32" else bf16


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


__all__ = ["prn", "say", "to_dev", "to_f64", "gpu_run", "gpu_run_fused", "gpu_sequential", "oracle_newton", "oracle_sequential",
           "tol", "small_inputs", "TORCH_DT"]
