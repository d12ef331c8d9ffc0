"""ctypes binding of libprn (include/prn.h): argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that live on the GPU (torch provides device memory and streams),
checks that their shapes, dtypes and layouts are what the C ABI expects, and
raises PrnError with the library's message on a non-OK status.  All
arithmetic happens in the HIP library; if the library is missing, loading
fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PRN_LIB", os.path.join(HERE, "libprn.so"))

PRN_OK, PRN_ERR_INVALID_ARG, PRN_ERR_UNSUPPORTED, PRN_ERR_WORKSPACE, PRN_ERR_DEVICE = range(5)
STATUS_NAMES = {0: "PRN_OK", 1: "PRN_ERR_INVALID_ARG", 2: "PRN_ERR_UNSUPPORTED",
                3: "PRN_ERR_WORKSPACE", 4: "PRN_ERR_DEVICE"}
CELLS = {"gru": 0, "lstm": 1}
GATES = {"gru": 3, "lstm": 4}
STATE = {"gru": 1, "lstm": 2}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

# every symbol include/prn.h declares
EXPORTS = ("prn_input_proj", "prn_newton_forward", "prn_newton_forward_fused", "prn_sequential_forward",
           "prn_workspace_bytes",
           "prn_newton_backward", "prn_backward_workspace_bytes", "prn_decode_step", "prn_head_newton_forward",
           "prn_head_sequential_forward", "prn_head_workspace_bytes", "prn_validate_cu_seqlens",
           "prn_last_error", "prn_version", "prn_newton_forward_noalloc", "prn_input_proj_backward",
           "prn_input_proj_backward_workspace_bytes")
NOALLOC_SCRATCH_BYTES = 32 << 20   # PRN_NOALLOC_SCRATCH_BYTES


class PrnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class PrnUnsupportedError(PrnError, TypeError):
    """PRN_ERR_UNSUPPORTED: a valid request pinned to a path the library does
    not implement (shapes/layout page: an unsupported pinned path raises
    TypeError, with no silent remap)."""


PRN_FAULT_LOOKBACK = 1   # bit of prn_params.error_out


class prn_params(ctypes.Structure):
    _fields_ = [
        ("cell", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_h", ctypes.c_int64),
        ("n_seqs", ctypes.c_int64),
        ("a", ctypes.c_void_p),
        ("state_last_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("states_out", ctypes.c_void_p),
        ("picard_iters", ctypes.c_int32),
        ("error_out", ctypes.c_void_p),
    ]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libprn.so (built by nonlinear_rnn_amd.build); raise if it is not there."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libprn not built: {LIB_PATH} is missing "
                               "(run python -m nonlinear_rnn_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(prn_params)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.prn_input_proj.argtypes = [vp, vp, vp, P, vp]
        L.prn_newton_forward.argtypes = [vp, P, vp, i32, vp, vp, vp]
        L.prn_newton_forward_fused.argtypes = [vp, vp, vp, P, vp, i32, vp, vp, vp, vp]
        L.prn_newton_forward_noalloc.argtypes = [vp, P, vp, i32, vp, vp, vp]
        L.prn_input_proj_backward.argtypes = [vp, vp, vp, P, vp, vp, vp]
        L.prn_input_proj_backward_workspace_bytes.argtypes = [P]
        L.prn_input_proj_backward_workspace_bytes.restype = ctypes.c_size_t
        L.prn_sequential_forward.argtypes = [vp, P, vp, vp, vp]
        L.prn_workspace_bytes.argtypes = [P, i32]
        L.prn_workspace_bytes.restype = ctypes.c_size_t
        L.prn_newton_backward.argtypes = [vp, P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.prn_backward_workspace_bytes.argtypes = [P]
        L.prn_decode_step.argtypes = [vp, vp, vp, P, vp, vp, vp]
        L.prn_head_newton_forward.argtypes = [vp, P, vp, i32, vp, i32, vp, vp]
        L.prn_head_sequential_forward.argtypes = [vp, P, vp, i32, vp, vp]
        L.prn_head_workspace_bytes.argtypes = [P, i32, i32]
        L.prn_head_workspace_bytes.restype = ctypes.c_size_t
        L.prn_backward_workspace_bytes.restype = ctypes.c_size_t
        L.prn_validate_cu_seqlens.argtypes = [vp, i64, i64]
        L.prn_last_error.restype = ctypes.c_char_p
        L.prn_version.restype = i32
        for name in ("prn_input_proj", "prn_input_proj_backward", "prn_newton_forward", "prn_newton_forward_fused",
                     "prn_newton_forward_noalloc",
                     "prn_sequential_forward",
                     "prn_newton_backward",
                     "prn_decode_step", "prn_head_newton_forward", "prn_head_sequential_forward",
                     "prn_validate_cu_seqlens"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def prn_last_error() -> str:
    return lib().prn_last_error().decode()


def prn_version() -> int:
    return int(lib().prn_version())


def _check(status: int) -> None:
    if status == PRN_ERR_UNSUPPORTED:
        raise PrnUnsupportedError(status, prn_last_error())
    if status != PRN_OK:
        raise PrnError(status, prn_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def make_params(cell: str, dtype: torch.dtype, B: int, T: int, d_h: int, *, d_in: int = 0, n_seqs: int = 0,
                a=None, state_last_out=None, states_out=None, workspace=None, stream=None,
                picard_iters: int = 0, error_out=None) -> prn_params:
    if cell not in CELLS:
        raise ValueError(f"unknown cell {cell!r}")
    if dtype not in DTYPES:
        raise TypeError(f"unsupported storage dtype {dtype}")
    p = prn_params()
    p.cell, p.dtype = CELLS[cell], DTYPES[dtype]
    p.B, p.T, p.d_in, p.d_h, p.n_seqs = B, T, d_in, d_h, n_seqs
    p.a = _ptr(a)
    p.state_last_out = _ptr(state_last_out)
    p.states_out = _ptr(states_out)
    p.picard_iters = int(picard_iters)
    p.error_out = _ptr(error_out)
    if workspace is not None:
        p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    p.stream = _stream(stream) if torch.cuda.is_available() else 0
    return p


def prn_workspace_bytes(cell: str, dtype: torch.dtype, B: int, T: int, d_h: int, K: int, n_seqs: int = 0,
                        picard_iters: int = 0) -> int:
    p = make_params(cell, dtype, B, T, d_h, n_seqs=n_seqs, picard_iters=picard_iters)
    n = int(lib().prn_workspace_bytes(ctypes.byref(p), K))
    if n == 0 and prn_last_error():
        raise PrnError(PRN_ERR_INVALID_ARG, prn_last_error())
    return n


def prn_validate_cu_seqlens(cu_host, N: int) -> None:
    """Check ragged offsets on a host int32 array / CPU tensor."""
    import numpy as np
    arr = np.ascontiguousarray(torch.as_tensor(cu_host).cpu().numpy(), dtype=np.int32)
    _check(lib().prn_validate_cu_seqlens(arr.ctypes.data, arr.size - 1, N))


def prn_input_proj(x, W, bias, xproj_out, *, cell: str, stream=None) -> None:
    """xproj_out (B,T,G,d_h) = x (B,T,d_in) @ W (G*d_h, d_in)^T + bias (G*d_h)."""
    _dev(x, "x")
    _dev(W, "W", x.dtype)
    _dev(bias, "bias", torch.float32)
    _dev(xproj_out, "xproj_out", x.dtype)
    B, T, d_in = x.shape
    G = GATES[cell]
    d_h = W.shape[0] // G
    if W.shape != (G * d_h, d_in) or xproj_out.shape != (B, T, G, d_h):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} W {tuple(W.shape)} xproj {tuple(xproj_out.shape)}")
    if bias is not None and bias.shape != (G * d_h,):
        raise ValueError("bias must have G*d_h entries")
    p = make_params(cell, x.dtype, B, T, d_h, d_in=d_in, stream=stream)
    _check(lib().prn_input_proj(_ptr(x), _ptr(W), _ptr(bias), ctypes.byref(p), _ptr(xproj_out)))


def prn_input_proj_backward_workspace_bytes(cell: str, dtype: torch.dtype, B: int, T: int, d_in: int,
                                            d_h: int) -> int:
    p = make_params(cell, dtype, B, T, d_h, d_in=d_in)
    n = int(lib().prn_input_proj_backward_workspace_bytes(ctypes.byref(p)))
    if n == 0 and prn_last_error():
        raise PrnError(PRN_ERR_INVALID_ARG, prn_last_error())
    return n


def prn_input_proj_backward(dxproj, x, W, *, cell: str, dx_out=None, dW_out=None, dbias_out=None, workspace=None,
                            stream=None) -> None:
    """dx_out (B,T,d_in) = dxproj W, dW_out (G*d_h, d_in) = dxproj^T x, dbias_out (G*d_h) fp32 = column sums
    of dxproj (B,T,G,d_h); each output optional."""
    _dev(dxproj, "dxproj")
    _dev(x, "x", dxproj.dtype)
    _dev(W, "W", dxproj.dtype)
    _dev(dx_out, "dx_out", dxproj.dtype)
    _dev(dW_out, "dW_out", dxproj.dtype)
    _dev(dbias_out, "dbias_out", torch.float32)
    B, T, G, d_h = dxproj.shape
    d_in = x.shape[-1]
    if G != GATES[cell] or x.shape != (B, T, d_in) or W.shape != (G * d_h, d_in):
        raise ValueError(f"shape mismatch: dxproj {tuple(dxproj.shape)} x {tuple(x.shape)} W {tuple(W.shape)}")
    if dx_out is not None and dx_out.shape != x.shape:
        raise ValueError("dx_out must have the shape of x")
    if dW_out is not None and dW_out.shape != W.shape:
        raise ValueError("dW_out must have the shape of W")
    if dbias_out is not None and dbias_out.shape != (G * d_h,):
        raise ValueError("dbias_out must have G*d_h entries")
    p = make_params(cell, dxproj.dtype, B, T, d_h, d_in=d_in, workspace=workspace, stream=stream)
    _check(lib().prn_input_proj_backward(_ptr(dxproj), _ptr(x), _ptr(W), ctypes.byref(p), _ptr(dx_out),
                                         _ptr(dW_out), _ptr(dbias_out)))


def _newton_common(xproj, a, H_out, h0, cu_seqlens, state_last_out, cell):
    _dev(xproj, "xproj")
    _dev(a, "a", torch.float32)
    _dev(H_out, "H_out", xproj.dtype)
    _dev(h0, "h0", xproj.dtype)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(state_last_out, "state_last_out", xproj.dtype)
    B, T, G, d_h = xproj.shape
    if G != GATES[cell] or a.shape != (G, d_h) or H_out.shape != (B, T, d_h):
        raise ValueError(f"shape mismatch: xproj {tuple(xproj.shape)} a {tuple(a.shape)} H_out {tuple(H_out.shape)}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    rows = B if cu_seqlens is None else n_seqs
    S = STATE[cell]
    for t, name in ((h0, "h0"), (state_last_out, "state_last_out")):
        if t is not None and t.shape != (rows, S, d_h):
            raise ValueError(f"{name} must be {(rows, S, d_h)}, got {tuple(t.shape)}")
    return B, T, d_h, n_seqs


def _states_out(states_out, xproj, cell):
    _dev(states_out, "states_out", xproj.dtype)
    B, T, _, d_h = xproj.shape
    if states_out is not None and states_out.shape != (B, T, STATE[cell], d_h):
        raise ValueError(f"states_out must be {(B, T, STATE[cell], d_h)}, got {tuple(states_out.shape)}")


def _error_word(error_out):
    _dev(error_out, "error_out", torch.int32)
    if error_out is not None and error_out.numel() < 1:
        raise ValueError("error_out needs one int32 element")


def prn_newton_forward(xproj, a, K: int, H_out, *, cell: str, h0=None, cu_seqlens=None, residual_out=None,
                       state_last_out=None, states_out=None, workspace=None, stream=None,
                       picard_iters: int = 0, error_out=None) -> None:
    B, T, d_h, n_seqs = _newton_common(xproj, a, H_out, h0, cu_seqlens, state_last_out, cell)
    _states_out(states_out, xproj, cell)
    _dev(residual_out, "residual_out", torch.float32)
    _error_word(error_out)
    if residual_out is not None and residual_out.numel() < K + 1:
        raise ValueError("residual_out needs K + 1 entries")
    p = make_params(cell, xproj.dtype, B, T, d_h, n_seqs=n_seqs, a=a, state_last_out=state_last_out,
                    states_out=states_out, workspace=workspace, stream=stream, picard_iters=picard_iters,
                    error_out=error_out)
    _check(lib().prn_newton_forward(_ptr(xproj), ctypes.byref(p), _ptr(h0), K, _ptr(cu_seqlens),
                                    _ptr(H_out), _ptr(residual_out)))


def prn_newton_forward_noalloc(xproj, a, K: int, H_out, *, cell: str, h0=None, cu_seqlens=None,
                               residual_out=None, state_last_out=None, states_out=None, stream=None,
                               picard_iters: int = 0, error_out=None) -> None:
    """prn_newton_forward with the library's own static scratch instead of a
    caller workspace (for callers that cannot allocate); calls on one GPU must
    not overlap."""
    B, T, d_h, n_seqs = _newton_common(xproj, a, H_out, h0, cu_seqlens, state_last_out, cell)
    _states_out(states_out, xproj, cell)
    _dev(residual_out, "residual_out", torch.float32)
    _error_word(error_out)
    if residual_out is not None and residual_out.numel() < K + 1:
        raise ValueError("residual_out needs K + 1 entries")
    p = make_params(cell, xproj.dtype, B, T, d_h, n_seqs=n_seqs, a=a, state_last_out=state_last_out,
                    states_out=states_out, stream=stream, picard_iters=picard_iters, error_out=error_out)
    _check(lib().prn_newton_forward_noalloc(_ptr(xproj), ctypes.byref(p), _ptr(h0), K, _ptr(cu_seqlens),
                                            _ptr(H_out), _ptr(residual_out)))


def prn_newton_forward_fused(x, W, bias, a, K: int, H_out, *, cell: str, h0=None, cu_seqlens=None,
                             residual_out=None, xproj_out=None, state_last_out=None, states_out=None,
                             workspace=None, stream=None, error_out=None) -> None:
    """prn_input_proj + prn_newton_forward in one kernel: x (B,T,d_in), W (G*d_h, d_in), bias (G*d_h)
    fp32 or None; xproj_out (B,T,G,d_h) optionally receives the projected inputs."""
    _dev(x, "x")
    _dev(W, "W", x.dtype)
    _dev(bias, "bias", torch.float32)
    _dev(a, "a", torch.float32)
    _dev(H_out, "H_out", x.dtype)
    _dev(h0, "h0", x.dtype)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(state_last_out, "state_last_out", x.dtype)
    _dev(xproj_out, "xproj_out", x.dtype)
    _dev(residual_out, "residual_out", torch.float32)
    B, T, d_in = x.shape
    G, S = GATES[cell], STATE[cell]
    d_h = W.shape[0] // G
    if W.shape != (G * d_h, d_in) or a.shape != (G, d_h) or H_out.shape != (B, T, d_h):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} W {tuple(W.shape)} a {tuple(a.shape)} "
                         f"H_out {tuple(H_out.shape)}")
    if bias is not None and bias.shape != (G * d_h,):
        raise ValueError("bias must have G*d_h entries")
    if xproj_out is not None and xproj_out.shape != (B, T, G, d_h):
        raise ValueError(f"xproj_out must be {(B, T, G, d_h)}, got {tuple(xproj_out.shape)}")
    _dev(states_out, "states_out", x.dtype)
    if states_out is not None and states_out.shape != (B, T, S, d_h):
        raise ValueError(f"states_out must be {(B, T, S, d_h)}, got {tuple(states_out.shape)}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    rows = B if cu_seqlens is None else n_seqs
    for t, name in ((h0, "h0"), (state_last_out, "state_last_out")):
        if t is not None and t.shape != (rows, S, d_h):
            raise ValueError(f"{name} must be {(rows, S, d_h)}, got {tuple(t.shape)}")
    if residual_out is not None and residual_out.numel() < K + 1:
        raise ValueError("residual_out needs K + 1 entries")
    _error_word(error_out)
    p = make_params(cell, x.dtype, B, T, d_h, d_in=d_in, n_seqs=n_seqs, a=a, state_last_out=state_last_out,
                    states_out=states_out, workspace=workspace, stream=stream, error_out=error_out)
    _check(lib().prn_newton_forward_fused(_ptr(x), _ptr(W), _ptr(bias), ctypes.byref(p), _ptr(h0), K,
                                          _ptr(cu_seqlens), _ptr(H_out), _ptr(residual_out), _ptr(xproj_out)))


def prn_sequential_forward(xproj, a, H_out, *, cell: str, h0=None, cu_seqlens=None, state_last_out=None,
                           states_out=None, stream=None) -> None:
    B, T, d_h, n_seqs = _newton_common(xproj, a, H_out, h0, cu_seqlens, state_last_out, cell)
    _states_out(states_out, xproj, cell)
    p = make_params(cell, xproj.dtype, B, T, d_h, n_seqs=n_seqs, a=a, state_last_out=state_last_out,
                    states_out=states_out, stream=stream)
    _check(lib().prn_sequential_forward(_ptr(xproj), ctypes.byref(p), _ptr(h0), _ptr(cu_seqlens), _ptr(H_out)))


def prn_backward_workspace_bytes(cell: str, dtype: torch.dtype, B: int, T: int, d_h: int, n_seqs: int = 0) -> int:
    p = make_params(cell, dtype, B, T, d_h, n_seqs=n_seqs)
    n = int(lib().prn_backward_workspace_bytes(ctypes.byref(p)))
    if n == 0 and prn_last_error():
        raise PrnError(PRN_ERR_INVALID_ARG, prn_last_error())
    return n


def prn_newton_backward(xproj, a, states, dH, dxproj_out, da_out, *, cell: str, h0=None, cu_seqlens=None,
                        dstate_last=None, dh0_out=None, workspace=None, stream=None, error_out=None) -> None:
    """Gradients through the recurrence at the trajectory `states` (B,T,S,d_h):
    dxproj_out (B,T,G,d_h), da_out (G,d_h) fp32 and optionally dh0_out (rows,S,d_h)."""
    _dev(xproj, "xproj")
    _dev(a, "a", torch.float32)
    _dev(states, "states", xproj.dtype)
    _dev(dH, "dH", xproj.dtype)
    _dev(dxproj_out, "dxproj_out", xproj.dtype)
    _dev(da_out, "da_out", torch.float32)
    _dev(h0, "h0", xproj.dtype)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(dstate_last, "dstate_last", xproj.dtype)
    _dev(dh0_out, "dh0_out", xproj.dtype)
    B, T, G, d_h = xproj.shape
    S = STATE[cell]
    if G != GATES[cell] or a.shape != (G, d_h) or da_out.shape != (G, d_h):
        raise ValueError(f"shape mismatch: xproj {tuple(xproj.shape)} a {tuple(a.shape)} da {tuple(da_out.shape)}")
    if states.shape != (B, T, S, d_h) or dH.shape != (B, T, d_h) or dxproj_out.shape != xproj.shape:
        raise ValueError(f"shape mismatch: states {tuple(states.shape)} dH {tuple(dH.shape)} "
                         f"dxproj {tuple(dxproj_out.shape)}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    rows = B if cu_seqlens is None else n_seqs
    for t, name in ((h0, "h0"), (dstate_last, "dstate_last"), (dh0_out, "dh0_out")):
        if t is not None and t.shape != (rows, S, d_h):
            raise ValueError(f"{name} must be {(rows, S, d_h)}, got {tuple(t.shape)}")
    _error_word(error_out)
    p = make_params(cell, xproj.dtype, B, T, d_h, n_seqs=n_seqs, a=a, workspace=workspace, stream=stream,
                    error_out=error_out)
    _check(lib().prn_newton_backward(_ptr(xproj), ctypes.byref(p), _ptr(h0), _ptr(cu_seqlens), _ptr(states),
                                     _ptr(dH), _ptr(dstate_last), _ptr(dxproj_out), _ptr(da_out), _ptr(dh0_out)))


def prn_decode_step(x, W, bias, a, state_out, *, cell: str, state_in=None, h_out=None, stream=None) -> None:
    """One T = 1 step for B slots: x (B, d_in), W (G*d_h, d_in), bias (G*d_h) fp32 or None,
    state_in / state_out (B, S, d_h) (distinct buffers), h_out (B, d_h) or None."""
    _dev(x, "x")
    _dev(W, "W", x.dtype)
    _dev(bias, "bias", torch.float32)
    _dev(a, "a", torch.float32)
    _dev(state_out, "state_out", x.dtype)
    _dev(state_in, "state_in", x.dtype)
    _dev(h_out, "h_out", x.dtype)
    Bn, d_in = x.shape
    G, S = GATES[cell], STATE[cell]
    d_h = W.shape[0] // G
    if W.shape != (G * d_h, d_in) or a.shape != (G, d_h) or state_out.shape != (Bn, S, d_h):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)} W {tuple(W.shape)} state_out {tuple(state_out.shape)}")
    if state_in is not None and state_in.shape != (Bn, S, d_h):
        raise ValueError("state_in must match state_out")
    if h_out is not None and h_out.shape != (Bn, d_h):
        raise ValueError("h_out must be (B, d_h)")
    p = make_params(cell, x.dtype, Bn, 1, d_h, d_in=d_in, a=a, stream=stream)
    _check(lib().prn_decode_step(_ptr(x), _ptr(W), _ptr(bias), ctypes.byref(p), _ptr(state_in), _ptr(state_out),
                                 _ptr(h_out)))


def _head_common(xproj, A, H_out, h0, state_last_out, d_head):
    _dev(xproj, "xproj")
    if xproj.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported storage dtype {xproj.dtype}")
    _dev(A, "A", torch.float32)
    for t, n in ((H_out, "H_out"), (h0, "h0"), (state_last_out, "state_last_out")):
        _dev(t, n, xproj.dtype)
    Bn, T, G, d_h = xproj.shape
    if G != 3 or d_h % d_head or A.shape != (3, d_h // d_head, d_head, d_head) or H_out.shape != (Bn, T, d_h):
        raise ValueError(f"shape mismatch: xproj {tuple(xproj.shape)} A {tuple(A.shape)} H_out {tuple(H_out.shape)}")
    for t, n in ((h0, "h0"), (state_last_out, "state_last_out")):
        if t is not None and t.shape != (Bn, d_h):
            raise ValueError(f"{n} must be (B, d_h)")
    return Bn, T, d_h


def prn_head_workspace_bytes(B: int, T: int, d_h: int, K: int, d_head: int = 16, dtype=torch.float32) -> int:
    p = make_params("gru", dtype, B, T, d_h)
    n = int(lib().prn_head_workspace_bytes(ctypes.byref(p), d_head, K))
    if n == 0 and T > 0 and prn_last_error():
        raise PrnError(PRN_ERR_INVALID_ARG, prn_last_error())
    return n


def prn_head_newton_forward(xproj, A, K: int, H_out, *, d_head: int = 16, h0=None, residual_out=None,
                            state_last_out=None, workspace=None, stream=None) -> None:
    """Head-mix GRU Newton forward: xproj (B,T,3,d_h) and H_out, h0, state_last_out in the storage dtype
    (fp32 or bf16), A (3, d_h/d_head, d_head, d_head) fp32."""
    Bn, T, d_h = _head_common(xproj, A, H_out, h0, state_last_out, d_head)
    _dev(residual_out, "residual_out", torch.float32)
    p = make_params("gru", xproj.dtype, Bn, T, d_h, state_last_out=state_last_out, workspace=workspace,
                    stream=stream)
    _check(lib().prn_head_newton_forward(_ptr(xproj), ctypes.byref(p), _ptr(A), d_head, _ptr(h0), int(K),
                                         _ptr(H_out), _ptr(residual_out)))


def prn_head_sequential_forward(xproj, A, H_out, *, d_head: int = 16, h0=None, state_last_out=None,
                                stream=None) -> None:
    Bn, T, d_h = _head_common(xproj, A, H_out, h0, state_last_out, d_head)
    p = make_params("gru", xproj.dtype, Bn, T, d_h, state_last_out=state_last_out, stream=stream)
    _check(lib().prn_head_sequential_forward(_ptr(xproj), ctypes.byref(p), _ptr(A), d_head, _ptr(h0), _ptr(H_out)))
