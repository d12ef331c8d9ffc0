"""Caller-facing helpers over the C ABI: allocation, contiguity, K schedules,
the residual gate and the agreement check.

Contract points from the pararnn-torch pages that live here:
  * shapes/layout page: fused paths copy strided views to a contiguous
    layout first (correct results, more traffic); ragged packs are x of
    batch 1 and length N plus cu_seqlens of length S+1, int32 or int64,
    validated before use; an unsupported pinned combination raises rather
    than silently running something else.
  * FAQs, "How many Newton iterations should I use?": K pinned, or looked
    up in a per-T table.
  * Numerics contract, "Two thresholds" / "1. Runtime": after K steps,
    max|F(H)| above residual_fail (1.0) raises NewtonDivergenceError; above
    the warn band a newton_residual_high warning is issued.
  * Numerics contract, "3. Opt-in oracle": verify_agreement runs Newton and
    the sequential unroll on one batch and compares them (max-abs, tau).
"""
from __future__ import annotations

import dataclasses
import warnings

import torch

from . import binding as B_

RESIDUAL_FAIL = 1.0
# warn band: 1e-3 for fp32 storage; bf16 storage rounds every stored state
# to 8 significant bits, which alone leaves |F| near 2^-9 max|h|.
RESIDUAL_WARN = {torch.float32: 1e-3, torch.bfloat16: 2e-2}
# agreement tau: 1e-4 in fp32 (FAQs); a wider band for bf16 storage
AGREEMENT_ATOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


class NewtonDivergenceError(RuntimeError):
    """max|F(H)| after K Newton steps exceeded residual_fail."""


class AgreementError(AssertionError):
    """Newton and the sequential unroll disagree by more than tau."""


class LookbackTimeoutError(RuntimeError):
    """A kernel's wait for a preceding chunk's record gave up (after about
    65 ms of polling, e.g. with the GPU starved by other work); the results of
    that call are NaN from the chunk on.  Raised instead of returning them."""


def _status_buffer(K: int, device):
    """One zeroed int32 buffer holding the K + 1 residual slots (viewed as
    fp32) and the library's error word after them: one host copy reads both."""
    buf = torch.zeros(K + 2, dtype=torch.int32, device=device)
    return buf, buf[:K + 1].view(torch.float32), buf[K + 1:]


def _read_status(buf, what: str) -> list:
    """Copy the residuals and the error word to the host (the forward's one
    sync); raise LookbackTimeoutError if the error word is set."""
    host = buf.cpu()
    _check_error_word(int(host[-1]), what)
    return host[:-1].view(torch.float32).tolist()


def _check_error_word(err: int, what: str) -> None:
    if err & B_.PRN_FAULT_LOOKBACK:
        raise LookbackTimeoutError(f"{what}: a wait for a preceding chunk's record timed out; the results are "
                                   "invalid (NaN)")


@dataclasses.dataclass
class AgreementReport:
    ok: bool
    max_abs: float
    atol: float
    K: int
    residuals: list
    device: str
    dtype: str

    def to_dict(self) -> dict:
        return dataclasses.asdict(self)


def resolve_k(T: int, table: dict) -> int:
    """K for length T from {T_key: K}: the entry with the smallest key >= T,
    else the largest key's entry."""
    keys = sorted(int(k) for k in table)
    if not keys:
        raise ValueError("empty K table")
    for k in keys:
        if T <= k:
            return int(table[k])
    return int(table[keys[-1]])


def validate_cu_seqlens(cu_seqlens, N: int, device=None) -> torch.Tensor:
    """Check ragged offsets on the host; return them as a contiguous int32 device tensor."""
    cu = torch.as_tensor(cu_seqlens)
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
    if cu.dtype not in (torch.int32, torch.int64):
        raise TypeError(f"cu_seqlens must be int32 or int64, got {cu.dtype}")
    host = cu.detach().cpu().to(torch.int64)
    if int(host.max()) >= 2 ** 31:
        raise ValueError("cu_seqlens values must fit in int32")
    B_.prn_validate_cu_seqlens(host.to(torch.int32), N)
    dev = device if device is not None else (cu.device if cu.device.type == "cuda" else "cuda")
    return host.to(torch.int32).to(dev).contiguous()


def _contig(t):
    return None if t is None else t.contiguous()


def input_proj(x, W, bias=None, *, cell: str) -> torch.Tensor:
    x, W = x.contiguous(), W.contiguous()
    bias = None if bias is None else bias.to(torch.float32).contiguous()
    G = B_.GATES[cell]
    Bn, T, _ = x.shape
    out = torch.empty((Bn, T, G, W.shape[0] // G), dtype=x.dtype, device=x.device)
    B_.prn_input_proj(x, W, bias, out, cell=cell)
    return out


def workspace_for(cell, xproj, K, n_seqs=0) -> torch.Tensor:
    Bn, T, _, d_h = xproj.shape
    n = B_.prn_workspace_bytes(cell, xproj.dtype, Bn, T, d_h, K, n_seqs=n_seqs)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=xproj.device)


def gate_residual(residuals, dtype, residual_fail=RESIDUAL_FAIL, residual_warn=None) -> None:
    """Apply the runtime echelon of the numerics contract to r_K (host values)."""
    rK = float(residuals[-1])
    if not (rK <= residual_fail):   # also catches NaN / Inf
        raise NewtonDivergenceError(
            f"max|F(H)| = {rK:.3e} after K = {len(residuals) - 1} Newton steps exceeds residual_fail = "
            f"{residual_fail}; skip the optimizer step on this batch")
    warn = RESIDUAL_WARN.get(dtype, 1e-3) if residual_warn is None else residual_warn
    if rK > warn:
        warnings.warn(f"newton_residual_high: max|F(H)| = {rK:.3e} > {warn:.1e}", RuntimeWarning, stacklevel=3)


def _resolve_depth(K, k_table, T: int, cell: str) -> int:
    if K is None and k_table is None:
        # max_iters=None: the measured K*(T) envelope of this cell (FAQs,
        # "How many Newton iterations should I use?")
        from .kstar import load_table
        k_table = load_table(cell)
    if k_table is not None and K is None:
        K = resolve_k(T, k_table)
    if K is None or int(K) < 1:
        raise ValueError("K must be >= 1")
    return int(K)


def newton_forward(xproj, a, K=3, *, cell: str, h0=None, cu_seqlens=None, k_table=None,
                   residual_fail=RESIDUAL_FAIL, residual_warn=None, gate=True, return_state=False):
    """Parallel Newton forward.  Returns (H (B,T,d_h), residuals [r_0..r_K] on
    the host[, final states]).  K may be None: then it comes from k_table, or
    from the cell's measured K*(T) table (nonlinear_rnn_amd/kstar_table.json)."""
    xproj = xproj.contiguous()
    a = a.to(torch.float32).contiguous()
    Bn, T, _, d_h = xproj.shape
    K = _resolve_depth(K, k_table, T, cell)
    cu = None if cu_seqlens is None else validate_cu_seqlens(cu_seqlens, T, xproj.device)
    n_seqs = 0 if cu is None else cu.numel() - 1
    rows = Bn if cu is None else n_seqs
    H = torch.empty((Bn, T, d_h), dtype=xproj.dtype, device=xproj.device)
    buf, res, err = _status_buffer(K, xproj.device)
    st = (torch.empty((rows, B_.STATE[cell], d_h), dtype=xproj.dtype, device=xproj.device)
          if return_state else None)
    ws = workspace_for(cell, xproj, K, n_seqs)
    B_.prn_newton_forward(xproj, a, K, H, cell=cell, h0=_contig(h0), cu_seqlens=cu, residual_out=res,
                          state_last_out=st, workspace=ws, error_out=err)
    residuals = _read_status(buf, "prn_newton_forward")   # the one host sync of a forward
    if gate:
        gate_residual(residuals, xproj.dtype, residual_fail, residual_warn)
    return (H, residuals, st) if return_state else (H, residuals)


def sequential_forward(xproj, a, *, cell: str, h0=None, cu_seqlens=None, return_state=False):
    xproj = xproj.contiguous()
    a = a.to(torch.float32).contiguous()
    Bn, T, _, d_h = xproj.shape
    cu = None if cu_seqlens is None else validate_cu_seqlens(cu_seqlens, T, xproj.device)
    rows = Bn if cu is None else cu.numel() - 1
    H = torch.empty((Bn, T, d_h), dtype=xproj.dtype, device=xproj.device)
    st = (torch.empty((rows, B_.STATE[cell], d_h), dtype=xproj.dtype, device=xproj.device)
          if return_state else None)
    B_.prn_sequential_forward(xproj, a, H, cell=cell, h0=_contig(h0), cu_seqlens=cu, state_last_out=st)
    return (H, st) if return_state else H


def forward(x, W, bias, a, K=3, *, cell: str, fused: bool = False, **kw):
    """Projection + Newton: the train-mode forward of one diagonal layer.
    fused=True runs both in one kernel (each Newton workgroup projects its own
    chunk; the same projected inputs, so the same results wherever both take
    the same chunk length)."""
    if fused:
        return forward_fused(x, W, bias, a, K, cell=cell, **kw)
    return newton_forward(input_proj(x, W, bias, cell=cell), a, K, cell=cell, **kw)


def forward_fused(x, W, bias, a, K=3, *, cell: str, h0=None, cu_seqlens=None, k_table=None,
                  residual_fail=RESIDUAL_FAIL, residual_warn=None, gate=True, return_state=False,
                  return_xproj=False):
    """prn_newton_forward_fused behind the same contract as newton_forward.
    Returns (H, residuals[, final states][, xproj])."""
    x, W = x.contiguous(), W.contiguous()
    bias = None if bias is None else bias.to(torch.float32).contiguous()
    a = a.to(torch.float32).contiguous()
    Bn, T, _ = x.shape
    d_h = W.shape[0] // B_.GATES[cell]
    K = _resolve_depth(K, k_table, T, cell)
    cu = None if cu_seqlens is None else validate_cu_seqlens(cu_seqlens, T, x.device)
    n_seqs = 0 if cu is None else cu.numel() - 1
    rows = Bn if cu is None else n_seqs
    H = torch.empty((Bn, T, d_h), dtype=x.dtype, device=x.device)
    buf, res, err = _status_buffer(K, x.device)
    st = (torch.empty((rows, B_.STATE[cell], d_h), dtype=x.dtype, device=x.device) if return_state else None)
    xp = (torch.empty((Bn, T, B_.GATES[cell], d_h), dtype=x.dtype, device=x.device) if return_xproj else None)
    n = B_.prn_workspace_bytes(cell, x.dtype, Bn, T, d_h, K, n_seqs=n_seqs)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    B_.prn_newton_forward_fused(x, W, bias, a, K, H, cell=cell, h0=_contig(h0), cu_seqlens=cu, residual_out=res,
                                xproj_out=xp, state_last_out=st, workspace=ws, error_out=err)
    residuals = _read_status(buf, "prn_newton_forward_fused")   # the one host sync of a forward
    if gate:
        gate_residual(residuals, x.dtype, residual_fail, residual_warn)
    out = (H, residuals)
    if return_state:
        out += (st,)
    if return_xproj:
        out += (xp,)
    return out


def verify_agreement(xproj, a, K=3, *, cell: str, h0=None, cu_seqlens=None, atol=None,
                     raise_on_fail=False) -> AgreementReport:
    """Run Newton and the sequential unroll on one batch; compare max-abs to tau."""
    H_n, res = newton_forward(xproj, a, K, cell=cell, h0=h0, cu_seqlens=cu_seqlens, gate=False)
    H_s = sequential_forward(xproj, a, cell=cell, h0=h0, cu_seqlens=cu_seqlens)
    atol = AGREEMENT_ATOL.get(xproj.dtype, 1e-4) if atol is None else atol
    m = float((H_n.float() - H_s.float()).abs().max()) if H_n.numel() else 0.0
    rep = AgreementReport(ok=bool(m <= atol), max_abs=m, atol=atol, K=K, residuals=res,
                          device=str(xproj.device), dtype=str(xproj.dtype))
    if raise_on_fail and not rep.ok:
        raise AgreementError(f"Newton vs sequential max_abs {m:.3e} > tau {atol:.1e}: {rep.to_dict()}")
    return rep


# ------------------------------------------------------------------ training surface ---
# The train-mode forward + backward of one diagonal layer (FAQs, "train() vs
# eval()"; shapes/layout page, the train forward+backward surface): the
# Newton forward keeps its trajectory (states_out) and the backward is
# prn_newton_backward at that trajectory.  With recompute=True (the pages'
# NewtonConfig(recompute=True) for long sequences) the forward keeps only
# its inputs and the backward runs the forward again to rebuild the
# trajectory: (B, T, S, d_h) less memory held between the passes, one more
# forward in the backward.  The projection's gradients (input_proj_apply)
# come from prn_input_proj_backward.

def _forward_states(xproj, a, h0, cell, K, cu, picard_iters, with_states):
    """Newton forward keeping the trajectory; returns (H, states, residuals on
    the host) after the forward's one host sync."""
    Bn, T, G, d_h = xproj.shape
    n_seqs = 0 if cu is None else cu.numel() - 1
    H = torch.empty((Bn, T, d_h), dtype=xproj.dtype, device=xproj.device)
    states = (torch.empty((Bn, T, B_.STATE[cell], d_h), dtype=xproj.dtype, device=xproj.device)
              if with_states else None)
    buf, res, err = _status_buffer(K, xproj.device)
    n = B_.prn_workspace_bytes(cell, xproj.dtype, Bn, T, d_h, K, n_seqs=n_seqs, picard_iters=picard_iters)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=xproj.device)
    B_.prn_newton_forward(xproj, a, K, H, cell=cell, h0=h0, cu_seqlens=cu, residual_out=res,
                          states_out=states, workspace=ws, picard_iters=picard_iters, error_out=err)
    return H, states, _read_status(buf, "prn_newton_forward")


class _NewtonFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xproj, a, h0, cell, K, cu, picard_iters, residual_fail, gate, recompute):
        H, states, ctx.residuals = _forward_states(xproj, a, h0, cell, K, cu, picard_iters, not recompute)
        if gate:
            gate_residual(ctx.residuals, xproj.dtype, residual_fail)
        ctx.cell, ctx.cu, ctx.K, ctx.picard_iters, ctx.recompute = cell, cu, K, picard_iters, recompute
        ctx.save_for_backward(xproj, a, h0 if h0 is not None else torch.empty(0),
                              states if states is not None else torch.empty(0))
        ctx.has_h0 = h0 is not None
        return H

    @staticmethod
    def backward(ctx, dH):
        xproj, a, h0, states = ctx.saved_tensors
        h0 = h0 if ctx.has_h0 else None
        cell, cu = ctx.cell, ctx.cu
        if ctx.recompute:
            _, states, _ = _forward_states(xproj, a, h0, cell, ctx.K, cu, ctx.picard_iters, True)
        Bn, T, G, d_h = xproj.shape
        n_seqs = 0 if cu is None else cu.numel() - 1
        rows = Bn if cu is None else n_seqs
        dxproj = torch.empty_like(xproj)
        da = torch.empty((G, d_h), dtype=torch.float32, device=xproj.device)
        dh0 = (torch.empty((rows, B_.STATE[cell], d_h), dtype=xproj.dtype, device=xproj.device)
               if ctx.needs_input_grad[2] else None)
        n = B_.prn_backward_workspace_bytes(cell, xproj.dtype, Bn, T, d_h, n_seqs=n_seqs)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=xproj.device)
        err = torch.zeros(1, dtype=torch.int32, device=xproj.device)
        B_.prn_newton_backward(xproj, a, states, dH.to(xproj.dtype).contiguous(), dxproj, da, cell=cell, h0=h0,
                               cu_seqlens=cu, dh0_out=dh0, workspace=ws, error_out=err)
        # the backward's one host sync: a timed-out wait must not hand NaN gradients to the optimizer
        _check_error_word(int(err.item()), "prn_newton_backward")
        return dxproj, da, dh0, None, None, None, None, None, None, None


def newton_apply(xproj, a, K=None, *, cell: str, h0=None, cu_seqlens=None, picard_iters: int = 0,
                 residual_fail=RESIDUAL_FAIL, gate=True, recompute: bool = False):
    """Differentiable Newton forward: H (B,T,d_h); gradients reach xproj, a
    and h0 through the backward pass.  K = None resolves the measured K*(T).
    recompute=True keeps no trajectory between the passes and rebuilds it in
    the backward (the same kernels on the same inputs, so bitwise the same
    trajectory)."""
    xproj = xproj.contiguous()
    Bn, T, _, _ = xproj.shape
    if K is None:
        from .kstar import load_table
        K = resolve_k(T, load_table(cell))
    cu = None if cu_seqlens is None else validate_cu_seqlens(cu_seqlens, T, xproj.device)
    # a of another dtype (a bf16 parameter) is cast here, so that autograd
    # casts its fp32 gradient back
    return _NewtonFunction.apply(xproj, a.to(torch.float32).contiguous(), _contig(h0), cell, int(K), cu,
                                 int(picard_iters), residual_fail, gate, bool(recompute))


class _ProjFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, W, bias, cell):
        ctx.save_for_backward(x, W)
        ctx.has_bias = bias is not None
        ctx.cell = cell
        return input_proj(x, W, bias, cell=cell)

    @staticmethod
    def backward(ctx, dxp):
        x, W = ctx.saved_tensors
        Bn, T, G, d_h = dxp.shape
        dxp = dxp.to(x.dtype).contiguous()
        want_x, want_W, want_b = ctx.needs_input_grad[:3]
        dx = torch.empty_like(x) if want_x else None
        dW = torch.empty_like(W) if want_W else None
        dbias = torch.empty(G * d_h, dtype=torch.float32, device=x.device) if (want_b and ctx.has_bias) else None
        n = B_.prn_input_proj_backward_workspace_bytes(ctx.cell, x.dtype, Bn, T, x.shape[-1], d_h)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
        B_.prn_input_proj_backward(dxp, x, W, cell=ctx.cell, dx_out=dx, dW_out=dW, dbias_out=dbias, workspace=ws)
        return dx, dW, dbias, None


def input_proj_apply(x, W, bias=None, *, cell: str):
    """Differentiable projection: xproj = x W^T + bias on the matrix cores;
    its backward (dx, dW, dbias) is prn_input_proj_backward, also on the
    matrix cores, with fixed summation orders."""
    return _ProjFunction.apply(x.contiguous(), W.contiguous(),
                               None if bias is None else bias.to(torch.float32).contiguous(), cell)
