#!/usr/bin/env python3
"""Throughput of the parallel-Newton diagonal GRU/LSTM forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the input projection (prn_input_proj) followed by
the K-iteration Newton solve (prn_newton_forward).  Prints ONE JSON line.

Default workload: the diagonal LSTM, B=2, T=131072, d_in=d_h=256, fp32,
K=2 (the long-sequence configuration the bandwidth target is stated for).
The other workloads (--workload) are parity cases; they can be timed too.

Timing: W untimed warm-up steps, then K timed steps bracketed by device
synchronisation; HIP events around every library call on the stream the
kernels run on give per-call durations.  Beside the step: the agreement of
the result with the GPU unroll at the bench's K, the same forward at the
measured K*(T), the backward, the fused forward, the decode step and the
head-mix GRU.  CPU baselines: the oracle (NumPy, float64, one thread) on a
bounded sample, and the unroll in plain C (float64, OpenMP, all host
threads) on the whole workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Newton-forward tokens/sec at K=3 (B*T/s) + achieved HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
# fp32 products run on the bf16 matrix cores as six products of exact bf16
# splits (csrc/bf16split.h): the executed matrix-core work per fp32 flop
F32_SPLIT_PRODUCTS = 6


def mfma_roofline(dtype: str, flops: float, ms: float, **extra) -> dict:
    """Roofline of a matrix-core contraction: algorithmic flops over time
    against the peak of the storage dtype's own matrix instruction; an fp32
    contraction also states the bf16 matrix-core work it executes (six term
    products per fp32 product) against the bf16 peak, the unit that bounds it."""
    ach = flops / (ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": ach, "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
         "frac": ach / MFMA_PEAK_TFLOPS[dtype], "algorithmic_flops": flops}
    if dtype == "f32":
        ex = F32_SPLIT_PRODUCTS * flops
        r["matrix_core"] = {"instruction": "v_mfma_f32_32x32x16_bf16 on exact bf16 splits",
                            "executed_flops": ex, "achieved": ex / (ms * 1e-3) / 1e12,
                            "peak": MFMA_PEAK_TFLOPS["bf16"],
                            "frac": ex / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"]}
    r.update(extra)
    return r


def algorithmic_newton_bytes(w) -> float:
    """Bytes the K-pass Newton method must move per forward: per channel-token,
    read xproj once per iteration (K*G), read the previous iterate and write
    each new one for iterations 2..K and 1..K-1 (2(K-1)S), write h (1)."""
    elt = 4 if w.dtype == "f32" else 2
    per = w.K * w.G + 2 * (w.K - 1) * w.S + 1
    return float(w.tokens) * w.d_h * per * elt


def algorithmic_backward_bytes(w) -> float:
    """Bytes the backward must move per forward: per channel-token, read the
    projected inputs (G), the previous state (S) and dL/dh (1) once, and
    write dL/dxproj (G)."""
    elt = 4 if w.dtype == "f32" else 2
    return float(w.tokens) * w.d_h * (2 * w.G + w.S + 1) * elt


# the sources each profiled kernel is built and launched from
KERNEL_SOURCES = {
    "k_newton_sp": ["prn_device.h", "bf16split.h", "fused_proj.h", "newton_kernels.h", "newton_sp.h", "prn_api.hip"],
    "k_bw_sp": ["prn_device.h", "bf16split.h", "fused_proj.h", "newton_kernels.h", "newton_sp.h", "backward.h", "prn_api.hip"],
    "k_newton_sp_fused": ["prn_device.h", "bf16split.h", "fused_proj.h", "newton_kernels.h", "newton_sp.h", "prn_api.hip"],
    "k_proj": ["proj.h", "bf16split.h", "proj.hip"],
    "k_hm": ["prn_device.h", "headmix.h", "prn_api.hip"],
}


def proj_tiles(w) -> str:
    """The tile shape prn_input_proj uses for this workload: 256 x 256 once there
    are at least 768 such tiles, else 128 x 128."""
    tiles = -(-w.B * w.T // 256) * -(-w.G * w.d_h // 256)
    return "256x256" if tiles >= 768 else "128x128"


def kernel_source_hash(kernel: str) -> str:
    """Hash of the HIP sources a kernel is built from; a profile taken from other sources is stale."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        with open(os.path.join(ROOT, "nonlinear_rnn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_fields(kernel: str, workload: str) -> dict:
    """Fields of the committed rocprofv3 summary of this kernel and workload,
    or {} if there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.txt")
    if not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_hash") != kernel_source_hash(kernel):
        return {}
    return fields


def _field(fields: dict, key: str):
    try:
        return float(fields[key].split()[0])
    except (KeyError, ValueError, IndexError):
        return None


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload (FETCH_SIZE + WRITE_SIZE, each scaled by what a
    512 MiB copy reads), or None if there is none or the kernels changed since."""
    return _field(profile_fields(kernel, workload), "traffic_bytes_per_launch")


VALU_F32_PEAK_TFLOPS = 157.3


def headmix_flops(Bn: int, T: int, d_h: int, K: int, d: int = 16) -> float:
    """Arithmetic of the head-mix Newton forward per (step, head), counted as
    2 flops per multiply-add: each iteration's chunk reduce applies J to the
    running 16 x 16 map (three block products, 3 * 2 d^3) and to its vector
    (three block matrix-vector products), and evaluates the gates (three
    more); the fix-up evaluates the gates and applies J to a vector again;
    the final residual pass evaluates the gates once more."""
    mv = 2 * d * d
    per_iter = 3 * 2 * d ** 3 + 3 * mv + 3 * mv + 3 * mv + 3 * mv
    return float(Bn) * T * (d_h // d) * (K * per_iter + 3 * mv)


def bench_headmix(torch, B, dev, steps: int, warmup: int, Bn: int = 8, T: int = 4096) -> dict:
    """Head-mix GRU (16 x 16 blocks, 16 heads, d_h = 256), K = 3, at B x T:
    the Newton forward and the unroll, timed with HIP events on the stream."""
    d_h, K = 256, 3
    g = torch.Generator(device=dev).manual_seed(4)
    xp = torch.randn((Bn, T, 3, d_h), generator=g, device=dev)
    A = (torch.rand((3, d_h // 16, 16, 16), generator=g, device=dev) - 0.5) / 4.0
    H = torch.empty((Bn, T, d_h), device=dev)
    res = torch.zeros(K + 1, device=dev)
    ws = torch.empty(B.prn_head_workspace_bytes(Bn, T, d_h, K), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in ev])

    t_n = timed(lambda: B.prn_head_newton_forward(xp, A, K, H, residual_out=res, workspace=ws, stream=stream))
    Hs = torch.empty_like(H)
    t_s = timed(lambda: B.prn_head_sequential_forward(xp, A, Hs, stream=stream))
    ms = float(t_n.mean())
    fl = headmix_flops(Bn, T, d_h, K)
    return {"config": {"cell": "head-mix GRU", "B": Bn, "T": T, "d_h": d_h, "d_head": 16, "K": K},
            "kernels": "k_hm_pass (reduce, fix-up) + k_hm_scan or k_hm_group, k_hm_scan, k_hm_expand per iteration (prn_head_newton_forward)",
            "newton_ms_mean": ms, "newton_ms_min": float(t_n.min()), "tokens_per_s": Bn * T / (ms * 1e-3),
            "sequential_ms_mean": float(t_s.mean()), "speedup_vs_unroll": float(t_s.mean()) / ms,
            "max_abs_vs_unroll": float((H - Hs).abs().max()), "residual_K": float(res[-1]),
            "roofline": {"bound": "alu", "achieved": fl / (ms * 1e-3) / 1e12, "peak": VALU_F32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": fl / (ms * 1e-3) / 1e12 / VALU_F32_PEAK_TFLOPS,
                         "traffic": None, "algorithmic_flops": fl}}


def proj_flops(w) -> float:
    return 2.0 * w.tokens * w.G * w.d_h * w.d_in


def cpu_baseline(w, budget_s: float = 20.0) -> dict:
    """The oracle as it stands (projection + Newton, float64 NumPy) on a
    bounded sample of the workload: one row, its first T_s steps, all
    channels, one thread, repeated until about budget_s seconds of CPU work."""
    from threadpoolctl import threadpool_limits

    from oracle import newton as onewton
    from oracle import proj as oproj
    from oracle import rounding as oround
    from workloads import make_inputs

    T_s = min(w.T, 32768)
    ws = w.scaled(B=1, T=T_s, n_seqs=0)
    inp = make_inputs(ws, seed=0)
    cu = None
    if w.n_seqs:
        full = make_inputs(w, seed=0)["cu_seqlens"]
        cu = np.concatenate([full[full < T_s], [T_s]]).astype(np.int64)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            xp = oproj.input_proj(oround.load(inp["x"], w.dtype), oround.load(inp["W"], w.dtype),
                                  inp["bias"].astype(np.float64), w.G)
            xp = oround.store(xp, w.dtype)
            onewton.newton(w.cell, xp, inp["a"].astype(np.float64), w.K, cu_seqlens=cu, dtype=w.dtype)
            reps += 1
            el = time.perf_counter() - t0
            if el > budget_s:
                break
        # the oracle's sequential unroll (the definition Newton approximates) on the same sample
        t1 = time.perf_counter()
        onewton.sequential(w.cell, xp, inp["a"].astype(np.float64), cu_seqlens=cu)
        el_seq = time.perf_counter() - t1
    tok = reps * ws.tokens
    return {"value": tok / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x (B=1, T={T_s}, all {w.d_h} channels, K={w.K}) of {w.name}: "
                      f"numpy float64 projection + Newton, 1 thread, {el:.1f} s",
            "sequential_unroll": {"value": ws.tokens / el_seq, "unit": "tokens/s", "cores": 1,
                                  "sample": f"1 x the same sample, the oracle's sequential unroll "
                                            f"(numpy float64), 1 thread, {el_seq:.1f} s"}}


def cpu_openmp_unroll(w, xproj_host, inp, cu) -> dict:
    """The multi-core CPU baseline: the sequential unroll in plain C (float64,
    OpenMP over blocks of channels; oracle/c/unroll.c) on the whole workload,
    all host threads, from the same stored projected inputs the GPU reads.
    Cross-checked against the NumPy oracle's unroll on a sample (row 0, 8
    channels, the first 4096 steps)."""
    from oracle import newton as onewton
    from oracle import unroll_c

    threads = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    a64 = inp["a"].astype(np.float64)
    unroll_c.unroll(w.cell, xproj_host[:1, :64], a64, cu_seqlens=None)   # load the library, start the threads
    t0 = time.perf_counter()
    h = unroll_c.unroll(w.cell, xproj_host, a64, cu_seqlens=cu)
    el = time.perf_counter() - t0
    Ts = min(w.T, 4096)
    cu_s = None if cu is None else np.concatenate([cu[cu < Ts], [Ts]]).astype(np.int64)
    ref, _ = onewton.sequential(w.cell, xproj_host[:1, :Ts, :, :8].astype(np.float64), a64[:, :8], cu_seqlens=cu_s)
    err = float(np.abs(h[:1, :Ts, :8] - ref[..., -1, :]).max())
    return {"value": w.tokens / el, "unit": "tokens/s", "cores": threads, "kind": "plain C unroll",
            "sample": f"the whole workload ({w.tokens} tokens x {w.d_h} channels), sequential unroll in C, "
                      f"float64, OpenMP over channel blocks, {threads} threads, {el:.2f} s",
            "max_abs_vs_numpy_oracle_sample": err}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lstm_t131k")
    ap.add_argument("--K", type=int, default=None, help="override the workload's Newton depth")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-decode", action="store_true", help="skip timing the T = 1 decode step")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip timing the fused forward (projection inside the Newton kernel)")
    ap.add_argument("--no-headmix", action="store_true", help="skip timing the head-mix GRU")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-kstar", action="store_true", help="skip the leg at the measured K*(T)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 512 MiB device-to-device copy first (a known-size reference for byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        return 2

    import torch

    import nonlinear_rnn_amd as prn
    from nonlinear_rnn_amd import binding as B
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if args.K:
        w = w.scaled(K=args.K)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    print(f"[bench] workload {w}", file=sys.stderr, flush=True)

    inp = make_inputs(w, seed=0)

    def up(arr):
        if w.dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(arr).to(dev)

    x, W = up(inp["x"]), up(inp["W"])
    bias = torch.from_numpy(inp["bias"]).to(dev)
    a = torch.from_numpy(inp["a"]).to(dev)
    cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(dev)
    n_seqs = 0 if cu is None else cu.numel() - 1
    xproj = torch.empty((w.B, w.T, w.G, w.d_h), dtype=dt, device=dev)
    H = torch.empty((w.B, w.T, w.d_h), dtype=dt, device=dev)
    res = torch.zeros(w.K + 1, dtype=torch.float32, device=dev)
    ws_n = B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, w.K, n_seqs=n_seqs)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        B.prn_input_proj(x, W, bias, xproj, cell=w.cell, stream=stream)
        if ev:
            ev[1].record(stream)
        B.prn_newton_forward(xproj, a, w.K, H, cell=w.cell, cu_seqlens=cu, residual_out=res, workspace=ws,
                             stream=stream)
        if ev:
            ev[2].record(stream)

    if args.calib_copy:
        src = torch.empty(128 * 2 ** 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 536870912 bytes read, 536870912 bytes written", file=sys.stderr, flush=True)
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done ({args.warmup} steps)", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_proj = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_newt = np.array([e[1].elapsed_time(e[2]) for e in evs])
    t_step = np.array([e[0].elapsed_time(e[2]) for e in evs])
    print(f"[bench] timed {args.steps} steps: wall {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # the same steps with the 256 MB last-level cache (MALL) flushed before each one by writing
    # a 1 GiB buffer, so that a working set that fits the cache is read from HBM again
    flush = torch.empty(2 ** 28, dtype=torch.float32, device=dev)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.zero_()
        step(fev[i])
    torch.cuda.synchronize()
    del flush
    t_newt_fl = np.array([e[1].elapsed_time(e[2]) for e in fev])
    t_proj_fl = np.array([e[0].elapsed_time(e[1]) for e in fev])

    backward = None
    if not args.no_backward:
        # the backward pass at the trajectory of one forward (states_out), timed on its own
        states = torch.empty((w.B, w.T, w.S, w.d_h), dtype=dt, device=dev)
        B.prn_newton_forward(xproj, a, w.K, H, cell=w.cell, cu_seqlens=cu, residual_out=res, workspace=ws,
                             states_out=states, stream=stream)
        gen = torch.Generator(device=dev).manual_seed(1)
        dH = torch.randn((w.B, w.T, w.d_h), generator=gen, device=dev).to(dt)
        dxp = torch.empty_like(xproj)
        da = torch.empty((w.G, w.d_h), dtype=torch.float32, device=dev)
        bws = torch.empty(max(B.prn_backward_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, n_seqs=n_seqs), 1),
                          dtype=torch.uint8, device=dev)

        def bstep():
            B.prn_newton_backward(xproj, a, states, dH, dxp, da, cell=w.cell, cu_seqlens=cu, workspace=bws,
                                  stream=stream)
        for _ in range(args.warmup):
            bstep()
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            bev[i][0].record(stream)
            bstep()
            bev[i][1].record(stream)
        torch.cuda.synchronize()
        t_bw = np.array([e[0].elapsed_time(e[1]) for e in bev])
        bw_ms = float(t_bw.mean())
        bw_bytes = algorithmic_backward_bytes(w)
        backward = {"kernels": "k_bw_sp + k_bw_da_partial + k_bw_da_reduce (prn_newton_backward)",
                    "ms_mean": bw_ms, "ms_min": float(t_bw.min()), "tokens_per_s": w.tokens / (bw_ms * 1e-3),
                    "roofline": {"bound": "hbm", "achieved": bw_bytes / (bw_ms * 1e-3) / 1e9,
                                 "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                 "frac": bw_bytes / (bw_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                 "traffic": profiled_traffic("k_bw_sp", w.name), "algorithmic_bytes": bw_bytes}}
        # the projection's gradients at the same dL/dxproj: dx = g W, dW = g^T x, dbias (the rest of the
        # training step's backward, prn_input_proj_backward)
        dxi = torch.empty_like(x)
        dWi = torch.empty_like(W)
        dbi = torch.empty(w.G * w.d_h, dtype=torch.float32, device=dev)
        pws = torch.empty(max(B.prn_input_proj_backward_workspace_bytes(w.cell, dt, w.B, w.T, w.d_in, w.d_h), 1),
                          dtype=torch.uint8, device=dev)

        def pstep():
            B.prn_input_proj_backward(dxp, x, W, cell=w.cell, dx_out=dxi, dW_out=dWi, dbias_out=dbi, workspace=pws,
                                      stream=stream)
        for _ in range(args.warmup):
            pstep()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            pev[i][0].record(stream)
            pstep()
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        t_pb = np.array([e[0].elapsed_time(e[1]) for e in pev])
        pb_ms = float(t_pb.mean())
        pfl = 2.0 * proj_flops(w)   # dx and dW: one projection's worth of products each
        backward["input_proj_backward"] = {
            "kernels": ("W transpose + k_proj (dx); k_proj_tn (fp32) / k_proj_tn_tr (bf16) split-K over tokens, "
                        "operand rows read directly (dW); k_splitk_sum; k_colsum64 + ordered sums (dbias) "
                        "(prn_input_proj_backward)"),
            "ms_mean": pb_ms, "ms_min": float(t_pb.min()), "workspace_bytes": int(pws.numel()),
            "roofline": mfma_roofline(w.dtype, pfl, pb_ms)}
        del dxi, dWi, pws
        print(f"[bench] backward timed ({args.steps} calls)", file=sys.stderr, flush=True)

    fused = None
    if not args.no_fused:
        # the same forward as one kernel: each Newton workgroup projects its own chunk on the matrix cores
        Hf = torch.empty_like(H)
        resf = torch.zeros_like(res)

        def fstep():
            B.prn_newton_forward_fused(x, W, bias, a, w.K, Hf, cell=w.cell, cu_seqlens=cu, residual_out=resf,
                                       workspace=ws, stream=stream)
        for _ in range(args.warmup):
            fstep()
        fev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            fev2[i][0].record(stream)
            fstep()
            fev2[i][1].record(stream)
        torch.cuda.synchronize()
        t_fx = np.array([e[0].elapsed_time(e[1]) for e in fev2])
        fx_ms = float(t_fx.mean())
        ffl = proj_flops(w)
        fused = {"kernel": "k_newton_sp, fused-projection instance (prn_newton_forward_fused)",
                 "ms_mean": fx_ms, "ms_min": float(t_fx.min()), "tokens_per_s": w.tokens / (fx_ms * 1e-3),
                 "speedup_vs_two_calls": float(t_step.mean()) / fx_ms,
                 "max_abs_vs_two_calls": float((Hf.float() - H.float()).abs().max().item()),
                 "residuals": resf.cpu().tolist(),
                 "roofline": mfma_roofline(w.dtype, ffl, fx_ms,
                                           traffic=profiled_traffic("k_newton_sp_fused", w.name))}
        del Hf
        print(f"[bench] fused forward timed ({args.steps} calls)", file=sys.stderr, flush=True)

    decode = None
    if not args.no_decode:
        # the serving step: one token for each of 64 slots per call (projection + cell fused), ping-pong carries
        slots, n_tok = 64, 64
        gen = torch.Generator(device=dev).manual_seed(2)
        xd = torch.randn((n_tok, slots, w.d_in), generator=gen, device=dev).to(dt)
        carry = [torch.zeros((slots, w.S, w.d_h), dtype=dt, device=dev) for _ in range(2)]
        hd = torch.empty((slots, w.d_h), dtype=dt, device=dev)

        def dstep(i):
            B.prn_decode_step(xd[i % n_tok], W, bias, a, carry[(i + 1) % 2], cell=w.cell, state_in=carry[i % 2],
                              h_out=hd, stream=stream)
        for i in range(8):
            dstep(i)
        n_calls = 4 * n_tok
        dev0, dev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        dev0.record(stream)
        for i in range(n_calls):
            dstep(i)
        dev1.record(stream)
        torch.cuda.synchronize()
        us_eager = dev0.elapsed_time(dev1) * 1e3 / n_calls   # includes the Python call per token
        # a serving loop replays captured steps: n_tok steps in one graph, replayed 4 times
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_tok):
                B.prn_decode_step(xd[i], W, bias, a, carry[(i + 1) % 2], cell=w.cell, state_in=carry[i % 2],
                                  h_out=hd)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_tok):
                B.prn_decode_step(xd[i], W, bias, a, carry[(i + 1) % 2], cell=w.cell, state_in=carry[i % 2],
                                  h_out=hd)
        graph.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.current_stream()
        dev0.record(gs)
        for _ in range(4):
            graph.replay()
        dev1.record(gs)
        torch.cuda.synchronize()
        us = dev0.elapsed_time(dev1) * 1e3 / (4 * n_tok)
        elt = 4 if w.dtype == "f32" else 2
        dbytes = elt * (w.G * w.d_h * w.d_in + slots * w.d_in + 2 * slots * w.S * w.d_h + slots * w.d_h) \
            + 4 * 2 * w.G * w.d_h
        decode = {"kernel": "k_decode (prn_decode_step)", "slots": slots, "us_per_step": us,
                  "us_per_step_eager": us_eager,
                  "tokens_per_s": slots / (us * 1e-6),
                  "roofline": {"bound": "hbm", "achieved": dbytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS,
                               "unit": "GB/s", "frac": dbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                               "traffic": None, "algorithmic_bytes": dbytes}}
        print(f"[bench] decode timed ({n_calls} calls)", file=sys.stderr, flush=True)

    headmix = None
    if not args.no_headmix:
        n = max(3, min(args.steps, 10))
        # the GRU workload's shape, and one long sequence (few chains: the regime parallel Newton is for)
        headmix = {"batch": bench_headmix(torch, B, dev, n, 2), "long": bench_headmix(torch, B, dev, n, 2, 1, 32768)}
        print("[bench] head-mix timed", file=sys.stderr, flush=True)

    # agreement with the unroll at the bench's own K (FAQs, "Does parallel Newton match sequential
    # unroll?"; Numerics contract, "Invariant": within tau at the measured K*(T)): the GPU unroll
    # (prn_sequential_forward) on the same projected inputs, every h compared on the host
    B.prn_newton_forward(xproj, a, w.K, H, cell=w.cell, cu_seqlens=cu, residual_out=res, workspace=ws,
                         stream=stream)
    H_seq = torch.empty_like(H)
    B.prn_sequential_forward(xproj, a, H_seq, cell=w.cell, cu_seqlens=cu, stream=stream)
    torch.cuda.synchronize()
    H_seq_host = H_seq.float().cpu().numpy()
    agreement = {"K": w.K, "max_abs_vs_unroll": float(np.abs(H.float().cpu().numpy() - H_seq_host).max()),
                 "tau_f32": 1e-4, "compared": "every h of the workload, Newton at this K vs the GPU unroll"}
    print(f"[bench] agreement at K={w.K}: {agreement['max_abs_vs_unroll']:.3e}", file=sys.stderr, flush=True)

    kstar = None
    if not args.no_kstar:
        # the same forward at the measured K*(T) of this cell (nonlinear_rnn_amd/kstar_table.json):
        # the depth at which it meets tau against the unroll
        from nonlinear_rnn_amd.kstar import load_table
        k_s = prn.resolve_k(w.T if not w.n_seqs else int(np.diff(inp["cu_seqlens"]).max()), load_table(w.cell))
        ws_k = torch.empty(max(B.prn_workspace_bytes(w.cell, dt, w.B, w.T, w.d_h, k_s, n_seqs=n_seqs), 1),
                           dtype=torch.uint8, device=dev)
        res_k = torch.zeros(k_s + 1, dtype=torch.float32, device=dev)
        Hk = torch.empty_like(H)

        def kstep():
            B.prn_newton_forward(xproj, a, k_s, Hk, cell=w.cell, cu_seqlens=cu, residual_out=res_k, workspace=ws_k,
                                 stream=stream)
        for _ in range(args.warmup):
            kstep()
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            kev[i][0].record(stream)
            kstep()
            kev[i][1].record(stream)
        torch.cuda.synchronize()
        t_k = np.array([e[0].elapsed_time(e[1]) for e in kev])
        k_ms = float(t_k.mean())
        wk = w.scaled(K=k_s)
        kb = algorithmic_newton_bytes(wk)
        kstar = {"K": k_s, "kernel": "k_newton_sp (prn_newton_forward)", "newton_ms_mean": k_ms,
                 "newton_ms_min": float(t_k.min()), "newton_tokens_per_s": w.tokens / (k_ms * 1e-3),
                 "step_tokens_per_s": w.tokens / ((k_ms + float(t_proj.mean())) * 1e-3),
                 "residuals": res_k.cpu().tolist(),
                 "max_abs_vs_unroll": float(np.abs(Hk.float().cpu().numpy() - H_seq_host).max()),
                 "roofline": {"bound": "hbm", "achieved": kb / (k_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                              "unit": "GB/s", "frac": kb / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "algorithmic_bytes": kb}}
        del Hk, ws_k
        print(f"[bench] K*={k_s} leg timed: {k_ms:.3f} ms, max|H - unroll| {kstar['max_abs_vs_unroll']:.3e}",
              file=sys.stderr, flush=True)
    del H_seq

    residuals = res.cpu().tolist()
    ms_step = wall * 1e3 / args.steps
    value = w.tokens / (wall / args.steps)

    newton_ms = float(t_newt.mean())
    proj_ms = float(t_proj.mean())
    alg_bytes = algorithmic_newton_bytes(w)
    prof = profile_fields("k_newton_sp", w.name)
    roof_newton = {"kernel": "k_newton_sp (prn_newton_forward)", "bound": "hbm",
                   "achieved": alg_bytes / (newton_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "traffic": _field(prof, "traffic_bytes_per_launch"),
                   "algorithmic_bytes": alg_bytes}
    roof_newton["frac"] = roof_newton["achieved"] / roof_newton["peak"]
    if roof_newton["traffic"]:
        # what the kernel really moves: the single-pass schedule reads the projected inputs once and
        # writes no iterate, so its counted bytes are well below the K-pass method's algorithmic count
        roof_newton["achieved_counted"] = roof_newton["traffic"] / (newton_ms * 1e-3) / 1e9
        roof_newton["frac_counted"] = roof_newton["achieved_counted"] / HBM_PEAK_GBPS
    if _field(prof, "valu_busy") is not None:
        roof_newton["valu_busy"] = _field(prof, "valu_busy")
        roof_newton["valu_lane_slots_per_channel_step"] = next(
            (_field(prof, k) for k in prof if k.startswith("valu_lane_slots_per_channel_step")), None)
    fl = proj_flops(w)
    roof_proj = {"kernel": f"k_proj, {proj_tiles(w)} tiles (prn_input_proj)",
                 **mfma_roofline(w.dtype, fl, proj_ms, traffic=profiled_traffic("k_proj", w.name))}
    dominant = roof_newton if newton_ms >= proj_ms else roof_proj

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "cell": f"diag_{w.cell}", "B": w.B, "T": w.T, "d_in": w.d_in,
                   "d_h": w.d_h, "K": w.K, "n_seqs": w.n_seqs, "tokens": w.tokens},
        "roofline": dominant,
        "roofline_newton": roof_newton,
        "roofline_proj": roof_proj,
        "breakdown_ms": {"proj_mean": proj_ms, "newton_mean": newton_ms, "newton_median": float(np.median(t_newt)),
                         "newton_min": float(t_newt.min()), "step_event_mean": float(t_step.mean())},
        "newton_tokens_per_s": w.tokens / (newton_ms * 1e-3),
        "breakdown_ms_mall_flushed": {"proj_mean": float(t_proj_fl.mean()), "newton_mean": float(t_newt_fl.mean()),
                                      "newton_median": float(np.median(t_newt_fl)),
                                      "newton_min": float(t_newt_fl.min()),
                                      "newton_hbm_frac": alg_bytes / (float(t_newt_fl.mean()) * 1e-3) / 1e9
                                      / HBM_PEAK_GBPS},
        "residuals": residuals,
        "agreement": agreement,
        "k_star": kstar,
        "backward": backward,
        "fused": fused,
        "decode": decode,
        "headmix": headmix,
        "device": torch.cuda.get_device_name(0),
        "hip_runtime": torch.version.hip,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        print("[bench] cpu baseline (OpenMP unroll) ...", file=sys.stderr, flush=True)
        xp_host = xproj.float().cpu().numpy()
        out["cpu_baseline"]["openmp"] = cpu_openmp_unroll(w, xp_host, inp, inp["cu_seqlens"])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
