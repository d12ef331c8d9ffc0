"""K*(T) campaign: the smallest Newton depth whose forward matches the
sequential unroll within tau, measured on the GPU through the C ABI
(FAQs, "What is critical Newton depth (K*)?"; Numerics contract, "2. Lab
campaign": measured envelopes become a per-T table that the training
config resolves K from).

    python -m nonlinear_rnn_amd.kstar --cell lstm      # measure, print the table
    python -m nonlinear_rnn_amd.kstar --write          # measure both cells, write kstar_table.json

Each cell is measured twice: plain Newton from 0, and after one Picard
sweep (picard_iters = 1), with the forward's time at each K*.

The agreement norm is max-abs over h (the pages' report.max_abs).  Inputs
follow the seeded workload recipe (x ~ N(0,1), W ~ N(0, 1/d_in), a ~
U(-0.5, 0.5), LSTM forget bias +1) at each T.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

from . import binding as B_

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE_PATH = os.path.join(HERE, "kstar_table.json")
TAU = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def agreement_errors(xproj, a, K_max: int, *, cell: str, h0=None, cu_seqlens=None, stream=None,
                     picard_iters: int = 0):
    """[max|h^(K) - h_seq| for K = 1..K_max], each K a separate Newton forward
    (after picard_iters Picard sweeps)."""
    Bn, T, _, d_h = xproj.shape
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    Hs = torch.empty((Bn, T, d_h), dtype=xproj.dtype, device=xproj.device)
    B_.prn_sequential_forward(xproj, a, Hs, cell=cell, h0=h0, cu_seqlens=cu_seqlens, stream=stream)
    ws = torch.empty(max(B_.prn_workspace_bytes(cell, xproj.dtype, Bn, T, d_h, K_max, n_seqs=n_seqs,
                                                picard_iters=picard_iters), 1),
                     dtype=torch.uint8, device=xproj.device)
    H = torch.empty_like(Hs)
    errs = []
    for K in range(1, K_max + 1):
        B_.prn_newton_forward(xproj, a, K, H, cell=cell, h0=h0, cu_seqlens=cu_seqlens, workspace=ws,
                              stream=stream, picard_iters=picard_iters)
        errs.append(float((H.float() - Hs.float()).abs().max()))
    return errs


def time_forward(xproj, a, K: int, *, cell: str, picard_iters: int = 0, reps: int = 10) -> float:
    """Mean ms of one prn_newton_forward (HIP events on the current stream)."""
    Bn, T, _, d_h = xproj.shape
    ws = torch.empty(max(B_.prn_workspace_bytes(cell, xproj.dtype, Bn, T, d_h, K, picard_iters=picard_iters), 1),
                     dtype=torch.uint8, device=xproj.device)
    H = torch.empty((Bn, T, d_h), dtype=xproj.dtype, device=xproj.device)
    run = lambda: B_.prn_newton_forward(xproj, a, K, H, cell=cell, workspace=ws, picard_iters=picard_iters)
    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def kstar(errors, tau):
    for k, e in enumerate(errors, start=1):
        if e <= tau:
            return k
    return None


def synthetic_xproj(cell: str, B: int, T: int, d_in: int, d_h: int, dtype, seed: int):
    """Projected inputs of the seeded recipe, made on the GPU by prn_input_proj."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    G = B_.GATES[cell]
    x = torch.randn((B, T, d_in), generator=g, device="cuda").to(dtype)
    W = (torch.randn((G * d_h, d_in), generator=g, device="cuda") / d_in ** 0.5).to(dtype)
    a = torch.rand((G, d_h), generator=g, device="cuda") - 0.5
    bias = torch.zeros(G * d_h, device="cuda")
    if cell == "lstm":
        bias[d_h:2 * d_h] = 1.0
    xproj = torch.empty((B, T, G, d_h), dtype=dtype, device="cuda")
    B_.prn_input_proj(x, W, bias, xproj, cell=cell)
    return xproj, a.contiguous()


def campaign(cell: str, Ts, *, B=2, d_in=256, d_h=256, dtype=torch.float32, K_max=6, seeds=(0, 1, 2), tau=None,
             picard_iters=0):
    """{T: {"kstar": max over seeds, "errors": per-seed error lists, "ms_at_kstar"}}."""
    tau = TAU[dtype] if tau is None else tau
    out = {}
    for T in Ts:
        per_seed, ks = [], []
        for s in seeds:
            xproj, a = synthetic_xproj(cell, B, T, d_in, d_h, dtype, seed=1000 * T + s)
            errs = agreement_errors(xproj, a, K_max, cell=cell, picard_iters=picard_iters)
            per_seed.append(errs)
            ks.append(kstar(errs, tau))
        k = None if any(v is None for v in ks) else max(ks)
        ms = time_forward(xproj, a, k, cell=cell, picard_iters=picard_iters) if k else None
        out[int(T)] = {"kstar": k, "errors": per_seed, "ms_at_kstar": ms}
        print(f"[kstar] {cell} P={picard_iters} T={T}: K* = {k}  (per seed {ks}; errors at K*: "
              f"{[e[k - 1] if k else None for e in per_seed]}; {ms} ms at K*)", file=sys.stderr, flush=True)
    return out


def monotone_table(result: dict) -> dict:
    """{T: K} made monotone in T (a longer sequence never gets a smaller K)."""
    tab, run = {}, 0
    for T in sorted(result):
        k = result[T]["kstar"]
        if k is None:
            break
        run = max(run, k)
        tab[int(T)] = run
    return tab


def load_table(cell: str) -> dict:
    """The committed per-T table of a cell ({T: K}), for resolve_k."""
    with open(TABLE_PATH) as f:
        data = json.load(f)
    return {int(k): int(v) for k, v in data["tables"][cell].items()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--cell", choices=["gru", "lstm"], default=None)
    ap.add_argument("--T", type=int, nargs="*", default=[64, 256, 1024, 4096, 16384, 65536, 131072])
    ap.add_argument("--K-max", type=int, default=6)
    ap.add_argument("--write", action="store_true", help=f"write {os.path.basename(TABLE_PATH)}")
    ap.add_argument("--out", default=None, help="write the table document to this path instead")
    args = ap.parse_args(argv)
    cells = [args.cell] if args.cell else ["gru", "lstm"]
    t0 = time.time()
    results = {c: campaign(c, args.T, K_max=args.K_max) for c in cells}
    results_p = {c: campaign(c, args.T, K_max=args.K_max, picard_iters=1) for c in cells}
    doc = {
        "what": "K*(T): smallest Newton depth with max|h_newton - h_sequential| <= tau, max over seeds",
        "tau": TAU[torch.float32], "dtype": "f32", "B": 2, "d_in": 256, "d_h": 256, "seeds": [0, 1, 2],
        "inputs": "x ~ N(0,1), W ~ N(0, 1/d_in), a ~ U(-0.5, 0.5), LSTM forget bias +1, h0 = 0",
        "device": torch.cuda.get_device_name(0),
        "command": "python -m nonlinear_rnn_amd.kstar" + (" --write" if args.write else ""),
        "seconds": round(time.time() - t0, 1),
        "tables": {c: monotone_table(results[c]) for c in cells},
        "tables_picard1": {c: monotone_table(results_p[c]) for c in cells},
        "measurements": {c: {str(T): v for T, v in results[c].items()} for c in cells},
        "measurements_picard1": {c: {str(T): v for T, v in results_p[c].items()} for c in cells},
    }
    print(json.dumps({"tables": doc["tables"], "tables_picard1": doc["tables_picard1"]}))
    if args.write or args.out:
        with open(args.out or TABLE_PATH, "w") as f:
            json.dump(doc, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
