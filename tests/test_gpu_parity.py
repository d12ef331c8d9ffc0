"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Tolerances (max-abs):
  * GPU Newton vs oracle Newton at equal K: 1e-5 with fp32 storage; 2e-2
    with bf16 storage (every stored state carries a rounding of up to 2^-9
    relative, which the next linearisation feeds on).
  * GPU Newton at K = 3 (GRU) or K = 4 (LSTM) vs the oracle's sequential
    unroll: tau = 1e-4 in fp32 (FAQs, "Does parallel Newton match sequential
    unroll?"), 2e-2 in bf16.
  * residuals r_k: 2e-5 + 1e-3 r (fp32), 2e-2 + 2e-2 r (bf16); r_K against
    an fp64 recomputation on the GPU's own output: 1e-6 + 1e-4 r.
  * projection: fp32 1e-5; bf16 one rounding of the fp32 sum (2^-8 |ref|)
    plus 1e-4.
The small cases span several chunks (32 steps), several 64-channel tiles
with a partial last tile, and a ragged time tail.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (gpu_run, gpu_sequential, oracle_newton, oracle_sequential, say, small_inputs, state_err, to_dev,
                         to_f64, tol, TORCH_DT)
import nonlinear_rnn_amd as prn
from oracle import proj as oproj
from oracle import newton as onewton
from oracle import rounding as oround
from workloads import Workload, WORKLOADS, random_state

pytestmark = pytest.mark.gpu

SMALL = [
    Workload("gru_small", "gru", 3, 1000, 24, 80, "f32", 3),
    Workload("lstm_small", "lstm", 2, 777, 16, 72, "f32", 2),
    Workload("gru_bf16_small", "gru", 2, 600, 32, 64, "bf16", 3),
    Workload("lstm_bf16_small", "lstm", 2, 300, 16, 130, "bf16", 3),
    Workload("gru_ragged_small", "gru", 1, 1500, 16, 40, "f32", 3, n_seqs=7),
    Workload("lstm_ragged_small", "lstm", 1, 900, 16, 64, "f32", 3, n_seqs=5, seg_lo=1, seg_hi=400),
    WORKLOADS["gru_tiny"],
]
IDS = [w.name for w in SMALL]


def xp64_of(w, xproj):
    return to_f64(xproj)


@pytest.fixture(params=["sp", "tp"])
def algo(request, monkeypatch):
    """Newton schedule: 'sp' single-pass look-back kernel (default), 'tp'
    three-phase kernels.  The library reads PRN_ALGO at every call."""
    monkeypatch.setenv("PRN_ALGO", request.param)
    return request.param


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_projection_matches_oracle(w):
    say(f"[case] projection {w}")
    inp = small_inputs(w)
    out = gpu_run(w, inp, 1)
    got = to_f64(out["xproj"])
    ref = oproj.input_proj(oround.load(inp["x"], w.dtype), oround.load(inp["W"], w.dtype),
                           inp["bias"].astype(np.float64), w.G)
    if w.dtype == "f32":
        assert np.abs(got - ref).max() <= 1e-5
    else:
        assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 1e-4)


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_newton_matches_oracle_at_equal_K(w, algo):
    say(f"[case] newton equal-K {w}")
    inp = small_inputs(w)
    out = gpu_run(w, inp, w.K)
    xp = xp64_of(w, out["xproj"])
    ref = oracle_newton(w, xp, inp["a"], w.K, cu=inp["cu_seqlens"])
    H = to_f64(out["H"])
    err = np.abs(H - ref["H"][..., -1, :]).max()
    say(f"  max|H_gpu - H_oracle| = {err:.3e}; residuals gpu {out['res']} oracle {ref['residuals']}")
    assert state_err(w, H, ref["H"][..., -1, :], 1e-5) <= 1
    last = to_f64(out["last"])
    assert state_err(w, last, ref["last"], 1e-5) <= 1
    r_g, r_o = out["res"], np.array(ref["residuals"])
    bound = (2e-5 + 1e-3 * r_o) if w.dtype == "f32" else (2e-2 + 2e-2 * r_o)
    assert np.all(np.abs(r_g - r_o) <= bound), (r_g, r_o)


@pytest.mark.parametrize("w", [w for w in SMALL if w.cell == "gru"] + [SMALL[1].scaled(K=4)],
                         ids=lambda w: f"{w.name}-K{w.K}")
def test_newton_agrees_with_sequential_within_tau(w, algo):
    say(f"[case] tau {w}")
    inp = small_inputs(w)
    out = gpu_run(w, inp, w.K)
    xp = xp64_of(w, out["xproj"])
    seq, _ = oracle_sequential(w, xp, inp["a"], cu=inp["cu_seqlens"])
    err = np.abs(to_f64(out["H"]) - seq[..., -1, :]).max()
    say(f"  max|H_newton - h_sequential| = {err:.3e}")
    assert state_err(w, to_f64(out["H"]), seq[..., -1, :], 1e-4) <= 1


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_sequential_kernel_matches_oracle(w):
    say(f"[case] sequential {w}")
    inp = small_inputs(w)
    out = gpu_run(w, inp, 1)
    H, last = gpu_sequential(w, inp, out["xproj"])
    xp = xp64_of(w, out["xproj"])
    seq, slast = oracle_sequential(w, xp, inp["a"], cu=inp["cu_seqlens"])
    assert state_err(w, to_f64(H), seq[..., -1, :], 1e-5) <= 1
    assert state_err(w, to_f64(last), slast, 1e-5) <= 1


@pytest.mark.parametrize("w", [SMALL[0], SMALL[4]], ids=["gru_small", "gru_ragged_small"])
def test_final_residual_equals_recomputation_on_output(w, algo):
    say(f"[case] residual recomputation {w}")
    inp = small_inputs(w)
    out = gpu_run(w, inp, w.K)
    xp = xp64_of(w, out["xproj"])
    H = to_f64(out["H"])[..., None, :]
    heads = onewton.head_segments(w.B, w.T, inp["cu_seqlens"])
    rows = w.B if inp["cu_seqlens"] is None else w.n_seqs
    r = onewton.residual("gru", H, xp, inp["a"].astype(np.float64), heads, np.zeros((rows, 1, w.d_h)))
    assert abs(out["res"][-1] - r) <= 1e-6 + 1e-4 * r


@pytest.mark.parametrize("w", [SMALL[1], SMALL[2], SMALL[4]], ids=lambda w: w.name)
def test_run_to_run_reproducibility(w, algo):
    """Both schedules combine the chunk carries in an order fixed by the
    chunk index (the single-pass look-back by a binary decomposition of the
    chunk index, never by which chunks happened to finish first): repeated
    runs are bitwise identical."""
    say(f"[case] reproducibility {w}")
    inp = small_inputs(w)
    o1 = gpu_run(w, inp, w.K)
    for _ in range(3):
        o2 = gpu_run(w, inp, w.K, xproj=o1["xproj"])
        assert torch.equal(o1["H"], o2["H"])
        assert torch.equal(o1["last"], o2["last"])
        assert np.array_equal(o1["res"], o2["res"])


def test_batch_rows_are_independent(algo):
    """A row computed alone equals the same row inside a batch, bit for bit
    (same chunk boundaries, same arithmetic; the LSTM's chunk length does not
    depend on the number of chains)."""
    w = SMALL[1]
    say(f"[case] batch independence {w}")
    inp = small_inputs(w)
    full = gpu_run(w, inp, w.K)
    for b in range(w.B):
        wb = w.scaled(B=1)
        ob = gpu_run(wb, inp, w.K, xproj=full["xproj"][b:b + 1].contiguous())
        assert torch.equal(ob["H"][0], full["H"][b])
        assert torch.equal(ob["last"][0], full["last"][b])


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_nonzero_h0_and_final_state(cell, algo):
    w = Workload(f"{cell}_h0", cell, 2, 200, 16, 48, "f32", 3)
    say(f"[case] h0 {w}")
    inp = small_inputs(w)
    h0 = random_state(w, w.B, seed=3)
    out = gpu_run(w, inp, w.K, h0=h0)
    xp = xp64_of(w, out["xproj"])
    ref = oracle_newton(w, xp, inp["a"], w.K, h0=h0)
    assert np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max() <= 1e-5
    assert np.abs(to_f64(out["last"]) - ref["last"]).max() <= 1e-5
    # continuation: the second half started from the first half's final state
    # equals the second half of one run (up to Newton's own error at K)
    K = 6
    whole = gpu_run(w, inp, K, h0=h0, xproj=out["xproj"])
    w1 = w.scaled(T=100)
    first = gpu_run(w1, inp, K, h0=h0, xproj=out["xproj"][:, :100].contiguous())
    second = gpu_run(w1, inp, K, h0=first["last"].float().cpu().numpy(),
                     xproj=out["xproj"][:, 100:].contiguous())
    assert torch.allclose(second["H"], whole["H"][:, 100:], atol=1e-5, rtol=0)


def test_packed_segments_match_separate_runs_and_empty_segments(algo):
    w = Workload("gru_pack", "gru", 1, 700, 16, 40, "f32", 3)
    say(f"[case] pack vs segments {w}")
    inp = small_inputs(w)
    cu = np.array([0, 0, 64, 64, 65, 300, 700, 700], dtype=np.int32)   # empty, length-1 and trailing empty
    h0 = random_state(w, len(cu) - 1, seed=5)
    wp = w.scaled(n_seqs=len(cu) - 1)
    pk = gpu_run(wp, inp, w.K, h0=h0, cu=cu)
    xp = xp64_of(w, pk["xproj"])
    ref = oracle_newton(wp, xp, inp["a"], w.K, h0=h0, cu=cu)
    assert np.abs(to_f64(pk["H"]) - ref["H"][..., -1, :]).max() <= 1e-5
    assert np.abs(to_f64(pk["last"]) - ref["last"]).max() <= 1e-5
    for j in range(len(cu) - 1):
        lo, hi = int(cu[j]), int(cu[j + 1])
        if hi == lo:
            assert torch.equal(pk["last"][j].cpu(), torch.from_numpy(h0[j]))
            continue
        ws = w.scaled(T=hi - lo)
        one = gpu_run(ws, inp, w.K, h0=h0[j:j + 1], xproj=pk["xproj"][:, lo:hi].contiguous())
        assert torch.allclose(one["H"][0], pk["H"][0, lo:hi], atol=1e-5, rtol=0)


# T at and just past whole single-pass chunks too: 64 steps (fp32 LSTM), 96
# (GRU below 64 chains)
@pytest.mark.parametrize("T,d_h,K", [(1, 16, 3), (31, 64, 2), (32, 64, 3), (33, 65, 3), (70, 1, 1),
                                     (45, 63, 50), (0, 16, 3), (64, 64, 3), (65, 40, 2), (96, 64, 3),
                                     (97, 64, 3), (192, 33, 4)])
@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_edge_shapes(cell, T, d_h, K, algo):
    w = Workload(f"{cell}_edge", cell, 2, T, 8, d_h, "f32", K)
    say(f"[case] edge {w}")
    inp = small_inputs(w)
    h0 = random_state(w, w.B, seed=9)
    out = gpu_run(w, inp, K, h0=h0)
    if T == 0:
        assert np.array_equal(out["res"], np.zeros(K + 1))
        assert np.abs(to_f64(out["last"]) - h0).max() == 0
        return
    xp = xp64_of(w, out["xproj"])
    ref = oracle_newton(w, xp, inp["a"], K, h0=h0)
    assert np.abs(to_f64(out["H"]) - ref["H"][..., -1, :]).max() <= 1e-5
    assert np.abs(to_f64(out["last"]) - ref["last"]).max() <= 1e-5
    if K >= T:   # Newton is exact after T iterations
        seq, _ = oracle_sequential(w, xp, inp["a"], h0=h0)
        assert np.abs(to_f64(out["H"]) - seq[..., -1, :]).max() <= 1e-5


def test_strided_view_example_from_the_shapes_page():
    """A (2, 32, 8) view with time stride 2 through the contiguity-copying
    wrapper: ParaGRU(8, 16), K = 3, must match the sequential unroll."""
    say("[case] strided view")
    g = torch.Generator().manual_seed(0)
    base = torch.randn(2, 64, 8, generator=g).cuda()
    x = base[:, ::2, :]
    assert not x.is_contiguous()
    W = (torch.randn(48, 8, generator=g) / 8 ** 0.5).cuda()
    a = (torch.rand(3, 16, generator=g) - 0.5).cuda()
    y_n, res = prn.forward(x, W, None, a, 3, cell="gru")
    y_s = prn.sequential_forward(prn.input_proj(x, W, None, cell="gru"), a, cell="gru")
    assert (y_n - y_s).abs().max().item() <= 1e-4
    rep = prn.verify_agreement(prn.input_proj(x, W, None, cell="gru"), a, 3, cell="gru")
    assert rep.ok and rep.max_abs <= 1e-4 and set(rep.to_dict()) >= {"ok", "max_abs"}


def test_divergence_gate_fires_on_non_finite_input(algo):
    say("[case] divergence gate")
    w = Workload("gru_nan", "gru", 1, 100, 8, 16, "f32", 3)
    inp = small_inputs(w)
    out = gpu_run(w, inp, 3)
    xp = out["xproj"].clone()
    xp[0, 50, 0, 3] = float("nan")
    a = torch.from_numpy(inp["a"]).cuda()
    with pytest.raises(prn.NewtonDivergenceError):
        prn.newton_forward(xp, a, 3, cell="gru")
    H, res = prn.newton_forward(xp, a, 3, cell="gru", gate=False)
    assert res[-1] == float("inf")
    assert prn.newton_forward(out["xproj"], a, 3, cell="gru")[1][-1] < 1e-3


def test_k_table_and_int64_offsets_through_the_wrapper():
    say("[case] k table / int64 cu")
    w = Workload("gru_tab", "gru", 1, 300, 8, 16, "f32", 3)
    inp = small_inputs(w)
    out = gpu_run(w, inp, 3)
    a = torch.from_numpy(inp["a"]).cuda()
    H1, r1 = prn.newton_forward(out["xproj"], a, None, cell="gru", k_table={64: 2, 1024: 3})
    assert len(r1) == 4 and torch.equal(H1, out["H"])
    cu = torch.tensor([0, 100, 300], dtype=torch.int64)
    H2, _ = prn.newton_forward(out["xproj"], a, 3, cell="gru", cu_seqlens=cu)
    with pytest.raises(prn.PrnError):
        prn.newton_forward(out["xproj"], a, 3, cell="gru", cu_seqlens=torch.tensor([0, 100, 299]))


@pytest.mark.parametrize("w", SMALL, ids=IDS)
def test_single_pass_and_three_phase_agree(w, monkeypatch):
    """Two independent schedules of the same Newton iteration (different
    chunking, carries from a look-back vs from a separate scan kernel)."""
    say(f"[case] sp vs tp {w}")
    inp = small_inputs(w)
    monkeypatch.setenv("PRN_ALGO", "sp")
    o1 = gpu_run(w, inp, w.K)
    monkeypatch.setenv("PRN_ALGO", "tp")
    o2 = gpu_run(w, inp, w.K, xproj=o1["xproj"])
    assert state_err(w, to_f64(o1["H"]), to_f64(o2["H"]), 1e-5) <= 1
    assert np.all(np.abs(o1["res"] - o2["res"]) <= tol(w, 2e-5) + 1e-3 * o2["res"])


@pytest.mark.parametrize("dtype,T,d_in,d_h,cell", [("f32", 262144 + 77, 36, 80, "lstm"),
                                                   ("bf16", 262144 + 77, 40, 72, "gru"),
                                                   ("f32", 262144 + 77, 256, 256, "lstm"),
                                                   ("f32", 262144, 128, 64, "lstm"),
                                                   ("bf16", 262144, 64, 64, "lstm")])
def test_large_projection_with_ragged_tiles(dtype, T, d_in, d_h, cell):
    """Projections large enough for the 256 x 256 direct-to-LDS tiles: with a
    partial last row tile, a partial last column tile and a partial last K
    stage (the guarded instance: rows past M / N load the last row, chunks
    past K a zero chunk), and exactly tiled (the unguarded instance): every
    output against the fp64 product."""
    w = Workload("proj_large", cell, 1, T, d_in, d_h, dtype, 1)
    say(f"[case] large projection {w}")
    inp = small_inputs(w)
    x = to_dev(inp["x"], dtype)
    W = to_dev(inp["W"], dtype)
    bias = torch.from_numpy(inp["bias"]).cuda()
    xproj = torch.full((w.B, w.T, w.G, w.d_h), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
    prn.binding.prn_input_proj(x, W, bias, xproj, cell=cell)
    torch.cuda.synchronize()
    got = to_f64(xproj)
    ref = oproj.input_proj(oround.load(inp["x"], dtype), oround.load(inp["W"], dtype),
                           inp["bias"].astype(np.float64), w.G)
    assert np.all(np.isfinite(got))
    if dtype == "f32":
        assert np.abs(got - ref).max() <= 1e-5
    else:
        assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 1e-4)


def test_device_bf16_rounding_matches_the_oracle_bitwise():
    """bf16 storage rounding on the device (v_cvt_pk_bf16_f32) against the
    oracle's round-to-nearest-even, bit for bit.  The projection with an
    identity W computes xproj = x + bias exactly in fp32 (one exact product,
    then one fp32 addition) and rounds it once, so crafted x and bias put the
    fp32 sums on exact ties (either parity of the kept bit), just beside
    them, at random, and past the largest bf16 value (overflow to Inf)."""
    rng = np.random.default_rng(11)
    d_h, G, T = 64, 3, 256
    N = G * d_h
    e = rng.integers(-20, 20, size=N)                      # binade of column n's x values
    kind = np.arange(N) % 6
    scale = np.exp2(e.astype(np.float64))
    half_ulp = scale * 2.0 ** -8                             # bf16 keeps 8 significant bits
    bias = np.where(kind == 0, half_ulp, np.where(kind == 1, -half_ulp,
                    np.where(kind == 2, half_ulp * (1 + 2.0 ** -12), np.where(kind == 3, half_ulp * (1 - 2.0 ** -12),
                    rng.standard_normal(N) * scale))))
    mant = 1.0 + rng.integers(0, 128, size=(T, N)) / 128.0   # 8 significant bits: exact in bf16
    sign = np.where(rng.random((T, N)) < 0.5, -1.0, 1.0)
    x = sign * mant * scale
    big = np.array([0x7F7F0000, 0x7F7E0000], dtype=np.uint32).view(np.float32).astype(np.float64)  # bf16 max, next below
    x[:, kind == 5] = np.where(rng.random((T, int((kind == 5).sum()))) < 0.5, big[0], big[1])
    bias[kind == 5] = np.where(np.arange(int((kind == 5).sum())) % 2 == 0, 3.0e35, 1.0e36)
    x32 = x.astype(np.float32)
    b32 = bias.astype(np.float32)
    assert np.array_equal(oround.bf16_round(x32), x32.astype(np.float64))   # x is exactly bf16
    xd = torch.from_numpy(x32.reshape(1, T, N)).to(torch.bfloat16).cuda()
    Wd = torch.eye(N, dtype=torch.float32).to(torch.bfloat16).cuda()
    xproj = torch.empty((1, T, G, d_h), dtype=torch.bfloat16, device="cuda")
    prn.binding.prn_input_proj(xd, Wd, torch.from_numpy(b32).cuda(), xproj, cell="gru")
    torch.cuda.synchronize()
    got = xproj.reshape(T, N).view(torch.int16).cpu().numpy().view(np.uint16)
    ref64 = oround.bf16_round((x32 + b32).astype(np.float64))   # fp32 sum, then round to bf16
    ref = (ref64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.isinf(ref64[:, kind == 5]).any() and not np.isinf(ref64[:, kind == 5]).all()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]:#06x} want {ref[tuple(bad[0])]:#06x}"
