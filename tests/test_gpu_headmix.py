"""GPU parity of the head-mix GRU (dense 16 x 16 recurrent blocks per head)
against the oracle (oracle/headmix.py), through the C ABI.

Tolerances (max-abs, fp32 storage): Newton vs the oracle's Newton at equal
K 1e-5 (each 16-term block product carries fp32 rounding into the next
linearisation); the sequential kernel vs the oracle's unroll 1e-5; Newton
at a converged K vs the unroll tau = 1e-4; residuals 2e-5 + 1e-3 r.  bf16
storage (xproj, h0, iterates, H): BF16_ABS on h against the oracle's Newton
with bf16 stores and against its float64 unroll; residuals 2e-2 + 2e-2 r.
The small cases span several 64-step chunks with a ragged tail, several
heads, B > 1, and T = 1.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import hm_dev as dev, hm_inputs as inputs, hm_newton as gpu_newton, hm_sequential as gpu_sequential, say, to_f64
from nonlinear_rnn_amd import binding as B
from gpu_helpers import BF16_ABS
from oracle import headmix as ohm
from oracle import rounding as oround

pytestmark = pytest.mark.gpu


# (B, T, d_h, seed): several 32-step chunks with a ragged tail, exactly one
# chunk, T = 1, and 38 chunks (the two-level carries: three groups of 16
# chunks, the last one partial)
CASES = [(2, 200, 32, 1), (1, 64, 16, 2), (3, 1, 48, 3), (2, 1000, 64, 4), (1, 129, 128, 5), (2, 1189, 32, 6)]


@pytest.mark.parametrize("Bn,T,d_h,seed", CASES)
@pytest.mark.parametrize("K", [1, 2, 3])
def test_newton_matches_oracle_at_equal_K(Bn, T, d_h, seed, K):
    say(f"[case] head-mix newton B={Bn} T={T} d_h={d_h} K={K}")
    xp, A, h0 = inputs(Bn, T, d_h, seed)
    H, res, last = gpu_newton(xp, A, K, h0, want_last=True)
    ref = ohm.newton(xp, A, K, h0=h0, dtype="f32")
    e = np.abs(H - ref["H"]).max()
    say(f"  H err {e:.2e}; residuals gpu {np.round(res, 6)} oracle {np.round(ref['residuals'], 6)}")
    assert e <= 1e-5
    assert np.array_equal(last, H[:, T - 1])
    r = np.asarray(ref["residuals"])
    assert np.all(np.abs(res - r) <= 2e-5 + 1e-3 * r)


@pytest.mark.parametrize("Bn,T,d_h,seed", CASES)
def test_sequential_kernel_matches_oracle(Bn, T, d_h, seed):
    xp, A, h0 = inputs(Bn, T, d_h, seed)
    H, last = gpu_sequential(xp, A, h0)
    ref, ref_last = ohm.sequential(xp, A, h0=h0)
    e = np.abs(H - ref).max()
    say(f"[case] head-mix sequential B={Bn} T={T} d_h={d_h}: {e:.2e}")
    assert e <= 1e-5 and np.abs(last - ref_last).max() <= 1e-5


def _bf16_case(Bn, T, d_h, seed):
    """Inputs held in bf16 (xproj and h0 rounded to nearest even once), A in fp32."""
    xp, A, h0 = inputs(Bn, T, d_h, seed)
    return oround.bf16_round(xp), A, (None if h0 is None else oround.bf16_round(h0))


def _dev16(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


@pytest.mark.parametrize("Bn,T,d_h,seed", CASES)
@pytest.mark.parametrize("K", [1, 3])
def test_bf16_newton_matches_oracle_at_equal_K(Bn, T, d_h, seed, K):
    """bf16 storage: iterates stored rounded (the oracle's store), every block
    product and the chain in fp32.  Band: BF16_ABS on h (a rounding flip of
    one stored iterate between fp32 and fp64 arithmetic moves h by one bf16
    step); residuals 2e-2 + 2e-2 r as for the diagonal bf16 cells."""
    say(f"[case] head-mix bf16 newton B={Bn} T={T} d_h={d_h} K={K}")
    xp, A, h0 = _bf16_case(Bn, T, d_h, seed)
    H = torch.empty((Bn, T, d_h), dtype=torch.bfloat16, device="cuda")
    res = torch.full((K + 1,), -1.0, device="cuda")
    last = torch.empty((Bn, d_h), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(B.prn_head_workspace_bytes(Bn, T, d_h, K, dtype=torch.bfloat16), 1), dtype=torch.uint8,
                     device="cuda")
    B.prn_head_newton_forward(_dev16(xp), dev(A), K, H, h0=_dev16(h0), residual_out=res, state_last_out=last,
                              workspace=ws)
    torch.cuda.synchronize()
    Hg, resg = to_f64(H), res.cpu().numpy().astype(np.float64)
    ref = ohm.newton(xp, A, K, h0=h0, dtype="bf16")
    e = np.abs(Hg - ref["H"]).max()
    say(f"  H err {e:.2e}; residuals gpu {np.round(resg, 5)} oracle {np.round(ref['residuals'], 5)}")
    assert e <= BF16_ABS
    assert np.array_equal(to_f64(last), Hg[:, T - 1])
    r = np.asarray(ref["residuals"])
    assert np.all(np.abs(resg - r) <= 2e-2 + 2e-2 * r)


@pytest.mark.parametrize("Bn,T,d_h,seed", CASES[:3])
def test_bf16_sequential_kernel_matches_oracle(Bn, T, d_h, seed):
    """bf16 storage: the chain in fp32, every output rounded once; against the
    oracle's float64 unroll on the same (rounded) inputs, band BF16_ABS."""
    xp, A, h0 = _bf16_case(Bn, T, d_h, seed)
    H = torch.empty((Bn, T, d_h), dtype=torch.bfloat16, device="cuda")
    last = torch.empty((Bn, d_h), dtype=torch.bfloat16, device="cuda")
    B.prn_head_sequential_forward(_dev16(xp), dev(A), H, h0=_dev16(h0), state_last_out=last)
    torch.cuda.synchronize()
    ref, ref_last = ohm.sequential(xp, A, h0=h0)
    e = np.abs(to_f64(H) - ref).max()
    say(f"[case] head-mix bf16 sequential B={Bn} T={T} d_h={d_h}: {e:.2e}")
    assert e <= BF16_ABS and np.abs(to_f64(last) - ref_last).max() <= BF16_ABS


def test_bf16_run_to_run_and_mixed_dtypes_rejected():
    xp, A, h0 = _bf16_case(2, 300, 32, 9)
    outs = []
    for _ in range(2):
        H = torch.empty((2, 300, 32), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(B.prn_head_workspace_bytes(2, 300, 32, 3, dtype=torch.bfloat16), dtype=torch.uint8,
                         device="cuda")
        B.prn_head_newton_forward(_dev16(xp), dev(A), 3, H, h0=_dev16(h0), workspace=ws)
        torch.cuda.synchronize()
        outs.append(H)
    assert torch.equal(outs[0], outs[1])
    with pytest.raises(TypeError):   # H_out must share xproj's storage dtype
        B.prn_head_newton_forward(_dev16(xp), dev(A), 3, torch.empty((2, 300, 32), device="cuda"), workspace=ws)


def test_newton_converges_to_the_unroll():
    xp, A, h0 = inputs(2, 1500, 64, seed=8)
    seq, _ = gpu_sequential(xp, A, h0)
    errs = []
    for K in (1, 2, 3, 4, 5, 6):
        H, res, _ = gpu_newton(xp, A, K, h0)
        errs.append(np.abs(H - seq).max())
    say(f"  head-mix newton vs unroll by K: {[f'{e:.1e}' for e in errs]}")
    assert errs[-1] <= 1e-4
    assert errs[2] < errs[0]


def test_zero_h0_and_no_optional_outputs():
    xp, A, _ = inputs(2, 130, 32, seed=6, with_h0=False)
    Bn, T, _, d_h = xp.shape
    H = torch.empty((Bn, T, d_h), device="cuda")
    ws = torch.empty(B.prn_head_workspace_bytes(Bn, T, d_h, 2), dtype=torch.uint8, device="cuda")
    B.prn_head_newton_forward(dev(xp), dev(A), 2, H, workspace=ws)
    torch.cuda.synchronize()
    ref = ohm.newton(xp, A, 2, dtype="f32")
    assert np.abs(to_f64(H) - ref["H"]).max() <= 1e-5


def test_diagonal_blocks_match_the_diagonal_gru_kernel():
    """Diagonal blocks diag(a) reproduce the diagonal GRU path at equal K."""
    rng = np.random.default_rng(12)
    Bn, T, d_h, K = 2, 300, 32, 3
    xp = rng.standard_normal((Bn, T, 3, d_h)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (3, d_h)).astype(np.float32)
    A = np.zeros((3, d_h // 16, 16, 16), dtype=np.float32)
    for g in range(3):
        for k in range(d_h // 16):
            A[g, k] = np.diag(a[g, 16 * k:16 * (k + 1)])
    Hh, _, _ = gpu_newton(xp.astype(np.float64), A.astype(np.float64), K)
    Hd = torch.empty((Bn, T, d_h), device="cuda")
    ws = torch.empty(B.prn_workspace_bytes("gru", torch.float32, Bn, T, d_h, K), dtype=torch.uint8, device="cuda")
    B.prn_newton_forward(dev(xp), dev(a), K, Hd, cell="gru", workspace=ws)
    torch.cuda.synchronize()
    e = np.abs(Hh - to_f64(Hd)).max()
    say(f"  diagonal blocks vs diagonal GRU kernel: {e:.2e}")
    assert e <= 1e-5


def test_full_size_against_the_unroll_and_sampled_oracle():
    """8 x 4096 x 256 (16 heads) at K = 3 and K = 5: the GPU unroll agrees with
    the oracle's unroll on one row, and Newton at K = 5 with the unroll within
    tau."""
    xp, A, h0 = inputs(8, 4096, 256, seed=21, with_h0=False)
    seq, _ = gpu_sequential(xp, A)
    ref1, _ = ohm.sequential(xp[5:6], A)
    e_seq = np.abs(seq[5:6] - ref1).max()
    H5, res5, _ = gpu_newton(xp, A, 5)
    e_n = np.abs(H5 - seq).max()
    say(f"[case] head-mix full size: unroll vs oracle row 5 {e_seq:.2e}; K=5 vs unroll {e_n:.2e}; r_5 {res5[-1]:.2e}")
    assert e_seq <= 1e-5 and e_n <= 1e-4
