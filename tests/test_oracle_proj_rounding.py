"""Pins for the oracle's projection (brute force) and bf16 rounding (library cast)."""
import numpy as np
import torch

from oracle import proj, rounding
from workloads import f32_to_bf16_bits, bf16_bits_to_f32


def test_projection_against_brute_force_loops():
    rng = np.random.default_rng(0)
    B, T, d_in, G, d_h = 2, 3, 5, 4, 3
    x = rng.standard_normal((B, T, d_in))
    W = rng.standard_normal((G * d_h, d_in))
    bias = rng.standard_normal(G * d_h)
    got = proj.input_proj(x, W, bias, G)
    for b in range(B):
        for t in range(T):
            for g in range(G):
                for i in range(d_h):
                    acc = bias[g * d_h + i]
                    for j in range(d_in):
                        acc += x[b, t, j] * W[g * d_h + i, j]
                    assert abs(got[b, t, g, i] - acc) < 1e-12


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9,
                  3.3895313892515355e38, 3.4e38, -3.4e38, np.inf, -np.inf, 1e-40, -1e-42]),
    ])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = rounding.bf16_round(v32.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.isnan(rounding.bf16_round(np.array([np.nan]))[0])
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert rounding.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert rounding.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_generator_bf16_bits_roundtrip():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(1000).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    np.testing.assert_array_equal(bf16_bits_to_f32(bits).astype(np.float64), rounding.bf16_round(v))
    np.testing.assert_array_equal(rounding.bf16_from_bits(bits), rounding.bf16_round(v))


def test_projection_backward_against_finite_differences():
    """dx, dW and dbias of the oracle's projection backward are the central
    finite differences of L = sum(w * input_proj(x, W, bias)) (exact up to
    rounding: L is linear in each operand), element by element."""
    rng = np.random.default_rng(11)
    B, T, d_in, d_h, G = 2, 3, 5, 4, 3
    x = rng.standard_normal((B, T, d_in))
    W = rng.standard_normal((G * d_h, d_in))
    bias = rng.standard_normal(G * d_h)
    w = rng.standard_normal((B, T, G, d_h))   # dL/dxproj

    def L(x_, W_, b_):
        return float((w * proj.input_proj(x_, W_, b_, G)).sum())

    dx, dW, db = proj.input_proj_backward(w, x, W)
    eps = 1e-6
    for arr, grad, args in ((x, dx, lambda a: (a, W, bias)), (W, dW, lambda a: (x, a, bias)),
                            (bias, db, lambda a: (x, W, a))):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            fd[idx] = (L(*args(ap)) - L(*args(am))) / (2 * eps)
        assert np.abs(fd - grad).max() <= 1e-7
