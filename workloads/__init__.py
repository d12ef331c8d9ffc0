"""Seeded synthetic inputs for the parallel-Newton diagonal GRU/LSTM forward.

This module only draws random numbers and casts them to the storage dtype.
It holds none of the method's arithmetic, so both the HIP path (through its
tests and the bench) and the CPU oracle can consume the same bytes.

Workloads (cell, batch, length, widths, storage dtype, Newton depth K):

  gru_tiny     diag GRU   B=1,  T=1024,   d_in=8,   d_h=16,  fp32, K=3
  gru_d256     diag GRU   B=8,  T=4096,   d_in=256, d_h=256, fp32, K=3
  gru_bf16     diag GRU   B=16, T=16384,  d_in=512, d_h=512, bf16, K=3
  lstm_t131k   diag LSTM  B=2,  T=131072, d_in=256, d_h=256, fp32, K=2
  gru_ragged   diag GRU   one pack of N=65536 tokens in 64 segments,
               d_in=256, d_h=256, fp32, K=3

Distributions: x ~ N(0, 1); W ~ N(0, 1/d_in) with rows gate-major
([z|r|c] for the GRU, [i|f|o|g] for the LSTM); diagonal recurrent weights
a ~ U(-0.5, 0.5) kept in fp32; biases 0 except the LSTM forget gate (+1);
h0 = 0.  Ragged segment lengths are drawn uniformly in [64, 2048] and
rescaled to sum to N: floor of the scaled lengths, the remainder handed out
one token at a time to the largest fractional parts (ties to the lower
index).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GATES = {"gru": 3, "lstm": 4}
STATE = {"gru": 1, "lstm": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cell: str          # "gru" | "lstm"
    B: int
    T: int             # for a ragged pack: N, the total token count
    d_in: int
    d_h: int
    dtype: str         # "f32" | "bf16"  (storage dtype of x, W, xproj, iterates)
    K: int
    n_seqs: int = 0    # 0 = rectangular batch; else number of packed segments
    seg_lo: int = 64
    seg_hi: int = 2048

    @property
    def G(self) -> int:
        return GATES[self.cell]

    @property
    def S(self) -> int:
        return STATE[self.cell]

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("gru_tiny", "gru", 1, 1024, 8, 16, "f32", 3),
        Workload("gru_d256", "gru", 8, 4096, 256, 256, "f32", 3),
        Workload("gru_bf16", "gru", 16, 16384, 512, 512, "bf16", 3),
        Workload("lstm_t131k", "lstm", 2, 131072, 256, 256, "f32", 2),
        Workload("gru_ragged", "gru", 1, 65536, 256, 256, "f32", 3, n_seqs=64),
    )
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.

    Input preparation only: the generator stores bf16 inputs as raw bits so
    every consumer sees the same bytes.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def segment_lengths(rng: np.random.Generator, n_seqs: int, N: int, lo: int, hi: int) -> np.ndarray:
    """Draw n_seqs lengths uniformly in [lo, hi] and rescale them to sum to N."""
    raw = rng.integers(lo, hi + 1, size=n_seqs).astype(np.int64)
    exact = raw.astype(np.float64) * N / raw.sum()
    base = np.floor(exact).astype(np.int64)
    rem = int(N - base.sum())
    frac = exact - base
    # largest fractional part first, ties broken by the lower index
    order = sorted(range(n_seqs), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    assert base.sum() == N
    return base


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw the inputs of workload ``w``.

    Returns numpy arrays in storage form: ``x`` (B,T,d_in) and ``W``
    (G*d_h, d_in) are float32 for dtype f32 and uint16 bf16 bits for bf16;
    ``a`` (G,d_h) and ``bias`` (G*d_h,) are float32; ``h0`` is None (zero
    initial state); ``cu_seqlens`` is an int32 (n_seqs+1,) array for a
    ragged pack, else None.
    """
    rng = np.random.default_rng(seed)
    G, d_h, d_in = w.G, w.d_h, w.d_in
    # every draw is float64 (numpy's default), then cast to the storage dtype
    x = rng.standard_normal((w.B, w.T, d_in)).astype(np.float32)
    W = (rng.standard_normal((G * d_h, d_in)) / math.sqrt(d_in)).astype(np.float32)
    a = rng.uniform(-0.5, 0.5, (G, d_h)).astype(np.float32)
    bias = np.zeros(G * d_h, dtype=np.float32)
    if w.cell == "lstm":
        bias[d_h:2 * d_h] = 1.0
    cu = None
    if w.n_seqs:
        assert w.B == 1
        L = segment_lengths(rng, w.n_seqs, w.T, w.seg_lo, w.seg_hi)
        cu = np.zeros(w.n_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(L)
    if w.dtype == "bf16":
        x = f32_to_bf16_bits(x)
        W = f32_to_bf16_bits(W)
    return {"x": x, "W": W, "a": a, "bias": bias, "h0": None, "cu_seqlens": cu}


def random_state(w: Workload, rows: int, seed: int, scale: float = 0.5) -> np.ndarray:
    """A non-zero initial state (rows, S, d_h) in fp32 for tests of h0 handling."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((rows, w.S, w.d_h))).astype(np.float32)


def random_xproj(w: Workload, seed: int, scale: float = 1.0) -> np.ndarray:
    """A projected-input tensor (B,T,G,d_h) drawn directly, in storage form.

    Used where a test exercises the Newton engine without the projection.
    """
    rng = np.random.default_rng(seed)
    xp = (scale * rng.standard_normal((w.B, w.T, w.G, w.d_h), dtype=np.float32))
    if w.cell == "lstm":
        xp[:, :, 1, :] += 1.0
    if w.dtype == "bf16":
        return f32_to_bf16_bits(xp)
    return xp
