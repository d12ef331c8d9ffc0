"""Input projection xproj = x W^T + bias (float64).

The FAQs and shapes/layout pages name the input weight W_x, applied once to
the whole sequence before the recurrence (decode_wx for single tokens).  The
projected tensor is laid out (B, T, G, d_h): for every token, G gate blocks
of d_h channels in gate order ([z|r|c] GRU, [i|f|o|g] LSTM), biases folded
in.  A library matmul is the step; nothing else is done.
"""
from __future__ import annotations

import numpy as np


def input_proj(x64: np.ndarray, W64: np.ndarray, bias64, G: int) -> np.ndarray:
    """x64 (B,T,d_in), W64 (G*d_h, d_in), bias64 (G*d_h,) or None -> (B,T,G,d_h)."""
    B, T, _ = x64.shape
    y = x64 @ W64.T
    if bias64 is not None:
        y = y + bias64
    return y.reshape(B, T, G, -1)


def input_proj_backward(g64: np.ndarray, x64: np.ndarray, W64: np.ndarray):
    """Gradients of a loss L through xproj = x W^T + bias, given
    g64 = dL/dxproj (B,T,G,d_h): the chain rule through a linear map,
    written as library matmuls:
        dx    = g W        (B,T,d_in)
        dW    = g^T x      (G*d_h, d_in), summed over every token
        dbias = sum of g   (G*d_h,)"""
    B, T = g64.shape[:2]
    g = g64.reshape(B * T, -1)
    x = x64.reshape(B * T, -1)
    return (g @ W64).reshape(B, T, -1), g.T @ x, g.sum(axis=0)
