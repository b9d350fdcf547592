"""fp64 reference for the weight-only dequantize-then-matmul.

aiwing.uk ch.22 sec.22.3 (weight-only quantization paragraph): activations stay
in FP16; the product is the plain matmul against the dequantized weights, which
a fused mixed-precision kernel only computes faster.  So the reference is that
definition written out:  W_hat[n][k] = (q[n][k] - z[n][g]) * scale[n][g] * s[k]
(AWQ equation of the same section, reading R6), and Y = X . W_hat^T.
The mhpq.cn notes (sec.2.1) write the product as W times X; with W stored
[N][K] (output x input features) and X as [M][K] rows that is Y = X W_hat^T.
TEST INFRASTRUCTURE: see the package docstring for who may import this.
"""
from __future__ import annotations

import numpy as np

_GROUP = 128


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               s: np.ndarray | None = None) -> np.ndarray:
    """W_hat[N][K] in fp64 from codes q[N][K] and per-group scales/zeros [N][K/128]."""
    q = np.asarray(q)
    N, K = q.shape
    g = np.arange(K) // _GROUP
    sc = np.asarray(scales, dtype=np.float64)[:, g]
    zr = np.asarray(zeros, dtype=np.float64)[:, g]
    w = (q.astype(np.float64) - zr) * sc      # (q - z) is a small integer: exact
    if s is not None:
        w = w * np.asarray(s, dtype=np.float64)[None, :]
    return w


def gemm(X: np.ndarray, q: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
         s: np.ndarray | None = None) -> np.ndarray:
    """Y[M][N] = X[M][K] . W_hat^T in fp64 (X given in fp16)."""
    X = np.asarray(X)
    if X.ndim != 2 or X.shape[1] != q.shape[1]:
        raise ValueError("X must be [M][K]")
    return X.astype(np.float64) @ dequantize(q, scales, zeros, s).T
