"""GPTQ-style quantizer producing the same packed INT4 format (an alternative to ``quantize``).

TEST INFRASTRUCTURE: see the package docstring for who may import this.

Follows aiwing.uk ch.22 sec.22.3, "GPTQ (2022): Hessian-based layer-wise quantization":
for a layer's weights W, find the quantized W_hat minimising ||W X - W_hat X||_F^2, X the
layer's input activations on a little calibration data; the Hessian H = 2 X X^T decides
the quantization order and the error compensation -- after a weight is quantized, its
error is spread over the not yet quantized weights of the same row (the Optimal Brain
Compression idea).

Readings where the page leaves a step open (taken identically by the library):
  Q1 the calibration activations are n rows of K features (the page's X is their
     transpose), so H = 2 X^T X (K x K).  With an AWQ scale s the quantized tensor is
     W' = W / s (reading R8) and its input is X diag(s): H = 2 (X s)^T (X s);
  Q2 damping: lambda * mean(diag H) is added to the diagonal (lambda = 0.01 by
     default), so that H is invertible with fewer samples than features;
  Q3 order: columns in their natural order 0 .. K-1 (the packed format ties each
     group to 128 consecutive columns, which a reordering would break);
  Q4 compensation with the upper Cholesky factor U of H^-1 (H^-1 = U^T U): for column k,
     err = (w_k - dequant(q_k)) / U[k][k] and w_j -= err * U[k][j] for every j > k;
  Q5 a group's scale and zero point are formed, by the rules R3-R7, from the current
     (already compensated) weights of the group when its first column is reached; later
     columns of the group are then coded against them, clamped to 0..15.
All arithmetic is fp64; codes, scales and zero points come out in ``QuantResult``.
"""
from __future__ import annotations

import numpy as np

from .quantizer import GROUP, QMAX, NonFiniteInput, QuantResult, ScaleOverflow, round_up_fp16

DAMP = 0.01


def hessian(Xcal: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    """H = 2 (X s)^T (X s) in fp64 (Q1)."""
    Xd = np.asarray(Xcal).astype(np.float64)
    if s is not None:
        Xd = Xd * np.asarray(s, dtype=np.float16).astype(np.float64)[None, :]
    return 2.0 * (Xd.T @ Xd)


def inverse_cholesky_upper(H: np.ndarray, damp: float = DAMP) -> np.ndarray:
    """U upper triangular with (H + damp * mean(diag H) I)^-1 = U^T U (Q2, Q4)."""
    K = H.shape[0]
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(K)
    Hinv = np.linalg.inv(Hd)
    Hinv = (Hinv + Hinv.T) / 2.0           # inv() leaves rounding-level asymmetry
    return np.linalg.cholesky(Hinv).T


def group_params(wg: np.ndarray):
    """Scale (fp16, rounded up) and zero point of groups (rows of wg) by R3-R7."""
    mn = np.minimum(wg.min(axis=1), 0.0)
    mx = np.maximum(wg.max(axis=1), 0.0)
    rng = mx - mn
    scale16 = round_up_fp16(rng / QMAX)
    if not np.all(np.isfinite(scale16)):
        raise ScaleOverflow("group scale exceeds the fp16 range")
    live = rng > 0
    scale = np.where(live, scale16.astype(np.float64), 1.0)
    z = np.where(live, np.rint(-mn / scale), 0.0)
    return np.where(live, scale16, np.float16(0)).astype(np.float16), z, scale, live


def quantize_gptq(W: np.ndarray, s: np.ndarray | None, Xcal: np.ndarray,
                  damp: float = DAMP) -> QuantResult:
    """GPTQ over fp16 W[N][K] with calibration activations Xcal[n][K] (Q1-Q5)."""
    W = np.asarray(W)
    N, K = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    Wp = W.astype(np.float64)
    if s is not None:
        Wp = Wp / np.asarray(s, dtype=np.float16).astype(np.float64)[None, :]
    if not np.all(np.isfinite(Wp)):
        raise NonFiniteInput("non-finite W or s, or s <= 0")
    U = inverse_cholesky_upper(hessian(Xcal, s), damp)
    G = K // GROUP
    q = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, G), dtype=np.float16)
    zeros = np.zeros((N, G), dtype=np.float16)
    for g in range(G):
        k0 = g * GROUP
        sc16, z, scale, live = group_params(Wp[:, k0:k0 + GROUP])
        scales[:, g] = sc16
        zeros[:, g] = z.astype(np.int64).astype(np.float16)
        for k in range(k0, k0 + GROUP):
            code = np.where(live, np.clip(np.rint(Wp[:, k] / scale) + z, 0, QMAX), 0.0)
            q[:, k] = code
            deq = np.where(live, (code - z) * scale, 0.0)
            err = (Wp[:, k] - deq) / U[k, k]
            Wp[:, k + 1:] -= np.outer(err, U[k, k + 1:])
    return QuantResult(q=q, scales=scales, zeros=zeros)


def layer_loss(W: np.ndarray, s: np.ndarray | None, res: QuantResult, Xcal: np.ndarray) -> float:
    """||W X - W_hat X||_F^2 with the dequantized W_hat (the page's objective)."""
    from .matmul import dequantize
    Wh = dequantize(res.q, res.scales, res.zeros, s)
    D = (np.asarray(W).astype(np.float64) - Wh) @ np.asarray(Xcal).astype(np.float64).T
    return float(np.sum(D * D))
