"""Exact-rational brute force for tiny inputs (pins for the fp64 oracle).

Nothing here is fast; it exists so the oracle can be checked against
definitions evaluated exactly:
  * ``gemm_exact``: Y = X . W_hat^T by a triple loop in ``fractions.Fraction``,
    with W_hat = (q - z) * scale * s (aiwing.uk ch.22 sec.22.3, AWQ equation and
    weight-only paragraph);
  * ``smallest_fp16_at_least``: exhaustive search over every finite fp16;
  * ``nearest_code``: the code minimising |t - (c - z)| over all 16 codes, ties
    going to the even (c - z), i.e. round-half-to-even of t followed by a shift
    and a clamp (readings R6, R7).
TEST INFRASTRUCTURE: see the package docstring for who may import this.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_ALL_FP16 = None


def _fp16_sorted_positive() -> list:
    global _ALL_FP16
    if _ALL_FP16 is None:
        bits = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. largest finite
        vals = bits.view(np.float16)
        _ALL_FP16 = [(Fraction(float(v)), int(b)) for v, b in zip(vals, bits)]
    return _ALL_FP16


def smallest_fp16_at_least(v: Fraction):
    """(value, bits) of the least finite fp16 >= v >= 0, or None past the range."""
    for val, bits in _fp16_sorted_positive():   # ascending order
        if val >= v:
            return val, bits
    return None


def nearest_code(t: Fraction, z: int, qmax: int = 15) -> int:
    """argmin over c in 0..qmax of |t - (c - z)|; a tie is resolved to the even (c - z)."""
    best = None
    for c in range(qmax + 1):
        d = abs(t - (c - z))
        key = (d, (c - z) % 2)   # distance first, then prefer even (c - z)
        if best is None or key < best[0]:
            best = (key, c)
    # the codes 0..qmax are a window of integers, so the unclamped nearest value
    # outside the window lands on the nearer end: that is the clamp.
    return best[1]


def gemm_exact(X, q, scales, zeros, s=None):
    """Exact Y[M][N] as nested lists of Fractions."""
    X = np.asarray(X)
    M, K = X.shape
    N = q.shape[0]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 128
                w = (Fraction(int(q[n, k])) - Fraction(float(zeros[n, g]))) * Fraction(float(scales[n, g]))
                if s is not None:
                    w *= Fraction(float(s[k]))
                acc += Fraction(float(X[m, k])) * w
            row.append(acc)
        out.append(row)
    return out
