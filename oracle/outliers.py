"""FP16 outlier side path: the largest-magnitude weights kept in fp16, the rest in INT4.

TEST INFRASTRUCTURE: see the package docstring for who may import this.

Follows the mhpq.cn notes, section 2.2 ("third line": outlier handling): find the
top 0.1% of the weights by magnitude, move them into an FP16 sub-tensor, quantize
everything else to INT4, and merge the two with where(mask, fp16_weight,
int4_weight), which needs no change to the rest of the engine.

Readings where the page leaves a step open (taken identically by the library):
  O1 the ranking key is |W'| = |W / s|, the value the INT4 grid has to cover
     (|W| when there is no AWQ scale), as one correctly rounded fp64 division.
     For fp16 W and s that division keeps the order of the exact quotients and
     keeps distinct quotients distinct, so the ranking is the exact one;
  O2 the number of kept weights is a parameter; the page's share is
     round(0.001 * N * K) per matrix (``page_count``);
  O3 ties at the threshold go to the lower flat index n * K + k;
  O4 the kept value is the original fp16 W[n][k].  The INT4 side quantizes W'
     with the kept positions set to 0: they drop out of the group range (which
     always contains 0), and their code comes out as the zero point, so the
     INT4 side contributes exactly 0 there;
  O5 the merged weight is W_hat = where(mask, W, (q - z) * scale * s); the
     sparse tensor is stored row-compressed: row_ptr int32 [N + 1], col int32
     and val fp16 in (row, column) order.
The page's figure that the fp16 part is 0.3% of the parameters does not follow
from a 0.1% share and is not reproduced.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .quantizer import NonFiniteInput, QuantResult, quantize, quantize_symmetric


def page_count(N: int, K: int) -> int:
    """The page's 0.1% share of an N x K matrix, N*K/1000 rounded half up (O2)."""
    return (N * K + 500) // 1000


def ranking_keys(W: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    """|W / s| in fp64 (O1)."""
    Wd = np.asarray(W, dtype=np.float16).astype(np.float64)
    if s is not None:
        Wd = Wd / np.asarray(s, dtype=np.float16).astype(np.float64)[None, :]
    return np.abs(Wd)


def select(W: np.ndarray, s: np.ndarray | None, count: int) -> np.ndarray:
    """Boolean mask of the `count` largest |W'|, ties to the lower flat index (O1, O3)."""
    N, K = W.shape
    if not 0 <= count <= N * K:
        raise ValueError("count must be in 0 .. N*K")
    key = ranking_keys(W, s).ravel()
    order = np.lexsort((np.arange(N * K), -key))    # by key descending, then index ascending
    mask = np.zeros(N * K, dtype=bool)
    mask[order[:count]] = True
    return mask.reshape(N, K)


@dataclass
class OutlierResult:
    quant: QuantResult       # the INT4 side (codes, scales, zero points)
    mask: np.ndarray         # bool [N][K]: kept in fp16
    row_ptr: np.ndarray      # int32 [N + 1]
    col: np.ndarray          # int32 [count]
    val: np.ndarray          # float16 [count]


def quantize_with_outliers(W: np.ndarray, s: np.ndarray | None, count: int,
                           symmetric: bool = False, granularity: str = "group",
                           bits: int = 4) -> OutlierResult:
    """Split W into `count` fp16 outliers and an INT4 remainder (O1-O5), the remainder on
    the symmetric grid or at an asymmetric granularity (group, channel or tensor); with
    bits = 8 the remainder takes INT8 codes instead (the same O1-O5 on the 0..255 grid)."""
    if symmetric and bits != 4:
        raise ValueError("the symmetric grid is INT4 only")
    W = np.asarray(W)
    if not np.all(np.isfinite(W.astype(np.float64))):
        raise NonFiniteInput("non-finite W (kept weights included)")   # R9
    mask = select(W, s, count)
    rest = np.where(mask, np.float16(0), W).astype(np.float16)        # O4
    quant = quantize_symmetric(rest, s) if symmetric else quantize(rest, s, granularity, bits)
    rows, cols = np.nonzero(mask)                                      # row-major order (O5)
    row_ptr = np.zeros(W.shape[0] + 1, dtype=np.int64)
    np.add.at(row_ptr, rows + 1, 1)
    return OutlierResult(quant, mask, np.cumsum(row_ptr).astype(np.int32),
                         cols.astype(np.int32), W[rows, cols].astype(np.float16))


def merged_weight(res: OutlierResult, W: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    """W_hat = where(mask, W, (q - z) * scale * s) in fp64 (O5)."""
    from .matmul import dequantize
    deq = dequantize(res.quant.q, res.quant.scales, res.quant.zeros, s)
    return np.where(res.mask, np.asarray(W, dtype=np.float16).astype(np.float64), deq)


def gemm(X: np.ndarray, res: OutlierResult, W: np.ndarray, s: np.ndarray | None) -> np.ndarray:
    """Y = X . W_hat^T in fp64 with the merged weight (the page's where-merge, then a matmul)."""
    return np.asarray(X).astype(np.float64) @ merged_weight(res, W, s).T   # X: fp16 or exact fp64
