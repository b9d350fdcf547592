"""Seeded synthetic inputs (NumPy ``default_rng``), in the value structure the pages describe.

Recipe (all draws float32, then cast to fp16 once at the end):
  * W[N][K]: N(0, 0.02^2) (0.02 is the standard deviation).  The rows are
    generated in chunks of 256; inside each chunk exactly round(0.001 * 256 * K)
    positions, drawn uniformly without replacement, are multiplied by 10 before
    the cast.  This plants the small fraction of large-magnitude weights the
    mhpq.cn notes (section 2.2, outlier handling) and the aiwing.uk chapter
    (section 22.3, AWQ: a small share of salient weights) talk about.
  * s[K]: LogNormal(mu=0, sigma=0.5) per input channel (AWQ scale), fp16.
  * X[M][K]: N(0, 1) (fp16, or bf16 bit patterns for the bf16 path).  For the prefill workload, round(0.01 * K) columns drawn
    uniformly without replacement are multiplied by 20 (activation outliers,
    aiwing.uk section 22.3, activation quantization paragraph).
Every stream is ``default_rng([0, key, matrix_index, tensor_id, ...])`` so any
row chunk can be regenerated on its own (sampled full-size checks use this).
"""
from __future__ import annotations

import numpy as np

SEED = 0
ROW_CHUNK = 256
_T_W, _T_S, _T_X, _T_XCOLS = 0, 1, 2, 3


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([SEED, *key])


def _weight_chunk(key: int, mat: int, chunk: int, rows: int, K: int) -> np.ndarray:
    rng = _rng(key, mat, _T_W, chunk)
    w = rng.standard_normal(rows * K, dtype=np.float32)
    w *= np.float32(0.02)
    n_out = int(round(0.001 * rows * K))
    if n_out:
        idx = rng.choice(rows * K, size=n_out, replace=False)
        w[idx] *= np.float32(10.0)
    return w.astype(np.float16).reshape(rows, K)


def weight_rows(key: int, mat: int, N: int, K: int, row0: int, row1: int) -> np.ndarray:
    """Rows [row0, row1) of the weight matrix ``weights(key, mat, N, K)``, regenerated alone."""
    if not (0 <= row0 <= row1 <= N):
        raise ValueError("row range out of bounds")
    out = np.empty((row1 - row0, K), dtype=np.float16)
    c0, c1 = row0 // ROW_CHUNK, (row1 + ROW_CHUNK - 1) // ROW_CHUNK
    for c in range(c0, c1):
        r0, r1 = c * ROW_CHUNK, min(N, (c + 1) * ROW_CHUNK)
        blk = _weight_chunk(key, mat, c, r1 - r0, K)
        a, b = max(r0, row0), min(r1, row1)
        if a < b:
            out[a - row0:b - row0] = blk[a - r0:b - r0]
    return out


def weights(key: int, mat: int, N: int, K: int, threads: int = 1) -> np.ndarray:
    """Full ``W[N][K]`` fp16.  ``threads > 1`` generates chunks in parallel (same values)."""
    out = np.empty((N, K), dtype=np.float16)
    nchunks = (N + ROW_CHUNK - 1) // ROW_CHUNK

    def fill(c: int) -> None:
        r0, r1 = c * ROW_CHUNK, min(N, (c + 1) * ROW_CHUNK)
        out[r0:r1] = _weight_chunk(key, mat, c, r1 - r0, K)

    if threads > 1 and nchunks > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    else:
        for c in range(nchunks):
            fill(c)
    return out


def awq_scales(key: int, mat: int, K: int) -> np.ndarray:
    """AWQ per-input-channel scale s[K] ~ LogNormal(0, 0.5), fp16 (all positive)."""
    rng = _rng(key, mat, _T_S)
    return rng.lognormal(mean=0.0, sigma=0.5, size=K).astype(np.float32).astype(np.float16)


def _activations_f32(key: int, mat: int, M: int, K: int, outliers: bool) -> np.ndarray:
    # one sequential stream: the first rows are the same whatever M is
    x = _rng(key, mat, _T_X).standard_normal((M, K), dtype=np.float32)
    if outliers:
        cols = _rng(key, mat, _T_XCOLS).choice(K, size=int(round(0.01 * K)), replace=False)
        x[:, cols] *= np.float32(20.0)
    return x


def activations(key: int, mat: int, M: int, K: int, outliers: bool = False) -> np.ndarray:
    """X[M][K] fp16 ~ N(0, 1); with ``outliers`` 1% of the columns are scaled by 20.

    Row i does not depend on M, so the M=1 input is the first row of any larger batch.
    """
    return _activations_f32(key, mat, M, K, outliers).astype(np.float16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), rounded to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact float64 values."""
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def activations_bf16(key: int, mat: int, M: int, K: int, outliers: bool = False) -> np.ndarray:
    """The same draws as ``activations``, rounded to bf16 instead: uint16 bit patterns."""
    return to_bf16_bits(_activations_f32(key, mat, M, K, outliers))
