"""fp64 reference quantizer: weight-only asymmetric INT4, groups of 128, AWQ pre-scale.

Follows, in order:
  * aiwing.uk ch.22 sec.22.3, AWQ equation: the weight is divided by the
    per-input-channel activation magnitude s before quantization and the
    dequantized value is multiplied by s again (W_hat = quant(W/s) * s);
  * discosf.com tutorial sec.2.1: quant() finds a scale and a zero point that
    map the float range of a group onto the integer range; one scale/zero pair
    per group of 128 elements.
Readings R1-R9 (package docstring) fix what the pages leave open.
TEST INFRASTRUCTURE: see the package docstring for who may import this.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 128   # elements per quantization group along K (discosf sec.2.1)
QMAX = 15     # unsigned 4-bit code range 0..15 (reading R1)
SYM_QMAX = 7  # symmetric signed grid -7..7 (mhpq.cn notes sec.2.1: INT4 max +-7)
SYM_ZERO = 8  # its fixed zero point: stored code = signed code + 8, in 1..15


class OracleError(ValueError):
    pass


class NonFiniteInput(OracleError):
    """W or s holds NaN/Inf, or some s <= 0 (reading R9)."""


class ScaleOverflow(OracleError):
    """A group's scale, rounded up to fp16, exceeds the largest finite fp16 (reading R9)."""


@dataclass
class QuantResult:
    q: np.ndarray       # uint8 [N][K], codes 0..15
    scales: np.ndarray  # float16 [N][K/128]
    zeros: np.ndarray   # float16 [N][K/128], integer-valued 0..15


def round_up_fp16(v: np.ndarray) -> np.ndarray:
    """Smallest fp16 value >= v, for float64 v >= 0 (reading R5); +inf past 65504.

    Done as: round to nearest fp16 (NumPy's correctly rounded float64 -> float16
    cast), then step one fp16 ulp up wherever the nearest value fell below v.
    """
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)
    below = h.astype(np.float64) < v
    h[below] = np.nextafter(h[below], np.float16(np.inf))
    return h


GRANULARITIES = ("group", "channel", "tensor")


def _extremes(Wp: np.ndarray, granularity: str):
    """min and max of W' over what one scale covers, per (row, group slot) [N][G]: the
    group itself, its whole row (channel), or the whole tensor (discosf sec.2.1)."""
    N, K = Wp.shape
    G = K // GROUP
    if granularity == "group":
        Wg = Wp.reshape(N, G, GROUP)
        return Wg.min(axis=2), Wg.max(axis=2)
    if granularity == "channel":
        return (np.repeat(Wp.min(axis=1, keepdims=True), G, axis=1),
                np.repeat(Wp.max(axis=1, keepdims=True), G, axis=1))
    return np.full((N, G), Wp.min()), np.full((N, G), Wp.max())


def quantize(W: np.ndarray, s: np.ndarray | None = None, granularity: str = "group",
             bits: int = 4) -> QuantResult:
    """Quantize fp16 ``W[N][K]`` (optionally divided by fp16 ``s[K]`` first) to INT4 groups.

    ``granularity`` (discosf sec.2.1: per-tensor, per-channel or per-group scales) picks
    the range a scale and zero point cover: each group of 128 (reading R2), each row
    (output channel), or the whole tensor.  The coarser ones keep the per-group storage:
    every group of a row (or of the tensor) carries the same scale and zero point.

    ``bits`` = 8 is the INT8 (W8A16) variant of the same readings: codes 0..255, so
    scale = range / 255 (aiwing sec.22.3's table: INT8 at one byte per parameter)."""
    if granularity not in GRANULARITIES:
        raise ValueError(f"granularity must be one of {GRANULARITIES}")
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    qmax = (1 << bits) - 1
    W = np.asarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise TypeError("W must be a 2-D float16 array")
    N, K = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    Wd = W.astype(np.float64)
    if s is None:
        sd = np.ones(K, dtype=np.float64)
    else:
        s = np.asarray(s)
        if s.dtype != np.float16 or s.shape != (K,):
            raise TypeError("s must be a float16 array of length K")
        sd = s.astype(np.float64)
    if not np.all(np.isfinite(Wd)) or not np.all(np.isfinite(sd)) or not np.all(sd > 0):
        raise NonFiniteInput("non-finite W or s, or s <= 0")

    # AWQ step (aiwing sec.22.3): W' = W / s, one correctly rounded fp64 division per element.
    Wp = Wd / sd[None, :]
    G = K // GROUP
    Wg = Wp.reshape(N, G, GROUP)

    # Range of each group (or row, or tensor), widened to contain 0 (R3);
    # scale = range / 15 rounded up to fp16 (R4, R5).
    lo, hi = _extremes(Wp, granularity)
    mn = np.minimum(lo, 0.0)
    mx = np.maximum(hi, 0.0)
    rng = mx - mn
    scale16 = round_up_fp16(rng / qmax)
    if not np.all(np.isfinite(scale16)):
        raise ScaleOverflow("group scale exceeds the fp16 range")
    scale = scale16.astype(np.float64)

    live = rng > 0   # an all-zero group keeps scale 0, zero point 0, codes 0 (R9)
    safe = np.where(live, scale, 1.0)
    # Zero point: the integer nearest to -min/scale (R6); lies in 0..qmax because scale >= range/qmax.
    z = np.where(live, np.rint(-mn / safe), 0.0)
    # Codes: rint (ties to even) of W'/scale, then shifted by z and clamped to 0..qmax (R7).
    t = np.rint(Wg / safe[:, :, None]) + z[:, :, None]
    q = np.where(live[:, :, None], np.clip(t, 0, qmax), 0.0)

    return QuantResult(
        q=q.reshape(N, K).astype(np.uint8),
        scales=np.where(live, scale16, np.float16(0)).astype(np.float16),
        zeros=z.astype(np.int64).astype(np.float16),   # integer -> fp16: never a negative zero
    )


def quantize_symmetric(W: np.ndarray, s: np.ndarray | None = None) -> QuantResult:
    """Symmetric variant of ``quantize``: signed codes -7..7 around a fixed zero point.

    Steps, in the same order as ``quantize``:
      * W' = W / s (aiwing sec.22.3's AWQ pre-scale), fp64;
      * per group of 128 (discosf sec.2.1), the scale maps the largest magnitude
        onto 7, the top of the signed 4-bit grid of the mhpq.cn notes sec.2.1:
        scale = max|W'| / 7 rounded UP to fp16 (as R5: so |W' / scale| <= 7 and
        no code is ever clamped);
      * signed code c = rint(W' / scale) (ties to even), clamped to -7..7;
      * stored as the unsigned code c + 8 (1..15) with zero point 8, so that the
        library's dequantization (q - z) * scale * s applies unchanged.
    An all-zero group stores scale 0, codes 8 and zero point 8 (so q - z = 0).
    """
    W = np.asarray(W)
    if W.dtype != np.float16 or W.ndim != 2:
        raise TypeError("W must be a 2-D float16 array")
    N, K = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    Wd = W.astype(np.float64)
    if s is None:
        sd = np.ones(K, dtype=np.float64)
    else:
        s = np.asarray(s)
        if s.dtype != np.float16 or s.shape != (K,):
            raise TypeError("s must be a float16 array of length K")
        sd = s.astype(np.float64)
    if not np.all(np.isfinite(Wd)) or not np.all(np.isfinite(sd)) or not np.all(sd > 0):
        raise NonFiniteInput("non-finite W or s, or s <= 0")
    Wp = Wd / sd[None, :]
    G = K // GROUP
    Wg = Wp.reshape(N, G, GROUP)
    amax = np.abs(Wg).max(axis=2)
    scale16 = round_up_fp16(amax / SYM_QMAX)
    if not np.all(np.isfinite(scale16)):
        raise ScaleOverflow("group scale exceeds the fp16 range")
    live = amax > 0
    safe = np.where(live, scale16.astype(np.float64), 1.0)
    c = np.clip(np.rint(Wg / safe[:, :, None]), -SYM_QMAX, SYM_QMAX)
    c = np.where(live[:, :, None], c, 0.0)
    return QuantResult(
        q=(c + SYM_ZERO).reshape(N, K).astype(np.uint8),
        scales=np.where(live, scale16, np.float16(0)).astype(np.float16),
        zeros=np.full((N, G), SYM_ZERO, dtype=np.float16),
    )
