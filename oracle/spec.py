"""Speculative-sampling verification (the accept / reject step after the verify pass).

TEST INFRASTRUCTURE: see the package docstring for who may import this.

Follows aiwing.uk ch.22 sec.22.1, "verification: accept-reject sampling":
  * for each draft token x_i (i = 0 .. K-1), accept it if u_i <= p_target(x_i) /
    p_draft(x_i), u_i ~ Uniform(0, 1); stop at the first rejection;
  * on a rejection at position i, draw one token from the corrected
    distribution normalize(max(0, p_target_i - p_draft_i)) and discard the
    later drafts;
and the expected-tokens formula of the same section, (1 - a^(K+1)) / (1 - a),
which counts a (K+1)-th token: when all K drafts are accepted, one more token
is drawn from the target distribution of position K.

Readings where the page leaves a step open (taken identically by the library):
  S1 inputs are probabilities (fp32, rows of V entries, not necessarily
     normalised); entries below 0 or NaN count as 0;
  S2 the acceptance test is the exact comparison u * p_draft <= p_target in
     fp64 (the product of two fp32 values is exact there), so p_draft = 0
     always accepts;
  S3 a draw is an inverse-CDF draw in fixed point, fx(p) = floor(p * 2^40).  The
     target row's weights are fx(p_target); the corrected residual's are
     fx(max(0, p_target - p_draft)): the page's difference, formed in fp64 from the
     two fp32 values (exact whenever their exponents are at most 29 apart, else
     rounded once to nearest), then taken to fixed point.  Weights are
     summed exactly in integers; with u' the sampling uniform, T = (floor(u' *
     2^32) * S) >> 32 for S = sum of the weights, and the token is the smallest
     x whose inclusive prefix sum exceeds T.  Sums are exact, so the order of
     summation cannot change the token; the fixed point moves the drawn
     distribution by at most about V * 2^-40 in total variation.  (Rows are
     taken to sum to less than 2^12, so every partial sum stays below 2^52.)
  S4 if the corrected residual has no mass in fixed point, the draw uses the
     target row of that position instead; if that has none either, the token
     is -1;
  S5 a draft id outside 0 .. V-1 is rejected; u' is clamped to [0, 1) on the
     2^-32 grid (NaN counts as 0).
"""
from __future__ import annotations

import numpy as np

FIX_BITS = 40   # fixed-point resolution of the sampling weights (S3)
U_BITS = 32     # resolution of the sampling uniform (S3)


def _clean(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    return np.where(p > 0, p, 0.0)          # NaN and negatives count as 0 (S1)


def fixed_weights(w: np.ndarray) -> np.ndarray:
    """fx(w) = floor(w * 2^40) for w >= 0, as int64 (S3)."""
    return np.floor(np.asarray(w, dtype=np.float64) * float(2 ** FIX_BITS)).astype(np.int64)


def draw_fixed(wi, u: float) -> int:
    """Inverse-CDF draw from non-negative integer weights (S3); -1 if they have no mass."""
    wi = [int(v) for v in wi]
    S = sum(wi)
    if S == 0:
        return -1
    uf = np.float64(np.float32(u))
    ui = int(np.floor(uf * float(2 ** U_BITS))) if uf > 0 else 0     # NaN, negatives: 0
    ui = min(ui, 2 ** U_BITS - 1)                                    # S5: u' < 1
    T = (ui * S) >> U_BITS
    acc = 0
    for x, v in enumerate(wi):
        acc += v
        if acc > T:
            return x
    raise AssertionError("T < S always")


def draw(w: np.ndarray, u: float) -> int:
    """Inverse-CDF draw from probabilities w >= 0 in fixed point (S3); -1 if no mass."""
    return draw_fixed(fixed_weights(w), u)


def residual_weights(pt_row: np.ndarray, pd_row: np.ndarray) -> np.ndarray:
    """The page's corrected residual max(0, p_target - p_draft), in fixed point (S3)."""
    d = np.asarray(pt_row, dtype=np.float64) - np.asarray(pd_row, dtype=np.float64)
    return fixed_weights(np.maximum(d, 0.0))


def verify(p_target: np.ndarray, p_draft: np.ndarray, draft: np.ndarray, u_accept: np.ndarray,
           u_sample: float) -> tuple[int, int]:
    """One sequence.  p_target [K+1][V], p_draft [K][V], draft [K] token ids, u_accept [K],
    u_sample.  Returns (number of accepted drafts, the token drawn after them)."""
    pt = _clean(p_target)
    pd = _clean(p_draft)
    K = pd.shape[0]
    V = pt.shape[1]
    for i in range(K):
        x = int(draft[i])
        u = np.float64(np.float32(u_accept[i]))
        if not (0 <= x < V) or not (u * pd[i, x] <= pt[i, x]):   # rejected (S2, S5)
            tok = draw_fixed(residual_weights(pt[i], pd[i]), u_sample)
            if tok < 0:
                tok = draw(pt[i], u_sample)      # S4
            return i, tok
    return K, draw(pt[K], u_sample)              # all accepted: the bonus token
