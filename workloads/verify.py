"""Seeded synthetic inputs for speculative-sampling verification.

Recipe, per sequence b (all float32 at the end):
  * target logits of each of the K+1 positions: N(0, 2^2) over V tokens, plus
    +6 on 8 tokens drawn uniformly (a peaked next-token distribution);
    p_target = softmax of them;
  * draft logits: the target logits of the same position plus N(0, sigma^2)
    noise (sigma = 1.0 by default), p_draft = softmax of them, so the draft
    model agrees with the target on most of the mass (acceptance rates of
    roughly 0.6 to 0.8, the range the aiwing.uk chapter's section 22.1 uses);
  * draft[b][i]: drawn from p_draft[b][i] (what a draft model emits);
  * u_accept[b][i], u_sample[b]: Uniform[0, 1) float32.
The softmax and the draft draws only build inputs; they are not the
verification step.  Every stream is ``default_rng([1, key, b, ...])``.
"""
from __future__ import annotations

import numpy as np

SEED = 1


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def sequence(key: int, b: int, K: int, V: int, sigma: float = 1.0):
    """Inputs of one sequence: (p_target [K+1][V], p_draft [K][V], draft [K], u_accept [K],
    u_sample)."""
    rng = np.random.default_rng([SEED, key, b])
    logits = rng.standard_normal((K + 1, V)) * 2.0
    for i in range(K + 1):
        logits[i, rng.choice(V, size=min(8, V), replace=False)] += 6.0
    p_target = _softmax(logits).astype(np.float32)
    p_draft = _softmax(logits[:K] + rng.standard_normal((K, V)) * sigma).astype(np.float32)
    cdf = np.cumsum(p_draft.astype(np.float64), axis=1)
    r = rng.random(K) * cdf[:, -1]
    draft = np.array([min(int(np.searchsorted(cdf[i], r[i], side="right")), V - 1)
                      for i in range(K)], dtype=np.int32)
    u_accept = rng.random(K, dtype=np.float32)
    u_sample = np.float32(rng.random(dtype=np.float32))
    return p_target, p_draft, draft, u_accept, u_sample


def batch(key: int, B: int, K: int, V: int, sigma: float = 1.0):
    """B sequences stacked: p_target [B][K+1][V], p_draft [B][K][V], draft [B][K],
    u_accept [B][K], u_sample [B]."""
    seqs = [sequence(key, b, K, V, sigma) for b in range(B)]
    return (np.stack([s[0] for s in seqs]), np.stack([s[1] for s in seqs]).reshape(B, K, V),
            np.stack([s[2] for s in seqs]).reshape(B, K), np.stack([s[3] for s in seqs]).reshape(B, K),
            np.array([s[4] for s in seqs], dtype=np.float32))
