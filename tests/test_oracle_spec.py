"""Pins for the speculative-verification oracle (aiwing.uk ch.22 sec.22.1).

V1  the page's expected-tokens formula (1 - a^(K+1)) / (1 - a), at its worked example
    a = 0.8, K = 4 (3.36), by Monte Carlo with drafts drawn from p_draft;
V2  the page's losslessness statement: the first token emitted follows p_target
    (chi-square goodness of fit), and so does the next one after an acceptance;
V3  special cases: p_draft = p_target accepts every draft; p_draft(x) = 0 accepts;
    p_target(x) = 0 < p_draft(x) rejects for every u > 0;
V4  the fixed-point draw against an exact rational inverse CDF where the fixed point
    is exact (dyadic weights, u on the 2^-32 grid), and its end points;
V5  the corrected residual on non-dyadic fp32 rows: its weights are exactly
    floor(2^40 * max(0, p_target - p_draft)) in rationals (the page's difference in
    fixed point), and the token drawn after a rejection, over a grid of 2^16 uniforms,
    follows normalize(max(0, p_target - p_draft)) within the grid's and the fixed
    point's total-variation bound.
Mutation tests swap the acceptance ratio (V1 and V2 catch it) and take the residual
on the fixed-point values, max(0, fx(p_target) - fx(p_draft)) (V5 catches it).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import spec


def _pair(alpha, V=8, seed=0):
    """p, q over V tokens with sum_x min(p, q) = alpha."""
    rng = np.random.default_rng(seed)
    base = rng.dirichlet(np.ones(V))
    extra_p = np.zeros(V)
    extra_q = np.zeros(V)
    extra_p[: V // 2] = rng.dirichlet(np.ones(V // 2))
    extra_q[V // 2:] = rng.dirichlet(np.ones(V - V // 2))
    p = alpha * base + (1 - alpha) * extra_p
    q = alpha * base + (1 - alpha) * extra_q
    assert abs(np.minimum(p, q).sum() - alpha) < 1e-9
    return p.astype(np.float32), q.astype(np.float32)


def _run(p, q, K, trials, seed, verify=spec.verify):
    rng = np.random.default_rng(seed)
    V = p.shape[0]
    pt = np.tile(p, (K + 1, 1))
    pd = np.tile(q, (K, 1))
    qn = q.astype(np.float64) / q.astype(np.float64).sum()
    out = []
    for _ in range(trials):
        draft = rng.choice(V, size=K, p=qn)
        u = rng.random(K).astype(np.float32)
        us = np.float32(rng.random())
        n, tok = verify(pt, pd, draft, u, us)
        first = int(draft[0]) if n > 0 else tok
        second = (int(draft[1]) if n > 1 else tok) if n > 0 else None
        out.append((n, tok, first, second))
    return out


def test_v1_expected_tokens_worked_example():
    alpha, K = 0.8, 4
    expected = (1 - alpha ** (K + 1)) / (1 - alpha)
    assert abs(expected - 3.3616) < 1e-12      # the page's "about 3.36"
    p, q = _pair(alpha)
    res = _run(p, q, K, 20000, seed=1)
    tokens = np.array([n + 1 for n, _, _, _ in res], dtype=np.float64)
    se = tokens.std() / np.sqrt(len(tokens))
    assert abs(tokens.mean() - expected) < 4 * se + 1e-3, (tokens.mean(), expected)


def _chi2(counts, probs):
    n = counts.sum()
    e = probs / probs.sum() * n
    return float(((counts - e) ** 2 / e).sum())


def test_v2_lossless_first_and_second_token():
    p, q = _pair(0.6, V=6, seed=3)
    res = _run(p, q, 3, 40000, seed=2)
    first = np.bincount([f for _, _, f, _ in res], minlength=6)
    second = np.bincount([s for _, _, _, s in res if s is not None], minlength=6)
    # chi-square, 5 degrees of freedom: P(chi2 > 25.7) = 1e-4
    assert _chi2(first, p.astype(np.float64)) < 25.7
    assert _chi2(second, p.astype(np.float64)) < 25.7


def test_v3_special_cases():
    V, K = 5, 3
    p = np.array([0.1, 0.2, 0.3, 0.4, 0.0], np.float32)
    pt = np.tile(p, (K + 1, 1))
    draft = np.array([3, 1, 2])
    u = np.array([0.999, 0.5, 0.9999], np.float32)
    n, tok = spec.verify(pt, pt[:K], draft, u, 0.25)
    assert n == K and tok == spec.draw(p, 0.25)          # p_draft = p_target: all accepted
    pd = pt[:K].copy()
    pd[0, 3] = 0                                          # p_draft(x) = 0: accepted
    assert spec.verify(pt, pd, draft, u, 0.25)[0] == K
    draft2 = np.array([4, 1, 2])                          # p_target(4) = 0 < p_draft(4)
    pd2 = pt[:K].copy()
    pd2[0] = [0.1, 0.1, 0.1, 0.1, 0.6]
    for uu in (1e-30, 0.5, 0.999):
        n, tok = spec.verify(pt, pd2, draft2, np.array([uu, 0.5, 0.5], np.float32), 0.3)
        assert n == 0
        # the corrected distribution max(0, p - q) has mass only on tokens 1, 2, 3
        assert tok in (1, 2, 3)


def test_v4_fixed_point_draw_exact_cases():
    rng = np.random.default_rng(5)
    for _ in range(200):
        V = int(rng.integers(1, 12))
        w = rng.integers(0, 17, size=V) / 16.0               # dyadic: exact in fixed point
        if w.sum() == 0:
            assert spec.draw(w, 0.5) == -1
            continue
        u = float(rng.integers(0, 2 ** 24)) / 2 ** 24        # on the 2^-32 grid, exact fp32
        # exact inverse CDF: smallest x with sum_{<= x} w > u * sum w
        target = Fraction(u) * sum(Fraction(x) for x in w)
        acc, want = Fraction(0), None
        for x, v in enumerate(w):
            acc += Fraction(v)
            if acc > target:
                want = x
                break
        assert spec.draw(w, np.float32(u)) == want
    w = np.array([0.0, 0.0, 0.5, 0.0, 0.25, 0.0], np.float32)
    assert spec.draw(w, 0.0) == 2                            # first token with mass
    assert spec.draw(w, np.float32(1 - 2 ** -24)) == 4      # last token with mass


def test_v4_residual_draw_exact_cases():
    """The token drawn after a rejection, for dyadic p_target / p_draft (exact in fixed
    point) and u on the 2^-32 grid, against the exact rational inverse CDF of the page's
    corrected distribution max(0, p_target - p_draft)."""
    rng = np.random.default_rng(8)
    checked = 0
    for _ in range(300):
        V = int(rng.integers(2, 10))
        pt = (rng.integers(0, 33, size=V) / 32.0).astype(np.float32)
        pd = (rng.integers(0, 33, size=V) / 32.0).astype(np.float32)
        x = int(rng.integers(0, V))
        if not (pt[x] < pd[x]):
            continue                                         # need a rejection at u = 1 - 2^-24
        u = float(rng.integers(0, 2 ** 24)) / 2 ** 24
        res = [max(Fraction(float(a)) - Fraction(float(b)), Fraction(0)) for a, b in zip(pt, pd)]
        n, tok = spec.verify(np.stack([pt, pt]), pd[None], np.array([x]),
                             np.array([1 - 2 ** -24], np.float32), np.float32(u))
        assert n == 0
        if sum(res) == 0:                                    # S4: the target row instead
            assert tok == spec.draw(pt, np.float32(u))
            continue
        target = Fraction(u) * sum(res)
        acc = Fraction(0)
        for y, v in enumerate(res):
            acc += v
            if acc > target:
                break
        assert tok == y
        checked += 1
    assert checked > 50


def test_mutation_swapped_ratio_breaks_v1_and_v2():
    def swapped(pt, pd, draft, u_acc, u_s):
        pt = np.asarray(pt, np.float64)
        pd = np.asarray(pd, np.float64)
        K = pd.shape[0]
        for i in range(K):
            x = int(draft[i])
            if not (float(u_acc[i]) * pt[i, x] <= pd[i, x]):    # planted: p_draft / p_target
                tok = spec.draw(np.maximum(pt[i] - pd[i], 0.0), u_s)
                return i, (tok if tok >= 0 else spec.draw(pt[i], u_s))
        return K, spec.draw(pt[K], u_s)
    p, q = _pair(0.6, V=6, seed=3)
    res = _run(p, q, 3, 20000, seed=2, verify=swapped)
    first = np.bincount([f for _, _, f, _ in res], minlength=6)
    assert _chi2(first, p.astype(np.float64)) > 25.7


def _nondyadic_rows(rng, V):
    """fp32 rows of tail probabilities, log-uniform in 2^-36 .. 2^-12 (the small entries
    of a large vocabulary), where floor(p * 2^40) drops fractional bits.  Exponents are
    at most 24 apart, so the fp64 difference of two entries is exact."""
    pt = np.exp2(rng.uniform(-36, -12, V)).astype(np.float32)
    pd = np.exp2(rng.uniform(-36, -12, V)).astype(np.float32)
    return pt, pd


def _check_v5_weights(seed=9, rows=400):
    """V5, first half: the residual weights in exact rationals.  Returns how many entries
    differ from the fixed-point difference max(0, fx(p_target) - fx(p_draft))."""
    rng = np.random.default_rng(seed)
    differ = 0
    for _ in range(rows):
        V = int(rng.integers(2, 9))
        pt, pd = _nondyadic_rows(rng, V)
        got = spec.residual_weights(pt.astype(np.float64), pd.astype(np.float64))
        for x in range(V):
            d = max(Fraction(float(pt[x])) - Fraction(float(pd[x])), Fraction(0))
            want = (d * 2 ** 40).__floor__()
            assert int(got[x]) == want, (pt[x], pd[x], int(got[x]), want)
            fx_t = (Fraction(float(pt[x])) * 2 ** 40).__floor__()
            fx_d = (Fraction(float(pd[x])) * 2 ** 40).__floor__()
            differ += want != max(fx_t - fx_d, 0)
    return differ


def test_v5_residual_weights_exact():
    # the pin tells the page's form apart from the fixed-point difference
    assert _check_v5_weights() > 50


def test_mutation_fixed_point_difference_fails_v5(monkeypatch):
    monkeypatch.setattr(spec, "residual_weights", lambda a, b: np.maximum(
        spec.fixed_weights(a) - spec.fixed_weights(b), 0))
    with pytest.raises(AssertionError):
        _check_v5_weights()


def test_v5_residual_draw_follows_corrected_distribution():
    """Token after a rejection at position 0, for u = j / 2^16 (j = 0 .. 2^16 - 1): its
    histogram against the exact normalize(max(0, p_target - p_draft)).  Each grid point
    stands for 2^16 points of the 2^-32 grid, so the histogram is within V * 2^-16 of the
    draw's own distribution in total variation; the fixed point adds at most V * 2^-40
    over the residual's mass."""
    rng = np.random.default_rng(10)
    for _ in range(3):
        V = int(rng.integers(3, 8))
        pt, pd = _nondyadic_rows(rng, V)
        x = int(np.argmax(pd.astype(np.float64) - pt.astype(np.float64)))   # pt[x] < pd[x]
        res = [max(Fraction(float(a)) - Fraction(float(b)), Fraction(0)) for a, b in zip(pt, pd)]
        mass = sum(res)
        exact = [float(r / mass) for r in res]
        counts = np.zeros(V)
        n_grid = 2 ** 16
        for j in range(n_grid):
            n, tok = spec.verify(np.stack([pt, pt]), pd[None], np.array([x]),
                                 np.array([1 - 2 ** -24], np.float32), np.float32(j / n_grid))
            assert n == 0
            counts[tok] += 1
        tv = 0.5 * np.abs(counts / n_grid - np.array(exact)).sum()
        assert tv <= V * 2.0 ** -16 + V * 2.0 ** -40 / float(mass), tv
