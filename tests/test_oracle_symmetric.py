"""Pins for the oracle's symmetric quantizer (signed -7..7 grid, mhpq.cn notes sec.2.1).

S1  round-trip bound |W' - c * scale| <= scale / 2 for every element (c = q - 8);
S2  exact reconstruction of weights on the symmetric grid;
S3  brute force in exact rationals: the scale is the least fp16 >= max|W'| / 7, and
    every signed code is the nearest of -7..7 to W' / scale (ties to even);
S4  an all-zero group: scale 0, codes 8, zero point 8.
A mutation test plants round-to-nearest for the scale and checks S3's scale
property catches it (on this grid S1 alone would not: a scale half an ulp low
still rounds every code into -7..7 within scale / 2).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import awq_scales, weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _sym_roundtrip_ok(W, s, res):
    Wp = W.astype(np.float64) / (np.ones(W.shape[1]) if s is None else s.astype(np.float64))[None, :]
    c = res.q.astype(np.float64) - 8.0
    sc = np.repeat(res.scales.astype(np.float64), 128, axis=1)
    return not (np.abs(Wp - c * sc) > sc / 2 * (1 + 1e-12) + 1e-300).any()


@pytest.mark.parametrize("awq", [False, True])
def test_s1_roundtrip_bound(awq):
    N, K = 256, 1024
    W = weights(31, 0, N, K)
    s = awq_scales(31, 0, K) if awq else None
    res = oracle.quantize_symmetric(W, s)
    assert res.q.min() >= 1 and res.q.max() <= 15
    assert np.all(res.zeros == 8)
    assert _sym_roundtrip_ok(W, s, res)


@pytest.mark.parametrize("with_s", [False, True])
def test_s2_exact_on_grid(with_s):
    rng = np.random.default_rng(7 + with_s)
    N, K = 32, 512
    G = K // 128
    c = rng.integers(-7, 8, size=(N, G, 128))
    c[:, :, 0] = 7          # the largest magnitude of every group is exactly 7 * scale
    c[:, :, 1] = -7
    m = rng.integers(64, 128, size=(N, G))
    e = rng.integers(-16, -8, size=(N, G))
    scale = np.ldexp(m.astype(np.float64), e)
    wp = (c * scale[:, :, None]).reshape(N, K)
    s = np.ldexp(1.0, rng.integers(-2, 3, size=K)).astype(np.float16) if with_s else None
    W = wp * (s.astype(np.float64)[None, :] if with_s else 1.0)
    W16 = W.astype(np.float16)
    assert np.array_equal(W16.astype(np.float64), W)
    res = oracle.quantize_symmetric(W16, s)
    assert np.array_equal(res.q.astype(np.int64) - 8, c.reshape(N, K))
    assert np.array_equal(res.scales.astype(np.float64), scale)
    assert np.all(res.zeros == 8)
    w_hat = oracle.dequantize(res.q, res.scales, res.zeros, s)
    assert np.array_equal(w_hat, W16.astype(np.float64))


@pytest.mark.parametrize("seed", range(4))
def test_s3_bruteforce_exact(seed):
    rng = np.random.default_rng(100 + seed)
    N, K = 3, 256
    W = (rng.standard_normal((N, K)) * rng.choice([0.01, 1.0, 300.0])).astype(np.float16)
    s = (rng.lognormal(0, 0.5, K)).astype(np.float16) if seed % 2 else None
    res = oracle.quantize_symmetric(W, s)
    for n in range(N):
        for g in range(K // 128):
            cols = range(128 * g, 128 * g + 128)
            wp = [Fraction(float(W[n, k])) / (Fraction(float(s[k])) if s is not None else 1)
                  for k in cols]
            amax = max(abs(v) for v in wp)
            sc = Fraction(float(res.scales[n, g]))
            if amax == 0:
                assert sc == 0 and all(res.q[n, k] == 8 for k in cols)
                continue
            # least fp16 >= amax / 7: sc is an fp16 value >= it, and the next fp16 below is < it
            assert sc >= amax / 7
            below = np.nextafter(np.float16(float(sc)), np.float16(0))
            assert Fraction(float(below)) < amax / 7
            for k, v in zip(cols, wp):
                t = v / sc
                best = min(range(-7, 8), key=lambda cc: (abs(t - cc), cc % 2))
                assert int(res.q[n, k]) - 8 == best, (n, k)


def test_s4_all_zero_group():
    W = np.zeros((16, 256), np.float16)
    W[3, 200] = 1.0
    res = oracle.quantize_symmetric(W, None)
    assert res.scales[0, 0] == 0 and res.scales[3, 0] == 0 and res.scales[3, 1] > 0
    assert np.all(res.q[:, :128] == 8) and np.all(res.zeros == 8)


def test_errors():
    with pytest.raises(oracle.NonFiniteInput):
        oracle.quantize_symmetric(np.full((16, 128), np.inf, np.float16))
    with pytest.raises(oracle.ScaleOverflow):
        oracle.quantize_symmetric(np.full((16, 128), 65504, np.float16),
                                  np.full(128, 2.0 ** -10, np.float16))


def _scale_covers_max(W, res):
    """S3's first half, vectorised: 7 * scale >= max|W'| in every group (exact in fp64)."""
    amax = np.abs(W.astype(np.float64)).reshape(W.shape[0], -1, 128).max(axis=2)
    return bool(np.all(7.0 * res.scales.astype(np.float64) >= amax))


def test_mutation_round_to_nearest_scale_breaks_s3(monkeypatch):
    import oracle.quantizer as qz
    W = weights(32, 0, 512, 1024)
    assert _scale_covers_max(W, qz.quantize_symmetric(W, None))
    monkeypatch.setattr(qz, "round_up_fp16", lambda v: np.asarray(v, np.float64).astype(np.float16))
    assert not _scale_covers_max(W, qz.quantize_symmetric(W, None))
