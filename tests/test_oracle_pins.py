"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, not by the oracle itself.

P1  round-trip bound |W' - (q - z) * scale| <= scale / 2 for every element;
P2  exact reconstruction of weights that lie on the quantization grid;
P3  byte counts printed on the pages (tests/golden/byte_counts.txt);
P4  brute force on tiny inputs in exact rationals (matmul, scale, zero point, codes);
P5  the integer special case s = 1, scale = 1, z = 8, where Y is an integer matmul;
P6  algebraic identities (AWQ fold, linearity, M=1 is row 0 of a batch).
Mutation tests at the end plant plausible mistakes in the oracle (on the CPU)
and check that one of these pins fails.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from workloads import activations, awq_scales, weights

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _roundtrip_ok(W, s, res):
    """P1 check; returns (ok, number of violating groups)."""
    Wd = W.astype(np.float64)
    sd = np.ones(W.shape[1]) if s is None else s.astype(np.float64)
    Wp = Wd / sd[None, :]
    w0 = oracle.dequantize(res.q, res.scales, res.zeros)      # quant(W/s), before * s
    half = np.repeat(res.scales.astype(np.float64), 128, axis=1) / 2
    bad = np.abs(Wp - w0) > half * (1 + 1e-12) + 1e-300
    return (not bad.any()), int(bad.reshape(W.shape[0], -1, 128).any(axis=2).sum())


def _on_grid(rng, N, K, with_s):
    """Weights that lie on the grid: codes with 0 and 15 in every group, z in 0..15,
    scale = m * 2^e with m in [64, 127] so that (q - z) * scale is an fp16 value."""
    G = K // 128
    q = rng.integers(0, 16, size=(N, G, 128))
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    perm = rng.permuted(np.tile(np.arange(128), (N, G, 1)), axis=2)
    q = np.take_along_axis(q, perm, axis=2)
    z = rng.integers(0, 16, size=(N, G))
    m = rng.integers(64, 128, size=(N, G))
    e = rng.integers(-16, -8, size=(N, G))
    scale = np.ldexp(m.astype(np.float64), e)
    wp = (q - z[:, :, None]) * scale[:, :, None]
    s = None
    if with_s:
        s = np.ldexp(1.0, rng.integers(-2, 3, size=K)).astype(np.float16)
        W = (wp.reshape(N, K) * s.astype(np.float64)[None, :])
    else:
        W = wp.reshape(N, K)
    W16 = W.astype(np.float16)
    assert np.array_equal(W16.astype(np.float64), W)  # really on the fp16 grid
    return W16, s, q.reshape(N, K).astype(np.uint8), scale.astype(np.float16), z.astype(np.float16)


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("case", ["gemv_1024", "awq_4096x1024", "heavy_tails"])
def test_p1_roundtrip_bound(case):
    if case == "gemv_1024":
        W, s = weights(0, 0, 1024, 1024), None
    elif case == "awq_4096x1024":
        W, s = weights(1, 0, 4096, 1024), awq_scales(1, 0, 1024)
    else:  # groups with very different ranges, subnormal-sized scales, exact zeros
        rng = np.random.default_rng(7)
        W = (rng.standard_t(2, size=(256, 512)) * np.exp(rng.uniform(-12, 3, size=(256, 1))))
        W[:, :128] = 0.0
        W = W.astype(np.float16)
        s = rng.lognormal(0, 1.0, 512).astype(np.float16)
    res = oracle.quantize(W, s)
    ok, nbad = _roundtrip_ok(W, s, res)
    assert ok, f"{nbad} groups exceed scale/2"
    assert res.q.max() <= 15 and res.zeros.min() >= 0 and res.zeros.max() <= 15
    assert np.array_equal(res.zeros, np.rint(res.zeros))


# ---------------------------------------------------------------- P2
@pytest.mark.parametrize("with_s", [False, True])
def test_p2_exact_on_grid(with_s):
    rng = np.random.default_rng(11 + with_s)
    W, s, q, scale, z = _on_grid(rng, 48, 512, with_s)
    res = oracle.quantize(W, s)
    assert np.array_equal(res.q, q)
    assert np.array_equal(res.scales.view(np.uint16), scale.view(np.uint16))
    assert np.array_equal(res.zeros.view(np.uint16), z.view(np.uint16))
    What = oracle.dequantize(res.q, res.scales, res.zeros, s)
    assert np.array_equal(What, W.astype(np.float64))


def test_all_zero_group_and_sign_of_zero():
    W = np.zeros((16, 256), dtype=np.float16)
    W[:, 128:] = -0.0
    W[3, 200] = np.float16(0.5)
    res = oracle.quantize(W)
    assert np.array_equal(res.scales[:, 0].view(np.uint16), np.zeros(16, np.uint16))
    assert np.array_equal(res.zeros.view(np.uint16)[:, 0], np.zeros(16, np.uint16))  # +0, not -0
    assert res.q[:, :128].max() == 0
    # a group holding only 0.5 and zeros: range [0, 0.5], scale = RU(0.5/15), z = 0
    assert res.zeros[3, 1] == 0 and res.q[3, 200] == 15


def test_errors():
    W = np.ones((16, 128), dtype=np.float16)
    with pytest.raises(oracle.NonFiniteInput):
        oracle.quantize(np.where(np.arange(128) == 5, np.float16(np.nan), W))
    with pytest.raises(oracle.NonFiniteInput):
        oracle.quantize(W, np.where(np.arange(128) == 3, np.float16(0), np.ones(128, np.float16)))
    with pytest.raises(oracle.NonFiniteInput):
        oracle.quantize(W, -np.ones(128, np.float16))
    big = W.copy()
    big[0, 0] = np.float16(60000)
    big[0, 1] = np.float16(-60000)
    with pytest.raises(oracle.ScaleOverflow):     # (120000 / 15) fits, but / s = 2^-4 does not
        oracle.quantize(big, np.full(128, 0.0625, np.float16))
    with pytest.raises(ValueError):
        oracle.quantize(np.ones((16, 100), np.float16))


# ---------------------------------------------------------------- P3
def test_p3_page_byte_counts(golden):
    for params, fmt, bpp, gb in golden("byte_counts.txt"):
        params = int(float(params))
        assert oracle.accounting.bytes_per_param(fmt) == Fraction(bpp)
        assert oracle.accounting.weight_bytes(params, fmt) == Fraction(gb) * 10**9


def test_p3_packed_sizes_and_quarter_of_fp16():
    # mhpq.cn sec.2.1: a 1024x1024 matrix in INT4 is a quarter of its FP16 size
    codes = oracle.pack_codes(np.zeros((1024, 1024), np.uint8))
    assert codes.nbytes * 4 == 1024 * 1024 * 2
    assert oracle.accounting.packed_sizes(1024, 1024) == (524288, 16384, 16384)
    # with one fp16 scale + one fp16 zero per 128 weights: 0.53125 B/param
    assert oracle.accounting.int4_group_bytes(7 * 10**9) == Fraction(371875, 100000) * 10**9
    assert oracle.accounting.int4_group_bytes(70 * 10**9) == Fraction(3718750, 100000) * 10**9


# ---------------------------------------------------------------- P4
@pytest.mark.parametrize("K,with_s", [(128, False), (256, True)])
def test_p4_bruteforce_gemm(K, with_s):
    rng = np.random.default_rng(K + with_s)
    W = (rng.standard_normal((4, K)) * 0.05).astype(np.float16)
    s = rng.lognormal(0, 0.5, K).astype(np.float16) if with_s else None
    X = rng.standard_normal((3, K)).astype(np.float16)
    res = oracle.quantize(W, s)
    Y = oracle.gemm(X, res.q, res.scales, res.zeros, s)
    Ye = exact.gemm_exact(X, res.q, res.scales, res.zeros, s)
    for m in range(3):
        for n in range(4):
            bound = Fraction(1, 10**13) * (1 + abs(Ye[m][n]))
            assert abs(Fraction(Y[m, n]) - Ye[m][n]) <= bound


@pytest.mark.parametrize("seed", [0, 1])
def test_p4_bruteforce_quantizer(seed):
    rng = np.random.default_rng(100 + seed)
    N, K = 6, 256
    W = (rng.standard_normal((N, K)) * rng.uniform(0.001, 2, size=(N, 1))).astype(np.float16)
    s = rng.lognormal(0, 0.5, K).astype(np.float16)
    res = oracle.quantize(W, s)
    Wp = W.astype(np.float64) / s.astype(np.float64)[None, :]   # reading R8: one fp64 division
    for n in range(N):
        for g in range(K // 128):
            blk = Wp[n, 128 * g:128 * (g + 1)]
            mn = min(Fraction(float(blk.min())), Fraction(0))
            mx = max(Fraction(float(blk.max())), Fraction(0))
            val, bits = exact.smallest_fp16_at_least((mx - mn) / 15)
            assert int(res.scales[n, g].view(np.uint16)) == bits
            # zero point: nearest integer to -mn/scale (ties to even)
            zt = -mn / val
            zc = exact.nearest_code(zt, 0)
            assert float(res.zeros[n, g]) == zc
            for k in range(128):
                t = Fraction(float(blk[k])) / val
                assert int(res.q[n, 128 * g + k]) == exact.nearest_code(t, zc)


def test_p4_round_up_fp16_exhaustive_neighbourhoods():
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.uniform(0, 1, 300) * np.exp2(rng.integers(-30, 16, 300)),
        np.arange(0, 0x7C00, 997, dtype=np.uint16).view(np.float16).astype(np.float64),
        [0.0, 2.0**-24, 2.0**-25, 2.0**-14, 65504.0, 65504.5],
    ])
    got = oracle.round_up_fp16(vals)
    for v, h in zip(vals, got):
        ref = exact.smallest_fp16_at_least(Fraction(float(v)))
        if ref is None:
            assert np.isinf(h)
        else:
            assert int(np.float16(h).view(np.uint16)) == ref[1]


def test_p4_tie_handling_rint_before_zero_shift():
    # group range [-7, 8]: scale = 1, z = 7 (odd); W' = 0.5 is a tie.
    W = np.zeros((16, 128), np.float16)
    W[:, 0], W[:, 1], W[:, 2], W[:, 3] = -7, 8, 0.5, -2.5
    res = oracle.quantize(W)
    assert float(res.scales[0, 0]) == 1.0 and float(res.zeros[0, 0]) == 7.0
    assert res.q[0, 2] == exact.nearest_code(Fraction(1, 2), 7) == 7     # (c - z) = 0 is even
    assert res.q[0, 3] == exact.nearest_code(Fraction(-5, 2), 7) == 5    # (c - z) = -2


# ---------------------------------------------------------------- P5
def test_p5_integer_special_case():
    rng = np.random.default_rng(5)
    N, K, M = 32, 256, 4
    Wi = rng.integers(-8, 8, size=(N, K))
    Wi[:, ::128] = -8
    Wi[:, 1::128] = 7
    res = oracle.quantize(Wi.astype(np.float16))
    assert np.all(res.scales == 1) and np.all(res.zeros == 8)
    assert np.array_equal(res.q.astype(np.int64), Wi + 8)
    X = rng.integers(-1, 2, size=(M, K))
    Y = oracle.gemm(X.astype(np.float16), res.q, res.scales, res.zeros)
    assert np.array_equal(Y, (X @ Wi.T).astype(np.float64))
    assert np.abs(Y).max() <= 2048


# ---------------------------------------------------------------- P6
def test_p6_identities():
    rng = np.random.default_rng(6)
    N, K = 32, 384
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = np.ldexp(1.0, rng.integers(0, 4, size=K)).astype(np.float16)   # 1, 2, 4, 8: X*s exact in fp16
    res = oracle.quantize(W, s)
    X = rng.standard_normal((5, K)).astype(np.float16)
    Xs = (X.astype(np.float64) * s.astype(np.float64)).astype(np.float16)
    assert np.array_equal(Xs.astype(np.float64), X.astype(np.float64) * s.astype(np.float64))
    Y1 = oracle.gemm(X, res.q, res.scales, res.zeros, s)
    Y2 = oracle.gemm(Xs, res.q, res.scales, res.zeros, None)
    np.testing.assert_allclose(Y1, Y2, rtol=1e-12, atol=1e-12)
    X2 = rng.standard_normal((5, K)).astype(np.float16)
    Ya = oracle.gemm(X, res.q, res.scales, res.zeros, s) + oracle.gemm(X2, res.q, res.scales, res.zeros, s)
    Yb = oracle.dequantize(res.q, res.scales, res.zeros, s) @ (X.astype(np.float64) + X2.astype(np.float64)).T
    np.testing.assert_allclose(Ya, Yb.T, rtol=1e-10, atol=1e-10)
    Y0 = oracle.gemm(X[:1], res.q, res.scales, res.zeros, s)
    assert np.array_equal(Y0[0], Y1[0])


def test_workload_activation_prefix():
    assert np.array_equal(activations(2, 1, 1, 4096), activations(2, 1, 9, 4096)[:1])


# ---------------------------------------------------------------- mutations
def test_mutation_round_to_nearest_scale_breaks_p1(monkeypatch):
    import oracle.quantizer as qm
    monkeypatch.setattr(qm, "round_up_fp16", lambda v: np.asarray(v).astype(np.float16))
    W, s = weights(1, 0, 2048, 1024), awq_scales(1, 0, 1024)
    ok, nbad = _roundtrip_ok(W, s, qm.quantize(W, s))
    assert not ok and nbad > 0


def test_mutation_zero_point_sign_breaks_p2(monkeypatch):
    import oracle.quantizer as qm
    real_rint = np.rint
    calls = {"n": 0}

    def bad_rint(x):   # the first rint in quantize() is the zero point; flip its sign
        calls["n"] += 1
        return -real_rint(x) if calls["n"] == 1 else real_rint(x)
    monkeypatch.setattr(qm.np, "rint", bad_rint)
    W, s, q, _, _ = _on_grid(np.random.default_rng(12), 16, 256, False)
    res = qm.quantize(W, s)
    monkeypatch.setattr(qm.np, "rint", real_rint)
    assert not np.array_equal(res.q, q)


def test_mutation_forgotten_awq_factor_breaks_p2():
    W, s, q, sc, z = _on_grid(np.random.default_rng(13), 16, 256, True)
    assert not np.array_equal(oracle.dequantize(q, sc, z, None), W.astype(np.float64))
    assert np.array_equal(oracle.dequantize(q, sc, z, s), W.astype(np.float64))


def test_mutation_transposed_weight_breaks_p4():
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((128, 128)) * 0.05).astype(np.float16)
    X = rng.standard_normal((2, 128)).astype(np.float16)
    res = oracle.quantize(W)
    wrong = X.astype(np.float64) @ oracle.dequantize(res.q, res.scales, res.zeros)   # missing .T
    Ye = exact.gemm_exact(X, res.q[:4], res.scales[:4], res.zeros[:4])
    assert any(abs(Fraction(wrong[0, n]) - Ye[0][n]) > Fraction(1, 10**6) for n in range(4))


def test_mutation_rint_after_zero_shift_breaks_tie_pin():
    # rint(W'/scale + z) instead of rint(W'/scale) + z moves the tie at 0.5 when z is odd
    t, z = 0.5, 7
    assert np.rint(t + z) != np.rint(t) + z
    assert np.rint(t) + z == exact.nearest_code(Fraction(1, 2), z)
