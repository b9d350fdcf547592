"""Pins for the outlier side path of the oracle (mhpq.cn notes sec.2.2).

O-1  the selection against brute force in exact rationals: the `count` largest
     |W| / s as Fractions, ties to the lower flat index (sorted by Python, not NumPy);
O-2  the merge: W_hat equals W exactly where kept, and the INT4 side is exactly 0
     there (code == zero point), for both grids;
O-3  removing outliers never widens a group: every group's scale is at most the
     plain quantizer's, strictly smaller where a planted outlier set the range, and
     the round-trip bound |W' - (q - z) scale| <= scale / 2 holds on what is left;
O-4  special cases: count 0 is the plain quantizer byte for byte; count N*K keeps
     every weight (all groups empty) and Y is the exact product X . W^T;
O-5  Y splits into the INT4 product plus the sparse fp16 product written as loops;
and mutation tests that plant a wrong ranking key and an unforced code.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import outliers as ol


def _data(rng, N, K, planted=0, with_s=True):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    if planted:
        idx = rng.choice(N * K, size=planted, replace=False)
        W.ravel()[idx] = (W.ravel()[idx].astype(np.float32) * 10).astype(np.float16)
    s = np.exp(rng.standard_normal(K) * 0.5).astype(np.float16) if with_s else None
    return W, s


@pytest.mark.parametrize("with_s", [False, True])
def test_o1_selection_brute_force(with_s):
    rng = np.random.default_rng(31 + with_s)
    for trial in range(6):
        N, K = int(rng.integers(1, 5)), 128
        W, s = _data(rng, N, K, with_s=with_s)
        if trial % 2:   # many exact ties: a handful of distinct values
            W = rng.choice(np.array([-0.5, -0.25, 0.0, 0.25, 0.5], np.float16), size=(N, K))
        for count in (0, 1, 7, N * K // 3, N * K):
            key = [(abs(Fraction(float(W[n, k]))) /
                    (Fraction(float(s[k])) if s is not None else 1), n * K + k)
                   for n in range(N) for k in range(K)]
            want = {i for _, i in sorted(key, key=lambda t: (-t[0], t[1]))[:count]}
            got = set(np.flatnonzero(ol.select(W, s, count)).tolist())
            assert got == want, (trial, count)


@pytest.mark.parametrize("symmetric", [False, True])
def test_o2_merge_keeps_fp16_and_zeroes_int4(symmetric):
    rng = np.random.default_rng(40 + symmetric)
    W, s = _data(rng, 48, 512, planted=25)
    res = ol.quantize_with_outliers(W, s, ol.page_count(48, 512) + 5, symmetric)
    assert res.mask.sum() == res.col.size == ol.page_count(48, 512) + 5
    g = np.arange(512) // 128
    z = res.quant.zeros.astype(np.float64)[:, g]
    assert np.all(res.quant.q[res.mask] == z[res.mask])                 # INT4 side is 0 there
    Wh = ol.merged_weight(res, W, s)
    assert np.array_equal(Wh[res.mask], W[res.mask].astype(np.float64))  # exact fp16 value
    # CSR in (row, column) order, values are W's
    for n in range(48):
        cols = res.col[res.row_ptr[n]:res.row_ptr[n + 1]]
        assert np.array_equal(cols, np.flatnonzero(res.mask[n]))
        assert np.array_equal(res.val[res.row_ptr[n]:res.row_ptr[n + 1]], W[n, cols])


def test_o3_groups_only_shrink_and_bound_holds():
    rng = np.random.default_rng(43)
    N, K, planted = 64, 1024, 40
    W, s = _data(rng, N, K, planted=planted)
    plain = oracle.quantize(W, s)
    res = ol.quantize_with_outliers(W, s, planted)
    sc, sc0 = res.quant.scales.astype(np.float64), plain.scales.astype(np.float64)
    assert np.all(sc <= sc0)
    # groups holding a kept weight that set their range shrink strictly
    Wp = W.astype(np.float64) / s.astype(np.float64)[None, :]
    G = K // 128
    for n, k in zip(*np.nonzero(res.mask)):
        grp = Wp[n, (k // 128) * 128:(k // 128 + 1) * 128]
        if abs(Wp[n, k]) == np.abs(grp).max() and np.sort(np.abs(grp))[-2] < abs(Wp[n, k]) / 2:
            assert sc[n, k // 128] < sc0[n, k // 128]
    # round-trip bound on the INT4 side
    g = np.arange(K) // 128
    recon = (res.quant.q.astype(np.float64) - res.quant.zeros.astype(np.float64)[:, g]) \
        * sc[:, g]
    err = np.abs(np.where(res.mask, 0.0, Wp) - recon)
    assert np.all(err <= sc[:, g] / 2 + 1e-300)
    assert G == 8


def test_o4_special_cases():
    rng = np.random.default_rng(44)
    W, s = _data(rng, 8, 256)
    plain = oracle.quantize(W, s)
    res = ol.quantize_with_outliers(W, s, 0)
    assert np.array_equal(res.quant.q, plain.q)
    assert np.array_equal(res.quant.scales.view(np.uint16), plain.scales.view(np.uint16))
    assert np.array_equal(res.quant.zeros.view(np.uint16), plain.zeros.view(np.uint16))
    assert res.col.size == 0 and np.all(res.row_ptr == 0)
    # everything kept: every group is empty and Y is the exact product with W
    X = rng.standard_normal((3, 256)).astype(np.float16)
    full = ol.quantize_with_outliers(W, s, 8 * 256)
    assert np.all(full.quant.scales == 0)
    Y = ol.gemm(X, full, W, s)
    ref = np.array([[float(sum(Fraction(float(X[m, k])) * Fraction(float(W[n, k]))
                               for k in range(256))) for n in range(8)] for m in range(3)])
    assert np.allclose(Y, ref, rtol=1e-14, atol=1e-15)


def test_o5_int4_plus_sparse_product():
    rng = np.random.default_rng(45)
    N, K, M = 32, 384, 4
    W, s = _data(rng, N, K, planted=12)
    X = rng.standard_normal((M, K)).astype(np.float16)
    res = ol.quantize_with_outliers(W, s, 20)
    Y = ol.gemm(X, res, W, s)
    dense = oracle.gemm(X, res.quant.q, res.quant.scales, res.quant.zeros, s)
    sparse = np.zeros((M, N))
    for n in range(N):
        for e in range(res.row_ptr[n], res.row_ptr[n + 1]):
            for m in range(M):
                sparse[m, n] += float(X[m, res.col[e]]) * float(res.val[e])
    assert np.allclose(Y, dense + sparse, rtol=1e-12, atol=1e-12)


def test_page_count():
    assert ol.page_count(4096, 4096) == 16777
    assert ol.page_count(1024, 1024) == 1049
    assert ol.page_count(16, 128) == 2


def test_mutations_are_caught():
    rng = np.random.default_rng(46)
    N, K = 4, 128
    W, s = _data(rng, N, K)
    s = s.copy()
    s[:8] = np.float16(8.0)     # a large s shrinks |W'| of the first columns: |W| ranks differently
    count = 10
    key = [(abs(Fraction(float(W[n, k]))) / Fraction(float(s[k])), n * K + k)
           for n in range(N) for k in range(K)]
    want = {i for _, i in sorted(key, key=lambda t: (-t[0], t[1]))[:count]}
    wrong_key = set(np.flatnonzero(ol.select(W, None, count)).tolist())   # ranks |W|
    assert wrong_key != want
    # unforced codes: quantizing W itself (outliers left in) breaks O-2
    res = ol.quantize_with_outliers(W, s, count)
    unforced = oracle.quantize(W, s)
    z = unforced.zeros.astype(np.float64)[:, np.arange(K) // 128]
    assert not np.all(unforced.q[res.mask] == z[res.mask])


def test_o_int8_remainder():
    """The same split with INT8 codes for the remainder: count 0 is the plain INT8
    quantizer byte for byte; kept positions decode to exactly 0 (code == zero point)
    and merge back to W exactly; groups only shrink; the round-trip bound holds on
    the 0..255 grid; selection and CSR do not depend on the code width."""
    rng = np.random.default_rng(46)
    N, K = 48, 512
    W, s = _data(rng, N, K, planted=25)
    plain8 = oracle.quantize(W, s, bits=8)
    r0 = ol.quantize_with_outliers(W, s, 0, bits=8)
    assert np.array_equal(r0.quant.q, plain8.q)
    assert np.array_equal(r0.quant.scales.view(np.uint16), plain8.scales.view(np.uint16))
    count = ol.page_count(N, K) + 5
    r8 = ol.quantize_with_outliers(W, s, count, bits=8)
    r4 = ol.quantize_with_outliers(W, s, count)
    assert np.array_equal(r8.mask, r4.mask) and np.array_equal(r8.col, r4.col)
    assert np.array_equal(r8.row_ptr, r4.row_ptr) and np.array_equal(r8.val.view(np.uint16),
                                                                    r4.val.view(np.uint16))
    g = np.arange(K) // 128
    z = r8.quant.zeros.astype(np.float64)[:, g]
    assert np.all(r8.quant.q[r8.mask] == z[r8.mask])
    assert np.array_equal(ol.merged_weight(r8, W, s)[r8.mask], W[r8.mask].astype(np.float64))
    sc = r8.quant.scales.astype(np.float64)
    assert np.all(sc <= plain8.scales.astype(np.float64))
    Wp = W.astype(np.float64) / s.astype(np.float64)[None, :]
    recon = (r8.quant.q.astype(np.float64) - z) * sc[:, g]
    assert np.all(np.abs(np.where(r8.mask, 0.0, Wp) - recon) <= sc[:, g] / 2 + 1e-300)
    assert r8.quant.q.max() > 15                      # the codes really use the byte
    with pytest.raises(ValueError):
        ol.quantize_with_outliers(W, s, count, symmetric=True, bits=8)
