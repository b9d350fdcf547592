"""Pins for the INT8 (W8A16) variant of the oracle quantizer and its packed layout.

I-1  hand-derived byte addresses (tests/golden/layout8_examples.txt) and a bijection
     between weights and the N*K code bytes;
I-2  the round-trip bound |W' - (q - z) scale| <= scale / 2 with codes 0..255;
I-3  weights lying on an INT8 grid are reconstructed exactly;
I-4  brute force in exact rationals: scale = least fp16 >= range / 255, z = rint(-min /
     scale), q = the nearest code;
I-5  aiwing.uk sec.22.3's table: INT8 takes one byte per parameter (twice INT4);
and a mutation (the 4-bit range used for 8-bit codes) that fails I-2's tightness.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from tests.conftest import ROOT


def test_i1_golden_addresses_and_bijection():
    rows = [l.split("#")[0].split() for l in open(os.path.join(ROOT, "tests", "golden",
                                                              "layout8_examples.txt"))]
    rows = [list(map(int, r)) for r in rows if r]
    assert len(rows) >= 5
    for N, K, n, k, byte in rows:
        assert int(oracle.byte_address8(n, k, N, K)) == byte, (N, K, n, k)
    N, K = 48, 384
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    addr = oracle.byte_address8(nn.ravel(), kk.ravel(), N, K)
    assert np.array_equal(np.sort(addr), np.arange(N * K))
    q = np.random.default_rng(1).integers(0, 256, size=(N, K)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_codes8(oracle.pack_codes8(q), N, K), q)


def _w(seed, N, K, awq=True):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = np.exp(rng.standard_normal(K) * 0.5).astype(np.float16) if awq else None
    return W, s


@pytest.mark.parametrize("awq", [False, True])
def test_i2_round_trip_bound(awq):
    W, s = _w(80 + awq, 64, 1024, awq)
    r = oracle.quantize(W, s, bits=8)
    g = np.arange(1024) // 128
    sc = r.scales.astype(np.float64)[:, g]
    Wp = W.astype(np.float64) / (s.astype(np.float64)[None, :] if awq else 1.0)
    rec = (r.q.astype(np.float64) - r.zeros.astype(np.float64)[:, g]) * sc
    assert np.all(np.abs(Wp - rec) <= sc / 2)
    assert r.q.max() == 255 and r.q.min() == 0      # the full 8-bit range is used


def test_i3_grid_exact():
    rng = np.random.default_rng(82)
    N, K = 16, 256
    scale = np.float16(2.0 ** -9)
    z = rng.integers(0, 256, size=(N, K // 128))
    q = rng.integers(0, 256, size=(N, K))
    q[:, ::128] = 0
    q[:, 1::128] = 255                               # every group spans the whole grid
    g = np.arange(K) // 128
    W = ((q - z[:, g]) * float(scale)).astype(np.float16)
    assert np.array_equal(W.astype(np.float64), (q - z[:, g]) * float(scale))   # exact in fp16
    r = oracle.quantize(W, None, bits=8)
    assert np.array_equal(oracle.dequantize(r.q, r.scales, r.zeros), W.astype(np.float64))


def test_i4_brute_force():
    rng = np.random.default_rng(83)
    N, K = 4, 256
    W = (rng.standard_normal((N, K)) * rng.uniform(0.001, 2, size=(N, 1))).astype(np.float16)
    s = rng.lognormal(0, 0.5, K).astype(np.float16)
    r = oracle.quantize(W, s, bits=8)
    Wp = W.astype(np.float64) / s.astype(np.float64)[None, :]
    for n in range(N):
        for g in range(K // 128):
            blk = Wp[n, 128 * g:128 * (g + 1)]
            mn = min(Fraction(float(blk.min())), Fraction(0))
            mx = max(Fraction(float(blk.max())), Fraction(0))
            val, bits = exact.smallest_fp16_at_least((mx - mn) / 255)
            assert int(r.scales[n, g].view(np.uint16)) == bits
            zt = -mn / val
            z = int(np.rint(float(zt)))
            assert int(r.zeros[n, g]) == z
            for k in range(0, 128, 7):
                t = Fraction(float(blk[k])) / val
                assert int(r.q[n, 128 * g + k]) == exact.nearest_code(t, z, 255)


def test_i5_byte_per_parameter():
    assert oracle.accounting.bytes_per_param("int8") == 1
    assert oracle.accounting.bytes_per_param("int4") * 2 == oracle.accounting.bytes_per_param("int8")
    for N, K in ((16, 128), (4096, 4096)):
        assert oracle.pack_codes8(np.zeros((N, K), np.uint8)).size == N * K   # one byte each


def test_mutation_four_bit_range_fails():
    W, s = _w(84, 16, 256)
    r8 = oracle.quantize(W, s, bits=8)
    r4 = oracle.quantize(W, s, bits=4)
    assert np.all(r8.scales.astype(np.float64) < r4.scales.astype(np.float64))   # 15x finer
