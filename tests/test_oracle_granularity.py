"""Pins for the coarser granularities of the oracle quantizer (discosf.com sec.2.1: a scale
per tensor, per channel or per group of 128).

G1  one group per row (K = 128) makes channel granularity identical to group granularity,
    and one row block whose rows share their extremes makes tensor equal to channel;
G2  every group of a row (channel) or of the tensor (tensor) carries the same scale and
    zero point, and that scale is the one the R4/R5 rule gives for the row's (tensor's)
    range: least fp16 >= range / 15, checked in exact rationals;
G3  the round-trip bound |W' - (q - z) scale| <= scale / 2 holds at every granularity;
G4  the page's ordering: coarser granularity never shrinks a group's scale, and on
    real-shaped weights the reconstruction error grows from group to channel to tensor;
and a mutation that leaves the range at the group's (never widened to the row or the
tensor) fails G2.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import smallest_fp16_at_least


def _w(rng, N, K, awq=True):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    s = np.exp(rng.standard_normal(K) * 0.5).astype(np.float16) if awq else None
    return W, s


def _same(a, b):
    return all(np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
               for x, y in zip((a.q, a.scales, a.zeros), (b.q, b.scales, b.zeros)))


def test_g1_special_cases():
    rng = np.random.default_rng(50)
    W, s = _w(rng, 32, 128)
    assert _same(oracle.quantize(W, s, "channel"), oracle.quantize(W, s, "group"))
    W, _ = _w(rng, 16, 512, awq=False)
    W[:, 0] = np.float16(-0.5)     # every row shares its min and max
    W[:, 1] = np.float16(0.75)
    assert _same(oracle.quantize(W, None, "tensor"), oracle.quantize(W, None, "channel"))


def _check_g2(gran, seed=51):
    rng = np.random.default_rng(seed)
    N, K = 16, 384
    W, s = _w(rng, N, K)
    r = oracle.quantize(W, s, gran)
    Wp = [[Fraction(float(W[n, k])) / Fraction(float(s[k])) for k in range(K)] for n in range(N)]
    for n in range(N):
        rows = Wp if gran == "tensor" else [Wp[n]]
        lo = min(min(row) for row in rows)
        hi = max(max(row) for row in rows)
        rng_ = max(hi, 0) - min(lo, 0)
        want, _ = smallest_fp16_at_least(rng_ / 15)
        assert all(Fraction(float(x)) == want for x in r.scales[n])
        assert len(set(r.zeros[n].tolist())) == 1
    if gran == "tensor":
        assert len(set(r.scales.ravel().tolist())) == 1


@pytest.mark.parametrize("gran", ["channel", "tensor"])
def test_g2_shared_metadata_and_exact_scale(gran):
    _check_g2(gran)


@pytest.mark.parametrize("gran", oracle.GRANULARITIES)
def test_g3_round_trip_bound(gran):
    rng = np.random.default_rng(52)
    N, K = 48, 1024
    W, s = _w(rng, N, K)
    r = oracle.quantize(W, s, gran)
    g = np.arange(K) // 128
    sc = r.scales.astype(np.float64)[:, g]
    Wp = W.astype(np.float64) / s.astype(np.float64)[None, :]
    rec = (r.q.astype(np.float64) - r.zeros.astype(np.float64)[:, g]) * sc
    assert np.all(np.abs(Wp - rec) <= sc / 2)


def test_g4_coarser_is_worse():
    rng = np.random.default_rng(53)
    N, K = 64, 2048
    W, s = _w(rng, N, K)
    W[5, 700] = np.float16(0.9)   # one large weight: widens its row and the tensor
    res = {gr: oracle.quantize(W, s, gr) for gr in oracle.GRANULARITIES}
    assert np.all(res["group"].scales <= res["channel"].scales)
    assert np.all(res["channel"].scales <= res["tensor"].scales)
    Wd = W.astype(np.float64)
    err = {gr: np.linalg.norm(oracle.dequantize(r.q, r.scales, r.zeros, s) - Wd)
           for gr, r in res.items()}
    assert err["group"] < err["channel"] < err["tensor"]


@pytest.mark.parametrize("gran", ["channel", "tensor"])
def test_mutation_unwidened_range_fails_g2(gran, monkeypatch):
    """Planted: the range is left at each group's own extremes (never widened to the row
    or the tensor); G2 must fail."""
    from oracle import quantizer
    real = quantizer._extremes
    monkeypatch.setattr(quantizer, "_extremes", lambda Wp, g: real(Wp, "group"))
    with pytest.raises(AssertionError):
        _check_g2(gran)
