"""Pins for the packed-layout spec in the oracle (round trip, bijection, hand-derived addresses)."""
import numpy as np
import pytest

import oracle


def test_layout_golden_addresses(golden):
    for N, K, n, k, byte, shift in (map(int, r) for r in golden("layout_examples.txt")):
        b, s = oracle.nibble_address(n, k, N, K)
        assert (int(b), int(s)) == (byte, shift)
        q = np.zeros((N, K), np.uint8)
        q[n, k] = 0xA
        buf = oracle.pack_codes(q)
        nz = np.flatnonzero(buf)
        assert list(nz) == [byte] and buf[byte] == (0xA << shift)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (64, 1024)])
def test_layout_roundtrip_and_bijection(N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    buf = oracle.pack_codes(q)
    assert buf.size == N * K // 2
    assert np.array_equal(oracle.unpack_codes(buf, N, K), q)
    assert np.all(oracle.pack_codes(np.full((N, K), 15, np.uint8)) == 0xFF)
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    byte, shift = oracle.nibble_address(nn.ravel(), kk.ravel(), N, K)
    key = byte * 2 + shift // 4
    assert np.unique(key).size == N * K and key.min() == 0 and key.max() == N * K - 1


def test_layout_word_semantics():
    # word t of lane (c, r) holds columns 32t + 8c + j; even j low half-word, odd j high.
    N, K = 16, 128
    q = np.zeros((N, K), np.uint8)
    r, c, t = 3, 2, 1
    for j in range(8):
        q[r, 32 * t + 8 * c + j] = j + 1
    buf = oracle.pack_codes(q)
    lane = 16 * c + r
    word = int(buf[16 * lane + 4 * t: 16 * lane + 4 * t + 4].view("<u4")[0])
    lo, hi = word & 0xFFFF, word >> 16
    assert [(lo >> (4 * i)) & 0xF for i in range(4)] == [1, 3, 5, 7]
    assert [(hi >> (4 * i)) & 0xF for i in range(4)] == [2, 4, 6, 8]


def test_meta_layout():
    N, K = 48, 512
    G = K // 128
    a = np.arange(N * G, dtype=np.float16).reshape(N, G)
    buf = oracle.pack_meta(a)
    assert np.array_equal(oracle.unpack_meta(buf, N, K), a)
    assert buf[oracle.meta_index(17, 2, N, K)] == a[17, 2]
    assert int(oracle.meta_index(17, 2, N, K)) == 17 * G + 2
    assert np.array_equal(buf, a.ravel())   # row-major: the identity on [N][G]


def test_layout_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((8, 128), np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((16, 64), np.uint8))
