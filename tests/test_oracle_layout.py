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
    # G = 5 groups -> 8 slots per row (quads of 4, zero padded)
    N, K = 48, 640
    G = K // 128
    a = (np.arange(N * G, dtype=np.float16) + 1).reshape(N, G)
    buf = oracle.pack_meta(a)
    assert buf.size == N * 8 and oracle.meta_groups(K) == 8
    assert np.array_equal(oracle.unpack_meta(buf, N, K), a)
    # hand-derived: NB = 3 row blocks; row 17 = block 1, r 1; group 4 = quad 1, slot 0
    # index ((1 * 3 + 1) * 16 + 1) * 4 + 0 = 260
    assert int(oracle.meta_index(17, 4, N, K)) == 260 and buf[260] == a[17, 4]
    # row 5, group 2: ((0 * 3 + 0) * 16 + 5) * 4 + 2 = 22
    assert int(oracle.meta_index(5, 2, N, K)) == 22
    # row 47 (block 2, r 15), group 3 (quad 0, slot 3): ((0 * 3 + 2) * 16 + 15) * 4 + 3 = 191
    assert int(oracle.meta_index(47, 3, N, K)) == 191
    # padding slots (groups 5..7) are zero, and every real value appears once
    assert np.count_nonzero(buf) == N * G
    # one 16-row block x 4 groups is one contiguous run of 64 elements (128 bytes)
    idx = oracle.meta_index(np.repeat(np.arange(16, 32), 4), np.tile(np.arange(4, 8), 16), N, K)
    assert sorted(idx.tolist()) == list(range(idx.min(), idx.min() + 64))
    # and the runs of one quad (all N rows x groups 4..7) follow each other
    idx = oracle.meta_index(np.repeat(np.arange(N), 4), np.tile(np.arange(4, 8), N), N, K)
    assert sorted(idx.tolist()) == list(range(N * 4, 2 * N * 4))


def test_layout_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((8, 128), np.uint8))
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((16, 64), np.uint8))
