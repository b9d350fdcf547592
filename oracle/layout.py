"""Byte-level packed layout of the INT4 codes and the per-group scale / zero point.

This is the layout the library's packer writes and its GEMM kernels read.  It
is this repository's own format (the pages only fix the content: 4-bit codes
at half a byte per weight, with the scale and zero point carried alongside,
discosf.com tutorial sec.2.3 and aiwing.uk ch.22 sec.22.3 table).  The oracle
restates it element by element from the definition below; nothing is shared
with the HIP packer.

Definition.  W is [N][K]; G = K / 128 groups per row; N is a multiple of 16;
NB = N / 16 row blocks.
  * Tile (b, g) covers rows 16b .. 16b+15 and the 128 columns of group g.  It
    is 1024 bytes at byte offset (g * NB + b) * 1024 of the code buffer: the
    tiles of one group are contiguous, row block after row block.
  * Inside a tile, 64 "lanes" own 16 bytes each: lane L = 16 * c + r (row
    r = 0..15 inside the tile, column octet c = 0..3) at byte 16 * L.
  * The lane's 16 bytes are four little-endian 32-bit words; word t (t = 0..3)
    holds the eight codes of columns 128 g + 32 t + 8 c + j, j = 0..7.
  * Inside a word, the 4-bit slot i (bits 4i .. 4i+3) holds column
    j = 2 * (i % 4) + i // 4: even j in the low half-word, odd j in the high
    half-word, each in increasing order.
  * Scales and zero points (fp16 each) are stored in quads of 4 groups:
    with Gq = ceil(G / 4), the value of row n = 16b + r, group g = 4u + i is
    element ((u * NB + b) * 16 + r) * 4 + i of its buffer (N * 4 * Gq
    elements; the slots of groups G .. 4*Gq - 1 hold zero).  So the metadata
    of one 16-row block and 4 consecutive groups is one contiguous 128-byte
    run (a single 8-byte load per row fetches 4 groups), and the runs of one
    quad follow each other row block after row block.
INT8 codes (the W8A16 variant, one byte per weight) use the same groups, row
blocks and metadata, with 2048-byte tiles:
  * tile (b, g) is at byte offset (g * NB + b) * 2048 of the code buffer;
  * lane L = 16 * c + r owns the 32 bytes at byte 32 * L;
  * its byte 8 * t + j holds the code of column 128 g + 32 t + 8 c + j
    (t = 0..3, j = 0..7): increasing column order.
TEST INFRASTRUCTURE: see the package docstring for who may import this.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 16
TILE_BYTES = 1024
TILE_BYTES8 = 2048
META_QUAD = 4
_GROUP = 128


def _check(N: int, K: int) -> int:
    if N <= 0 or K <= 0 or N % TILE_ROWS or K % _GROUP:
        raise ValueError("N must be a positive multiple of 16 and K of 128")
    return K // _GROUP


def nibble_address(n, k, N: int, K: int):
    """(byte offset, bit shift) of the code of W[n][k].  Works on scalars or index arrays."""
    G = _check(N, K)
    n = np.asarray(n, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    NB = N // TILE_ROWS
    b, r = n // TILE_ROWS, n % TILE_ROWS          # tile row block, row inside the tile
    g, kk = k // _GROUP, k % _GROUP               # group, column inside the group
    t, c, j = kk // 32, (kk % 32) // 8, kk % 8    # word, column octet (lane), column in octet
    slot = (j // 2) + 4 * (j % 2)                 # inverse of j = 2*(slot % 4) + slot // 4
    lane = 16 * c + r
    byte = (g * NB + b) * TILE_BYTES + 16 * lane + 4 * t + slot // 2
    shift = 4 * (slot % 2)
    return byte, shift


def pack_codes(q: np.ndarray) -> np.ndarray:
    """uint8 codes q[N][K] (0..15) -> packed uint8 buffer of N*K/2 bytes."""
    q = np.asarray(q)
    N, K = q.shape
    _check(N, K)
    if q.dtype != np.uint8 or q.max(initial=0) > 15:
        raise ValueError("codes must be uint8 in 0..15")
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    byte, shift = nibble_address(nn.ravel(), kk.ravel(), N, K)
    out = np.zeros(N * K // 2, dtype=np.uint8)
    # each byte receives exactly two codes (shift 0 and shift 4); OR them in.
    np.bitwise_or.at(out, byte, (q.ravel().astype(np.uint8) << shift.astype(np.uint8)))
    return out


def unpack_codes(buf: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed buffer -> uint8 codes q[N][K]."""
    _check(N, K)
    buf = np.asarray(buf, dtype=np.uint8).ravel()
    if buf.size != N * K // 2:
        raise ValueError("buffer size mismatch")
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    byte, shift = nibble_address(nn.ravel(), kk.ravel(), N, K)
    return ((buf[byte] >> shift.astype(np.uint8)) & 0xF).astype(np.uint8).reshape(N, K)


def meta_groups(K: int) -> int:
    """Groups per row in the metadata buffers: G rounded up to a multiple of 4."""
    G = K // _GROUP
    return -(-G // META_QUAD) * META_QUAD


def meta_index(n, g, N: int, K: int):
    """Element index of (row n, group g) in the scale / zero-point buffers."""
    _check(N, K)
    Gq = meta_groups(K) // META_QUAD
    n = np.asarray(n, dtype=np.int64)
    g = np.asarray(g, dtype=np.int64)
    NB = N // TILE_ROWS
    b, r = n // TILE_ROWS, n % TILE_ROWS
    u, i = g // META_QUAD, g % META_QUAD
    return ((u * NB + b) * TILE_ROWS + r) * META_QUAD + i


def pack_meta(a: np.ndarray) -> np.ndarray:
    """Per-group array a[N][G] (fp16) -> flat buffer of N * meta_groups(K) elements."""
    a = np.asarray(a)
    N, G = a.shape
    K = G * _GROUP
    nn, gg = np.meshgrid(np.arange(N), np.arange(G), indexing="ij")
    out = np.zeros(N * meta_groups(K), dtype=a.dtype)
    out[meta_index(nn.ravel(), gg.ravel(), N, K)] = a.ravel()
    return out


def unpack_meta(buf: np.ndarray, N: int, K: int) -> np.ndarray:
    """Flat metadata buffer -> a[N][G]."""
    _check(N, K)
    G = K // _GROUP
    buf = np.asarray(buf).ravel()
    if buf.size != N * meta_groups(K):
        raise ValueError("buffer size mismatch")
    nn, gg = np.meshgrid(np.arange(N), np.arange(G), indexing="ij")
    return buf[meta_index(nn.ravel(), gg.ravel(), N, K)].reshape(N, G)


def byte_address8(n, k, N: int, K: int):
    """Byte offset of the INT8 code of W[n][k].  Works on scalars or index arrays."""
    _check(N, K)
    n = np.asarray(n, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    NB = N // TILE_ROWS
    b, r = n // TILE_ROWS, n % TILE_ROWS
    g, kk = k // _GROUP, k % _GROUP
    t, c, j = kk // 32, (kk % 32) // 8, kk % 8
    return (g * NB + b) * TILE_BYTES8 + 32 * (16 * c + r) + 8 * t + j


def pack_codes8(q: np.ndarray) -> np.ndarray:
    """uint8 codes q[N][K] (0..255) -> packed buffer of N*K bytes."""
    q = np.asarray(q)
    N, K = q.shape
    _check(N, K)
    if q.dtype != np.uint8:
        raise ValueError("codes must be uint8")
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    out = np.zeros(N * K, dtype=np.uint8)
    out[byte_address8(nn.ravel(), kk.ravel(), N, K)] = q.ravel()
    return out


def unpack_codes8(buf: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed INT8 buffer -> codes q[N][K]."""
    _check(N, K)
    buf = np.asarray(buf, dtype=np.uint8).ravel()
    if buf.size != N * K:
        raise ValueError("buffer size mismatch")
    nn, kk = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    return buf[byte_address8(nn.ravel(), kk.ravel(), N, K)].reshape(N, K)
