"""The largest inputs the library accepts, against the oracle on sampled rows.

The packed codes of one matrix are addressed with 32-bit byte offsets, so the library
takes N * K / 2 <= 2^31 - 2^20 INT4 code bytes (N * K for INT8 codes).  These tests
pack a matrix of exactly that size (65504 x 65536, 4.29e9 weights, an 8.6 GB fp16
input) and run it through the streaming and tiled kernels; the oracle checks 64
sampled rows, which depend on nothing but their own weights.  A second case takes a
very long K (2^21 columns, 16384 groups) through K windows and the tiled kernel.
Inputs: W ~ N(0, 0.02) drawn on the device by torch's seeded generator (the oracle
reads the same sampled rows back), s and X from workloads.
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, h16_bits, note, to_dev, to_host, torch_cuda
from workloads import activations, awq_scales

pytestmark = pytest.mark.gpu

LIMIT_BYTES = (1 << 31) - (1 << 20)


def device_weights(torch, N, K, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    W = torch.randn((N, K), dtype=torch.float16, device="cuda", generator=g)
    return W.mul_(0.02)


def sample_rows(N, count, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(np.arange(16, N - 16), count - 4, replace=False)
    return np.sort(np.concatenate([[0, 15, N - 16, N - 1], rows]))   # first and last blocks too


def gather(torch, buf, idx):
    return buf[torch.from_numpy(np.ascontiguousarray(idx).ravel()).to("cuda")].cpu().numpy()


def check_int4_rows(torch, pw, Wd, s, rows, N, K):
    ref = oracle.quantize(Wd[torch.from_numpy(rows).to("cuda")].cpu().numpy(), s)
    nn, kk = np.meshgrid(rows, np.arange(K), indexing="ij")
    byte, shift = oracle.nibble_address(nn, kk, N, K)
    q = (gather(torch, pw.wq, byte).reshape(byte.shape) >> shift) & 15
    assert np.array_equal(q, ref.q)
    gg = np.arange(K // 128)
    mi = oracle.meta_index(rows[:, None], gg[None, :], N, K)
    assert np.array_equal(h16_bits(gather(torch, pw.scales, mi).reshape(mi.shape)), h16_bits(ref.scales))
    assert np.array_equal(h16_bits(gather(torch, pw.zeros, mi).reshape(mi.shape)), h16_bits(ref.zeros))
    return ref


def test_largest_int4_matrix():
    torch = torch_cuda()
    N, K = 65504, 65536
    assert N * K // 2 == LIMIT_BYTES
    assert w4.w4a16_packed_sizes(N, K)[0] == LIMIT_BYTES
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_packed_sizes(N + 16, K)
    s = awq_scales(40, 0, K)
    note(f"largest INT4 matrix N={N} K={K}: generate and pack")
    Wd = device_weights(torch, N, K, 40)
    pw = w4.w4a16_quantize_pack(Wd, to_dev(s))
    rows = sample_rows(N, 64, 40)
    ref = check_int4_rows(torch, pw, Wd, s, rows, N, K)
    for M in (1, 17):
        X = activations(40, M, M, K)
        note(f"largest INT4 matrix gemm M={M}")
        Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
        assert_close(Y[:, rows], oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"M={M}")
    del pw, Wd
    torch.cuda.empty_cache()


def test_largest_int8_matrix():
    torch = torch_cuda()
    N, K = 32752, 65536
    assert N * K == LIMIT_BYTES
    s = awq_scales(41, 0, K)
    note(f"largest INT8 matrix N={N} K={K}: generate and pack")
    Wd = device_weights(torch, N, K, 41)
    pw = w4.w4a16_quantize_pack(Wd, to_dev(s), mode=w4.QUANT_ASYM8)
    rows = sample_rows(N, 64, 41)
    ref = oracle.quantize(Wd[torch.from_numpy(rows).to("cuda")].cpu().numpy(), s, bits=8)
    nn, kk = np.meshgrid(rows, np.arange(K), indexing="ij")
    addr = oracle.byte_address8(nn, kk, N, K)
    assert np.array_equal(gather(torch, pw.wq, addr).reshape(addr.shape), ref.q)
    X = activations(41, 1, 1, K)
    note("largest INT8 matrix gemm M=1")
    Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
    assert_close(Y[:, rows], oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), "int8 M=1")
    del pw, Wd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 5, 16, 17])
def test_very_long_rows(M):
    """K = 2^21: 16384 groups per row.  X * s of even one row is 4 MiB, past the
    streaming kernel's LDS budget, so M = 1..16 run with K windows; M = 17 goes to
    the tiled kernel."""
    torch = torch_cuda()
    N, K = 16, 1 << 21
    s = awq_scales(42, 0, K)
    Wd = device_weights(torch, N, K, 42)
    pw = w4.w4a16_quantize_pack(Wd, to_dev(s))
    ref = oracle.quantize(Wd.cpu().numpy(), s)
    assert np.array_equal(to_host(pw.wq), oracle.pack_codes(ref.q))
    X = activations(42, M, M, K)
    note(f"very long rows M={M} K={K}")
    Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"K=2^21 M={M}")
