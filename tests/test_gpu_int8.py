"""INT8 codes (W8A16): the GPU packer against the oracle's INT8 variant, bit for bit, and
the dequantize-matmul on INT8 codes against the fp64 oracle on every kernel path, with fp16
and with bf16 activations.

The streaming kernel takes M <= 16 (whole-row X * s staging when it fits in LDS, K
windows otherwise), the tiled
kernel larger M (with K split across workgroups for the small output grids).  The
tolerance is the fp16 one: INT8 codes decode to exact fp16 values (q - z), as INT4
codes do, so the rounding budget is unchanged.
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import (MAX_REL_BF16, REL_L2_BF16, assert_close, h16_bits, note, to_dev,
                               to_host, torch_cuda)
from workloads import (activations, activations_bf16, awq_scales, bf16_bits_to_f64, to_bf16_bits,
                       weights)

pytestmark = pytest.mark.gpu


def pack8(W, s):
    torch_cuda()
    pw = w4.w4a16_quantize_pack(to_dev(W), None if s is None else to_dev(s), mode=w4.QUANT_ASYM8)
    assert pw.wbits == 8 and pw.wq.numel() == W.size
    return pw


def check_pack_exact(W, s, tag):
    note(f"int8 pack {tag} N={W.shape[0]} K={W.shape[1]} awq={s is not None}")
    pw = pack8(W, s)
    ref = oracle.quantize(W, s, bits=8)
    assert np.array_equal(to_host(pw.wq), oracle.pack_codes8(ref.q)), tag
    assert np.array_equal(h16_bits(to_host(pw.scales)), h16_bits(oracle.pack_meta(ref.scales))), tag
    assert np.array_equal(h16_bits(to_host(pw.zeros)), h16_bits(oracle.pack_meta(ref.zeros))), tag


@pytest.mark.parametrize("awq", [False, True])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 640), (1024, 4096)])
def test_pack_int8_exact(N, K, awq):
    check_pack_exact(weights(21, 1, N, K), awq_scales(21, 1, K) if awq else None, f"{N}x{K}")


def test_pack_int8_edge_groups():
    rng = np.random.default_rng(23)
    N, K = 64, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[0:16, 0:128] = 0                                  # all-zero group
    W[16, 128:256] = np.float16(-0.0)                   # signed zeros only
    W[17, 256:384] = 3.0                                # constant positive group
    W[18, 256:384] = -3.0                               # constant negative group
    W[19, 384:512] = np.float16(6e-8)                   # subnormal weights -> tiny scale
    W[21, 640:768] = np.float16(60000.0)                # near the top of fp16
    W[22, 768:896] *= 500                               # outlier-heavy group
    W[23, 896:1024] = np.linspace(-1, 1, 128).astype(np.float16)
    check_pack_exact(W, None, "edge groups")
    s = np.exp(rng.uniform(-1, 1, K)).astype(np.float16)
    check_pack_exact(W, s, "edge groups + awq")


def test_pack_int8_codes_span_the_byte():
    """Groups whose weights take both signs use nearly all of 0..255: the minimum codes
    to about 0 and the maximum to about 255 (scale is range / 255, rounded up)."""
    W = weights(22, 0, 272, 640)
    pw = pack8(W, None)
    codes = to_host(pw.wq)
    q = oracle.unpack_codes8(codes, 272, 640)
    per_group = q.reshape(272, 5, 128)
    assert per_group.max(axis=2).min() >= 250 and per_group.min(axis=2).max() <= 5
    assert np.array_equal(q, oracle.quantize(W, None, bits=8).q)


_CACHE = {}


def case(N, K, awq=True, key=24):
    k = (N, K, awq, key)
    if k not in _CACHE:
        W = weights(key, N + K, N, K)
        s = awq_scales(key, N + K, K) if awq else None
        _CACHE[k] = (pack8(W, s), s, oracle.quantize(W, s, bits=8))
    return _CACHE[k]


def gemm8(X, pw, s):
    return to_host(w4.w4a16_gemm(to_dev(X), pw, None if s is None else to_dev(s)))


@pytest.mark.parametrize("awq", [False, True])
@pytest.mark.parametrize("M", [1, 2, 5, 9, 16, 17, 40, 64, 80, 129, 300])
def test_gemm_int8_matches_oracle(M, awq):
    N, K = 272, 640
    pw, s, ref = case(N, K, awq)
    X = activations(24, M, M, K, outliers=True)
    note(f"int8 gemm M={M} N={N} K={K} awq={awq} path={w4.w4a16_select_path(M, N, K)}")
    assert_close(gemm8(X, pw, s), oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"M={M}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 14336), (16, 64, 14336), (9, 48, 18944),
                                   (2, 1024, 128), (16, 16, 4096), (5, 528, 1152)])
def test_gemm_int8_streaming_shapes(M, N, K):
    """Whole-row staging, and K windows where X * s of the call exceeds the 96 KiB
    staging limit (M = 16 at K = 14336 and 4096, M = 9 at K = 18944)."""
    pw, s, ref = case(N, K)
    X = activations(25, M, M, K)
    note(f"int8 streaming M={M} N={N} K={K}")
    assert_close(gemm8(X, pw, s), oracle.gemm(X, ref.q, ref.scales, ref.zeros, s),
                 f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(40, 272, 4096), (64, 272, 14336), (257, 16, 4096),
                                   (17, 1024, 2048), (100, 528, 1152)])
def test_gemm_int8_split_k(M, N, K):
    """Tiled shapes whose small output grid splits K across workgroups: matches the
    oracle, and two calls give the same bits (the partials add in a fixed order)."""
    torch = torch_cuda()
    pw, s, ref = case(N, K, key=26)
    X = activations(26, M, M, K, outliers=True)
    Xd, sd = to_dev(X), to_dev(s)
    call = w4.GroupedCall([(Xd, pw, sd, torch.empty((M, N), dtype=torch.float16, device="cuda"))])
    note(f"int8 split-K M={M} N={N} K={K} workspace={call.ws_bytes}")
    call()
    a = to_host(call.items[0][3]).copy()
    call()
    b = to_host(call.items[0][3])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert_close(a, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"split {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 9, 16, 24, 64])
def test_gemm_int8_integer_case_bit_exact(M):
    """s = 1, integer weights -128..127 with both ends in every group: scale 1, zero
    point 128, so the codes are the weights + 128; X in {-1, 0, 1} and sparse enough
    that every |Y| stays within 2048, where fp16 holds every integer: Y is exact."""
    rng = np.random.default_rng(27)
    N, K = 64, 256
    W = rng.integers(-128, 128, size=(N, K))
    W[:, 0::128], W[:, 1::128] = -128, 127
    W = W.astype(np.float16)
    X = (rng.integers(-1, 2, size=(M, K)) * (rng.random((M, K)) < 0.06)).astype(np.float16)
    X[:, 0:2] = 0
    ref = oracle.quantize(W, None, bits=8)
    assert np.all(ref.scales == 1) and np.all(ref.zeros == 128)
    Yref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.abs(Yref).max() <= 2048
    note(f"int8 integer case M={M}")
    Y = gemm8(X, pack8(W, None), None)
    assert np.array_equal(Y.astype(np.float64), Yref)


def test_gemm_int8_zero_weights_give_zero():
    W = np.zeros((32, 256), np.float16)
    pw = pack8(W, None)
    for M in (3, 40):
        note(f"int8 zero weights M={M}")
        assert np.all(gemm8(activations(28, M, M, 256), pw, None) == 0)


def test_grouped_mixes_int4_and_int8():
    """One grouped call over INT4 and INT8 problems on both kernels: the launcher keeps
    each code width in its own kernel instance; every output matches the oracle and
    the single call."""
    torch_cuda()
    specs = [(1, 272, 640, 8), (1, 272, 640, 4), (9, 528, 1152, 8), (40, 272, 640, 4),
             (40, 272, 640, 8), (3, 48, 384, 4), (16, 64, 14336, 8), (100, 16, 4096, 8)]
    items, refs = [], []
    for i, (M, N, K, bits) in enumerate(specs):
        W = weights(29, i, N, K)
        s = awq_scales(29, i, K)
        if bits == 8:
            pw, ref = pack8(W, s), oracle.quantize(W, s, bits=8)
        else:
            pw, ref = w4.w4a16_quantize_pack(to_dev(W), to_dev(s)), oracle.quantize(W, s)
        X = activations(29, i, M, K)
        items.append((to_dev(X), pw, to_dev(s)))
        refs.append(oracle.gemm(X, ref.q, ref.scales, ref.zeros, s))
    note(f"grouped int4/int8 call over {len(specs)} problems")
    Ys = [to_host(y) for y in w4.w4a16_gemm_grouped(items)]
    for (M, N, K, bits), (Xd, pw, sd), Y, Yref in zip(specs, items, Ys, refs):
        assert_close(Y, Yref, f"grouped {M}x{N}x{K} int{bits}")
        assert_close(Y, to_host(w4.w4a16_gemm(Xd, pw, sd)), f"vs single {M}x{N}x{K} int{bits}")


def test_int8_full_size_decode_sampled():
    """An 8B-class decode projection (N = 4096, K = 14336) in INT8 at M = 1 and M = 16
    (windowed): packed codes of sampled row blocks bit-exact, and 512 sampled outputs
    against the oracle computed row by row."""
    torch_cuda()
    N, K = 4096, 14336
    W = weights(30, 0, N, K)
    s = awq_scales(30, 0, K)
    note(f"int8 full-size pack N={N} K={K}")
    pw = pack8(W, s)
    codes = to_host(pw.wq)
    scales = to_host(pw.scales)
    rng = np.random.default_rng(30)
    rows = np.sort(rng.choice(N, 512, replace=False))
    ref = oracle.quantize(W[rows], s, bits=8)        # per-row (per-group) results hold per row
    q_gpu = codes[oracle.byte_address8(rows[:, None], np.arange(K)[None, :], N, K)]
    assert np.array_equal(q_gpu, ref.q)
    sc_gpu = oracle.unpack_meta(scales, N, K)[rows]
    assert np.array_equal(h16_bits(sc_gpu), h16_bits(ref.scales))
    for M in (1, 16):
        X = activations(30, M, M, K)
        note(f"int8 full-size gemm M={M}")
        Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
        Yref = oracle.gemm(X, ref.q, ref.scales, ref.zeros, s)
        assert_close(Y[:, rows], Yref, f"full-size M={M}")


def bf16_dev(bits):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def bf16_host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("M,N,K", [(1, 272, 640), (5, 528, 1152), (1, 64, 14336),
                                   (9, 48, 18944), (16, 64, 14336), (16, 16, 4096),
                                   (17, 1024, 2048), (64, 272, 4096), (300, 272, 640)])
def test_gemm_int8_bf16_matches_oracle(M, N, K):
    """INT8 codes with bf16 activations and outputs on every path (whole-row and
    windowed streaming, tiled with and without split K), at the bf16 tolerance."""
    torch_cuda()
    pw, s, ref = case(N, K, key=31)
    xb = activations_bf16(31, M, M, K, outliers=True)
    note(f"int8 bf16 gemm M={M} N={N} K={K} path={w4.w4a16_select_path(M, N, K)}")
    Y = w4.w4a16_gemm(bf16_dev(xb), pw, to_dev(s))
    assert str(Y.dtype) == "torch.bfloat16"
    assert_close(bf16_host(Y), oracle.gemm(bf16_bits_to_f64(xb), ref.q, ref.scales, ref.zeros, s),
                 f"int8 bf16 {M}x{N}x{K}", REL_L2_BF16, MAX_REL_BF16)


@pytest.mark.parametrize("M", [1, 9, 40])
def test_gemm_int8_bf16_integer_case(M):
    """The integer case with bf16 activations: Y is the exact integer result (within
    2048, so exact in fp32 partial sums), rounded once to bf16."""
    rng = np.random.default_rng(32)
    N, K = 64, 256
    W = rng.integers(-128, 128, size=(N, K))
    W[:, 0::128], W[:, 1::128] = -128, 127
    W = W.astype(np.float16)
    X = (rng.integers(-1, 2, size=(M, K)) * (rng.random((M, K)) < 0.06)).astype(np.float32)
    X[:, 0:2] = 0
    Yref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.abs(Yref).max() <= 2048
    note(f"int8 bf16 integer case M={M}")
    Y = bf16_host(w4.w4a16_gemm(bf16_dev(to_bf16_bits(X)), pack8(W, None)))
    assert np.array_equal(Y, bf16_bits_to_f64(to_bf16_bits(Yref.astype(np.float32))))


@pytest.mark.parametrize("M,N,K", [(9, 1024, 14336), (16, 272, 4096)])
def test_int8_bf16_prescaled_windows_are_identical(M, N, K):
    """bf16 windows over INT8 codes: prescaled X * s (with a workspace) gives the same
    bits as the in-kernel scaling (without one)."""
    torch = torch_cuda()
    pw, s, _ = case(N, K, key=33)
    X = bf16_dev(activations_bf16(33, M, M, K))
    outs = []
    for ws in (True, False):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        call = w4.GroupedCall([(X, pw, to_dev(s), Y)], workspace=ws)
        assert (call.ws_bytes > 0) == ws
        note(f"int8 bf16 windows M={M} N={N} K={K} workspace={call.ws_bytes}")
        call()
        outs.append(bf16_host(Y))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("N,K,awq", [(16, 128, False), (272, 640, True), (1024, 1024, True)])
def test_int8_outlier_pack_matches_oracle(N, K, awq):
    """fp16 outliers over INT8 codes: the row-compressed outliers and the packed INT8
    rest bit-exact with the oracle's split (count 0, one, the page's share, many)."""
    from oracle import outliers as ol
    W = weights(34, 1, N, K)
    s = awq_scales(34, 1, K) if awq else None
    for count in (0, 1, ol.page_count(N, K), 37 * N):
        note(f"int8 outlier pack N={N} K={K} count={count}")
        pw = w4.w4a16_quantize_pack_outliers(to_dev(W), None if s is None else to_dev(s), count,
                                             w4.QUANT_ASYM8)
        assert pw.wbits == 8
        ref = ol.quantize_with_outliers(W, s, count, bits=8)
        assert np.array_equal(to_host(pw.o_row_ptr), ref.row_ptr)
        assert np.array_equal(to_host(pw.o_col), ref.col)
        assert np.array_equal(h16_bits(to_host(pw.o_val)), h16_bits(ref.val))
        assert np.array_equal(to_host(pw.wq), oracle.pack_codes8(ref.quant.q))
        assert np.array_equal(h16_bits(to_host(pw.scales)),
                              h16_bits(oracle.pack_meta(ref.quant.scales)))
        assert np.array_equal(h16_bits(to_host(pw.zeros)),
                              h16_bits(oracle.pack_meta(ref.quant.zeros)))


@pytest.mark.parametrize("bf", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 272, 640), (5, 528, 1152), (9, 48, 18944),
                                   (16, 64, 14336), (40, 272, 4096), (300, 272, 640)])
def test_gemm_int8_with_outliers(M, N, K, bf):
    """INT8 codes plus fp16 outliers (the page's share, and extra ones planted in one
    group) on every path, fp16 and bf16 activations, against the oracle's merged
    weight."""
    from oracle import outliers as ol
    torch_cuda()
    W = weights(35, N + K, N, K)
    s = awq_scales(35, N + K, K)
    W[3, 130:134] = np.float16(0.9)             # several kept weights in one group
    count = ol.page_count(N, K) + 4
    pw = w4.w4a16_quantize_pack_outliers(to_dev(W), to_dev(s), count, w4.QUANT_ASYM8)
    res = ol.quantize_with_outliers(W, s, count, bits=8)
    assert res.mask[3, 130:134].all()
    note(f"int8 outliers gemm M={M} N={N} K={K} bf16={bf}")
    if bf:
        xb = activations_bf16(35, M, M, K, outliers=True)
        Y = bf16_host(w4.w4a16_gemm(bf16_dev(xb), pw, to_dev(s)))
        assert_close(Y, ol.gemm(bf16_bits_to_f64(xb), res, W, s), f"int8+out bf16 {M}x{N}x{K}",
                     REL_L2_BF16, MAX_REL_BF16)
    else:
        X = activations(35, M, M, K, outliers=True)
        Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
        assert_close(Y, ol.gemm(X, res, W, s), f"int8+out {M}x{N}x{K}")
