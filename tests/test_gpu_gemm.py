"""GPU dequantize-matmul vs the fp64 oracle, element by element, on both kernel paths.

Shapes span several packed tiles and ragged tails: N = 272 is 17 row tiles (not a
multiple of the tiled kernel's 128-row block), K = 640 is 5 groups, and M runs
over every value from 1 to 17 plus ragged larger batches.
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, note, to_dev, to_host, torch_cuda
from workloads import activations, awq_scales, weights

pytestmark = pytest.mark.gpu

PATHS = {"auto": w4.PATH_AUTO, "skinny": w4.PATH_SKINNY, "tiled": w4.PATH_TILED,
         "window": w4.PATH_SKINNY_WINDOW}


def packed_case(N, K, awq, key=2, mat=0):
    W = weights(key, mat, N, K)
    s = awq_scales(key, mat, K) if awq else None
    torch_cuda()
    pw = w4.w4a16_quantize_pack(to_dev(W), None if s is None else to_dev(s))
    ref = oracle.quantize(W, s)
    return pw, s, ref


_CACHE = {}


def cached_case(N, K, awq):
    key = (N, K, awq)
    if key not in _CACHE:
        _CACHE[key] = packed_case(N, K, awq)
    return _CACHE[key]


def run(X, pw, s, path):
    Xd = to_dev(X)
    sd = None if s is None else to_dev(s)
    return to_host(w4.w4a16_gemm_path(Xd, pw, sd, PATHS[path]))


@pytest.mark.parametrize("path", ["skinny", "window", "tiled"])
@pytest.mark.parametrize("awq", [False, True])
@pytest.mark.parametrize("M", list(range(1, 18)))
def test_small_M_all_paths(M, awq, path):
    N, K = 272, 640
    pw, s, ref = cached_case(N, K, awq)
    X = activations(2, 0, M, K)
    note(f"gemm path={path} M={M} N={N} K={K} awq={awq}")
    Y = run(X, pw, s, path)
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"M={M} {path}")


@pytest.mark.parametrize("path", ["auto", "skinny", "window", "tiled"])
@pytest.mark.parametrize("M", [31, 64, 100, 128, 129, 257])
def test_larger_M(M, path):
    N, K = 272, 640
    pw, s, ref = cached_case(N, K, True)
    X = activations(2, 1, M, K, outliers=True)
    note(f"gemm path={path} M={M} N={N} K={K}")
    Y = run(X, pw, s, path)
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"M={M} {path}")


@pytest.mark.parametrize("N,K", [(16, 128), (16, 4096), (1024, 128), (528, 1152), (64, 14336)])
@pytest.mark.parametrize("M", [1, 5, 33])
def test_shape_extremes(N, K, M):
    pw, s, ref = packed_case(N, K, True, key=3, mat=N + K)
    X = activations(3, 0, M, K)
    note(f"gemm auto M={M} N={N} K={K}")
    Y = run(X, pw, s, "auto")
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"{M}x{N}x{K}")


@pytest.mark.parametrize("N,K", [(16, 128), (16, 4096), (1024, 128), (528, 1152), (64, 14336),
                                 (48, 18944)])
@pytest.mark.parametrize("M", [2, 9, 16])
def test_window_shapes(N, K, M):
    """K windows of every width the launcher picks (1..8 chunks), windows that run
    past K, and row blocks that do not fill a workgroup."""
    pw, s, ref = packed_case(N, K, True, key=3, mat=N + K)
    X = activations(3, 1, M, K, outliers=True)
    note(f"gemm window M={M} N={N} K={K}")
    Y = run(X, pw, s, "window")
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(40, 272, 4096), (64, 272, 14336), (100, 528, 1152),
                                   (257, 16, 4096), (64, 48, 18944), (17, 1024, 2048)])
def test_split_k(M, N, K):
    """Large-M calls whose output blocks are too few for the GPU split K across
    workgroups (fp32 partials in the workspace, reduced in a fixed order): the result
    matches the oracle, is reproducible, and agrees with the unsplit kernel."""
    torch_cuda()
    pw, s, ref = packed_case(N, K, True, key=11, mat=N + K)
    assert w4.w4a16_select_path(M, N, K) == w4.PATH_TILED
    X = activations(11, M, M, K, outliers=True)
    Xd, sd = to_dev(X), to_dev(s)
    call = w4.GroupedCall([(Xd, pw, sd, w4._torch().empty((M, N), dtype=w4._torch().float16,
                                                         device="cuda"))])
    assert call.ws_bytes > 0, "this shape is expected to split K"
    note(f"split-K M={M} N={N} K={K} workspace={call.ws_bytes}")
    call()
    a = to_host(call.items[0][3]).copy()
    call()
    b = to_host(call.items[0][3])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert_close(a, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"split {M}x{N}x{K}")
    unsplit = run(X, pw, s, "tiled")
    assert_close(a, unsplit, f"split vs unsplit {M}x{N}x{K}")


@pytest.mark.parametrize("path", ["skinny", "window", "tiled"])
@pytest.mark.parametrize("M", [1, 9, 40])
def test_symmetric_weights(M, path):
    """Weights packed on the signed -7..7 grid run through the same kernels."""
    torch_cuda()
    N, K = 272, 1152
    W = weights(12, 0, N, K)
    s = awq_scales(12, 0, K)
    pw = w4.w4a16_quantize_pack(to_dev(W), to_dev(s), mode=w4.QUANT_SYM)
    ref = oracle.quantize_symmetric(W, s)
    X = activations(12, 0, M, K)
    note(f"symmetric weights path={path} M={M}")
    Y = run(X, pw, s, path)
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"sym M={M} {path}")


@pytest.mark.parametrize("gran,mode", [("channel", w4.QUANT_ASYM_CHANNEL),
                                       ("tensor", w4.QUANT_ASYM_TENSOR)])
@pytest.mark.parametrize("M,path", [(1, "skinny"), (9, "window"), (40, "tiled")])
def test_coarser_granularity_weights(gran, mode, M, path):
    """Per-channel and per-tensor packs (their scale repeated in every group) run through
    the same kernels."""
    torch_cuda()
    N, K = 272, 1152
    W = weights(13, 0, N, K)
    s = awq_scales(13, 0, K)
    pw = w4.w4a16_quantize_pack(to_dev(W), to_dev(s), mode=mode)
    ref = oracle.quantize(W, s, gran)
    X = activations(13, 0, M, K)
    note(f"{gran} weights path={path} M={M}")
    Y = run(X, pw, s, path)
    assert_close(Y, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"{gran} M={M} {path}")


@pytest.mark.parametrize("path", ["skinny", "window", "tiled"])
def test_integer_case_bit_exact(path):
    """Pin P5: s = 1, integer weights with codes 0 and 15 in every group -> scale 1,
    zero point 8; X in {-1, 0, 1}: Y is an integer matmul, exact in fp16."""
    rng = np.random.default_rng(9)
    N, K, M = 64, 256, 24
    W = rng.integers(-8, 8, size=(N, K))
    W[:, 0::128] = -8
    W[:, 1::128] = 7
    W = W.astype(np.float16)
    X = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    ref = oracle.quantize(W, None)
    assert np.all(ref.scales == 1) and np.all(ref.zeros == 8)
    torch_cuda()
    pw = w4.w4a16_quantize_pack(to_dev(W))
    note(f"integer case path={path}")
    Y = run(X, pw, None, path)
    Yref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(Y.astype(np.float64), Yref)


def test_zero_weights_give_zero():
    N, K, M = 32, 256, 3
    W = np.zeros((N, K), np.float16)
    torch_cuda()
    pw = w4.w4a16_quantize_pack(to_dev(W))
    X = activations(4, 0, M, K)
    for path in ("skinny", "window", "tiled"):
        note(f"zero weights path={path}")
        assert np.all(run(X, pw, None, path) == 0)


def test_deterministic_and_row_independent():
    """Same inputs twice -> identical bits; row 0 of a batch equals the M = 1 result
    computed by the same kernel (pin P6's batch identity, on the GPU)."""
    N, K = 1024, 4096
    pw, s, _ = packed_case(N, K, True, key=5)
    for path, M in (("skinny", 9), ("window", 9), ("tiled", 40)):
        X = activations(5, 0, M, K)
        note(f"determinism path={path} M={M}")
        a = run(X, pw, s, path)
        b = run(X, pw, s, path)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    X = activations(5, 0, 5, K)
    full = run(X, pw, s, "skinny")
    one = run(X[:1], pw, s, "skinny")
    assert np.array_equal(full[:1].view(np.uint16), one.view(np.uint16))


def test_empty_batch():
    torch = torch_cuda()
    pw, s, _ = cached_case(272, 640, False)
    X = torch.empty((0, 640), dtype=torch.float16, device="cuda")
    Y = w4.w4a16_gemm(X, pw)
    assert tuple(Y.shape) == (0, 272)


def test_grouped_matches_single_calls_and_oracle():
    """One grouped call over problems of mixed shapes, M (including 0 and a tiled-path M)
    and AWQ scales: each output matches the oracle and the single-call output within
    tolerance, and the same call again gives the same bits.  Nine streaming problems
    take two launches; one problem (M=16, K=4096) needs K windows, so its launch is a
    mixed one: that problem's workgroups walk windows, the others stage whole rows."""
    torch_cuda()
    cases = [(1, 272, 640, True), (1, 16, 128, False), (5, 528, 1152, True), (0, 64, 256, False),
             (40, 272, 640, False), (16, 1024, 4096, True), (3, 48, 384, False),
             (9, 128, 1280, True), (2, 64, 14336, True), (1, 32, 256, False), (7, 80, 512, True)]
    items, refs = [], []
    for i, (M, N, K, awq) in enumerate(cases):
        pw, s, ref = packed_case(N, K, awq, key=8, mat=i)
        X = activations(8, i, M, K)
        sd = None if s is None else to_dev(s)
        items.append((to_dev(X), pw, sd))
        refs.append(oracle.gemm(X, ref.q, ref.scales, ref.zeros, s))
    note(f"grouped call over {len(cases)} problems")
    Ys = [to_host(y) for y in w4.w4a16_gemm_grouped(items)]
    again = [to_host(y) for y in w4.w4a16_gemm_grouped(items)]
    for (M, N, K, _), (Xd, pw, sd), Y, Y2, Yref in zip(cases, items, Ys, again, refs):
        assert Y.shape == (M, N)
        if M == 0:
            continue
        assert_close(Y, Yref, f"grouped {M}x{N}x{K}")
        assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16)), f"{M}x{N}x{K}"
        single = to_host(w4.w4a16_gemm(Xd, pw, sd))
        assert_close(Y, single, f"grouped vs single {M}x{N}x{K}")


@pytest.mark.parametrize("M", [4, 5, 9])
def test_mixed_launch_verify_layer(M):
    """The 8B layer's seven shapes at a verify batch (fewer rows of W each).  At M = 4
    and 5 down's X * s (K = 14336, 115 and 143 KB) exceeds the 8-wave workgroups' stage
    but fits the 16-wave ones', so the launch stages whole rows in 16-wave workgroups;
    at M = 9 it does not fit at all, and one launch mixes whole-row staging and K
    windows.  Each output matches the oracle and the single call, and repeats bit for
    bit."""
    torch_cuda()
    shapes = [(256, 4096), (64, 4096), (64, 4096), (256, 4096), (512, 4096), (512, 4096),
              (256, 14336)]
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        pw, s, ref = packed_case(N, K, True, key=11, mat=i)
        X = activations(11, 10 * M + i, M, K)
        items.append((to_dev(X), pw, to_dev(s)))
        refs.append(oracle.gemm(X, ref.q, ref.scales, ref.zeros, s))
    note(f"mixed streaming launch, 8B layer shapes, M={M}")
    Ys = [to_host(y) for y in w4.w4a16_gemm_grouped(items)]
    again = [to_host(y) for y in w4.w4a16_gemm_grouped(items)]
    for (N, K), (Xd, pw, sd), Y, Y2, Yref in zip(shapes, items, Ys, again, refs):
        assert_close(Y, Yref, f"mixed {M}x{N}x{K}")
        assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16)), f"{M}x{N}x{K}"
        assert_close(Y, to_host(w4.w4a16_gemm(Xd, pw, sd)), f"mixed vs single {M}x{N}x{K}")


@pytest.mark.parametrize("K,wide", [(15232, True), (15360, False)])
def test_wide_stage_boundary(K, wide):
    """M = 5 rows of X * s at the edge of the 16-wave whole-row stage (150 KB):
    K = 15232 fits (152,400 bytes with the row padding) and the call stages whole
    rows; K = 15360 does not (153,680 bytes) and walks K windows.  Either way, with a
    second problem that fits the 8-wave stage, the outputs match the oracle."""
    torch_cuda()
    M = 5
    items, refs = [], []
    for i, (N, KK) in enumerate([(64, K), (48, 4096)]):
        pw, s, ref = packed_case(N, KK, True, key=13, mat=i)
        X = activations(13, 20 + i, M, KK)
        items.append((to_dev(X), pw, to_dev(s)))
        refs.append(oracle.gemm(X, ref.q, ref.scales, ref.zeros, s))
    note(f"wide stage boundary M={M} K={K} (whole rows: {wide})")
    for Y, Yref, (Xd, pw, sd) in zip(w4.w4a16_gemm_grouped(items), refs, items):
        assert_close(to_host(Y), Yref, f"wide boundary K={K} N={pw.N}")
        assert_close(to_host(w4.w4a16_gemm(Xd, pw, sd)), Yref, f"single K={K} N={pw.N}")


def test_graph_replay_matches_eager():
    """A grouped call captured in a HIP graph and replayed several times, with eager
    work and synchronisations in between, gives the eager result on every replay."""
    torch = torch_cuda()
    items = []
    for i, (M, N, K, awq) in enumerate([(1, 1024, 4096, True), (1, 272, 640, False),
                                        (5, 528, 1152, True), (40, 272, 640, True),
                                        (64, 272, 4096, False)]):
        pw, s, _ = packed_case(N, K, awq, key=10, mat=i)
        X = to_dev(activations(10, i, M, K))
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        items.append((X, pw, None if s is None else to_dev(s), Y))
    call = w4.GroupedCall(items)
    assert call.ws_bytes > 0  # the M = 64 problem splits K: the reduction runs in the graph
    call()
    eager = [to_host(it[3]).copy() for it in items]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph capture of a grouped call")
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for it in items:
            it[3].fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for it, ref in zip(items, eager):
            assert np.array_equal(to_host(it[3]).view(np.uint16), ref.view(np.uint16)), rep


@pytest.mark.parametrize("awq", [False, True])
@pytest.mark.parametrize("M,N,K", [(17, 272, 640), (31, 272, 4096), (32, 48, 18944),
                                   (33, 272, 640), (40, 528, 1152), (48, 528, 1152),
                                   (49, 272, 4096), (64, 48, 18944),
                                   (65, 272, 640), (96, 272, 4096), (97, 48, 18944),
                                   (100, 528, 1152), (128, 256, 4096),
                                   (129, 272, 640), (257, 16, 4096), (300, 1024, 2048),
                                   (520, 784, 1408)])
def test_dma_tiled_kernel(M, N, K, awq):
    """The tiled kernel with X * s brought into LDS by DMA (fp16 activations, INT4 codes;
    32-, 48-, 64-, 96- or 128-row wave tiles, the fewest that cover M; each size at and
    past its edge): through w4a16_gemm, which passes
    a workspace (X * s
    prescaled there when s is given; K split where the blocks are few), and through the
    forced tiled path without a workspace (X straight from its buffer when s is null,
    else the register-staged kernel).  Ragged M (rows past M re-read row M - 1 and are not
    stored), N not a multiple of 256, K a multiple of 128 but not of 512."""
    pw, s, ref = packed_case(N, K, awq, key=12, mat=N + K)
    X = activations(12, M, M, K, outliers=True)
    want = oracle.gemm(X, ref.q, ref.scales, ref.zeros, s)
    note(f"dma tiled M={M} N={N} K={K} awq={awq}")
    Y = to_host(w4.w4a16_gemm(to_dev(X), pw, None if s is None else to_dev(s)))
    assert_close(Y, want, f"dma {M}x{N}x{K} awq={awq}")
    note(f"dma tiled forced path M={M} N={N} K={K} awq={awq}")
    assert_close(run(X, pw, s, "tiled"), want, f"tiled path {M}x{N}x{K} awq={awq}")


@pytest.mark.parametrize("M", [40, 130])
def test_dma_shared_activation_prescale(M):
    """A grouped call whose problems share X and s (the q, k and v projections of one
    layer input) prescales X * s once and all of them read it; a fourth problem with its
    own s in the same call gets its own copy.  Each output matches the oracle."""
    torch_cuda()
    K = 1152
    s = awq_scales(21, 0, K)
    s2 = awq_scales(21, 1, K)
    X = activations(21, 0, M, K, outliers=True)
    Xd, sd, s2d = to_dev(X), to_dev(s), to_dev(s2)
    cases = []
    for j, (N, sv, svd) in enumerate([(272, s, sd), (48, s, sd), (48, s, sd), (528, s2, s2d)]):
        W = weights(21, 10 + j, N, K)
        pw = w4.w4a16_quantize_pack(to_dev(W), svd)
        cases.append((pw, sv, svd, oracle.quantize(W, sv), N))
    T = w4._torch()
    items = [(Xd, pw, svd, T.empty((M, N), dtype=T.float16, device="cuda"))
             for pw, sv, svd, ref, N in cases]
    note(f"shared-activation prescale M={M}")
    call = w4.GroupedCall(items)
    call()
    for (pw, sv, svd, ref, N), it in zip(cases, items):
        assert_close(to_host(it[3]), oracle.gemm(X, ref.q, ref.scales, ref.zeros, sv),
                     f"shared X*s M={M} N={N}")


def test_dma_one_slice_blocks_at_small_m():
    """At M <= 64 a launch with more 64 x 128 blocks than two-slice slots takes blocks of
    one K slice (the launch model prefers four-wave blocks, four per CU, there): a
    131072 x 256 matrix at M = 40 has 1024 blocks.  Whole-matrix packing on the GPU; the
    oracle checks 3 sampled 16-row blocks (first, last, one inside) of the output."""
    torch_cuda()
    N, K, M = 131072, 256, 40
    W = weights(23, 0, N, K)
    s = awq_scales(23, 0, K)
    X = activations(23, 0, M, K)
    pw = w4.w4a16_quantize_pack(to_dev(W), to_dev(s))
    note(f"dma one-slice M={M} N={N} K={K}")
    Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
    assert np.isfinite(Y.astype(np.float32)).all()
    for b in (0, N // 16 // 2 + 3, N // 16 - 1):
        rows = slice(16 * b, 16 * b + 16)
        ref = oracle.quantize(W[rows], s)
        assert_close(Y[:, rows], oracle.gemm(X, ref.q, ref.scales, ref.zeros, s),
                     f"one-slice block {b}")


def test_activations_past_the_dma_buffer_range():
    """M * K * 2 >= 2^31 bytes of X: the DMA-staged kernel's buffer resource cannot
    cover X, so the call takes the register-staged tiled kernel (64-bit row offsets).
    M = 65600, K = 16384 (2.15 GB of X), N = 272 (not a multiple of the block width),
    AWQ s; the oracle checks sampled rows of Y, first and last included."""
    torch_cuda()
    M, N, K = 65600, 272, 16384
    assert M * K * 2 >= 1 << 31
    pw, s, ref = packed_case(N, K, True, key=24, mat=0)
    X = activations(24, 1, M, K)
    note(f"large X M={M} N={N} K={K}")
    Y = to_host(w4.w4a16_gemm(to_dev(X), pw, to_dev(s)))
    rng = np.random.default_rng(24)
    rows = np.unique(np.concatenate([[0, 1, M - 1], rng.choice(M, 40, replace=False)]))
    assert_close(Y[rows], oracle.gemm(X[rows], ref.q, ref.scales, ref.zeros, s), "large X rows")
    assert np.isfinite(Y.astype(np.float32)).all()
