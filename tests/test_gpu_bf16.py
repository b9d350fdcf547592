"""bf16 activations (X and Y in bf16, packed INT4 weights and fp16 s unchanged) against the
fp64 oracle on every kernel path, at the tolerance derived for bf16 (tests/gpu_helpers.py)."""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from oracle import outliers as ol
from tests.gpu_helpers import (MAX_REL_BF16, REL_L2_BF16, assert_close, note, to_dev,
                               torch_cuda)
from workloads import activations_bf16, awq_scales, bf16_bits_to_f64, to_bf16_bits, weights

pytestmark = pytest.mark.gpu


def bf16_dev(bits):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(
        torch.bfloat16)


def bf16_host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def check(Y, ref, tag):
    return assert_close(Y, ref, tag, REL_L2_BF16, MAX_REL_BF16)


@pytest.mark.parametrize("M,N,K,awq", [
    (1, 4096, 4096, True),       # streaming, whole-row X * s
    (4, 1040, 3584, False),      # streaming, ragged N
    (9, 1024, 14336, True),      # streaming, K windows
    (16, 2048, 4096, True),      # streaming, K windows
    (17, 1024, 2048, True),      # tiled, ragged M
    (40, 528, 2048, True),       # tiled, 48-row tiles
    (64, 4096, 4096, True),      # tiled, split K
    (65, 272, 640, True),        # tiled, 96-row tiles at their lower edge
    (97, 528, 18944, True),      # tiled, 128-row tiles at their lower edge, split K
    (130, 528, 4096, True),      # tiled, 128-row tiles, ragged M across two tiles
    (257, 272, 2048, False),     # tiled, 128-row tiles, three M blocks, ragged
    (300, 1296, 1536, False),    # tiled, ragged M and N
])
def test_bf16_matches_oracle(M, N, K, awq):
    torch_cuda()
    W = weights(20, 0, N, K)
    s = awq_scales(20, 0, K) if awq else None
    xb = activations_bf16(20, 0, M, K)
    note(f"bf16 gemm M={M} N={N} K={K} awq={awq}")
    pw = w4.w4a16_quantize_pack(to_dev(W), None if s is None else to_dev(s))
    Y = w4.w4a16_gemm(bf16_dev(xb), pw, None if s is None else to_dev(s))
    assert str(Y.dtype) == "torch.bfloat16"
    q = oracle.quantize(W, s)
    ref = oracle.gemm(bf16_bits_to_f64(xb), q.q, q.scales, q.zeros, s)
    rel, mx = check(bf16_host(Y), ref, f"bf16 M={M} N={N} K={K}")
    note(f"rel-L2 {rel:.2e} max-rel {mx:.2e}")


@pytest.mark.parametrize("M", [1, 9, 40])
def test_bf16_with_outliers(M):
    torch_cuda()
    N, K = 1024, 4096
    W = weights(21, 0, N, K)
    s = awq_scales(21, 0, K)
    xb = activations_bf16(21, 0, M, K)
    count = ol.page_count(N, K)
    note(f"bf16 outliers M={M}")
    pw = w4.w4a16_quantize_pack_outliers(to_dev(W), to_dev(s), count)
    Y = w4.w4a16_gemm(bf16_dev(xb), pw, to_dev(s))
    ref = ol.gemm(bf16_bits_to_f64(xb), ol.quantize_with_outliers(W, s, count), W, s)
    check(bf16_host(Y), ref, f"bf16 outliers M={M}")


def test_bf16_and_fp16_problems_in_one_grouped_call():
    torch = torch_cuda()
    items, refs, kinds = [], [], []
    for i, (M, N, K, bf) in enumerate([(1, 1024, 4096, True), (1, 512, 2048, False),
                                       (33, 1024, 4096, True), (33, 512, 2048, False)]):
        W = weights(22 + i, 0, N, K)
        s = awq_scales(22 + i, 0, K)
        pw = w4.w4a16_quantize_pack(to_dev(W), to_dev(s))
        q = oracle.quantize(W, s)
        if bf:
            xb = activations_bf16(22 + i, 0, M, K)
            X, Xf = bf16_dev(xb), bf16_bits_to_f64(xb)
        else:
            from workloads import activations
            x16 = activations(22 + i, 0, M, K)
            X, Xf = to_dev(x16), x16.astype(np.float64)
        Y = torch.empty((M, N), dtype=X.dtype, device="cuda")
        items.append((X, pw, to_dev(s), Y))
        refs.append(oracle.gemm(Xf, q.q, q.scales, q.zeros, s))
        kinds.append(bf)
    note("grouped fp16 + bf16")
    w4.GroupedCall(items)()
    for (_, _, _, Y), ref, bf in zip(items, refs, kinds):
        if bf:
            check(bf16_host(Y), ref, "grouped bf16")
        else:
            torch.cuda.synchronize()
            assert_close(Y.cpu().numpy(), ref, "grouped fp16")


def test_bf16_integer_case():
    """Integer weights with codes 0 and 15 in every group, s = 1 and small-integer
    activations: every product and partial sum is exact in fp32, so the bf16 output is the
    exact integer result rounded once to bf16."""
    torch_cuda()
    rng = np.random.default_rng(23)
    N, K, M = 64, 512, 3
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::128] = 0
    q[:, 1::128] = 15
    W = (q - 8).astype(np.float16)            # groups span -8..7: scale 1, zero point 8
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    xb = np.asarray(X, dtype=np.float32).view(np.uint32) >> 16
    pw = w4.w4a16_quantize_pack(to_dev(W), None)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    for path_M in (M, 24):                    # streaming, and tiled with rows repeated
        Xm = np.resize(xb.astype(np.uint16), (path_M, K))
        Y = bf16_host(w4.w4a16_gemm(bf16_dev(Xm), pw))
        ref = np.resize(exact, (path_M, N))
        want = bf16_bits_to_f64(to_bf16_bits(np.asarray(ref, dtype=np.float32)))  # exact -> RNE
        assert np.array_equal(Y, want), path_M


@pytest.mark.parametrize("M,N,K,awq,outl", [
    (9, 1024, 14336, True, False),
    (16, 2048, 4096, True, False),
    (5, 528, 18944, False, False),
    (8, 272, 14336, True, True),
    (16, 1024, 4096, True, True),
])
def test_bf16_prescaled_windows_are_identical(M, N, K, awq, outl):
    """With a workspace, bf16 problems that stage X * s in K windows get it from a
    small first kernel (once per call) instead of computing it in every workgroup:
    the same values, so the outputs are bit-identical to the call without one."""
    torch = torch_cuda()
    W = weights(22, M, N, K)
    s = awq_scales(22, M, K) if awq else None
    sd = None if s is None else to_dev(s)
    pw = (w4.w4a16_quantize_pack_outliers(to_dev(W), sd, count=ol.page_count(N, K)) if outl
          else w4.w4a16_quantize_pack(to_dev(W), sd))
    X = bf16_dev(activations_bf16(22, M, M, K))
    outs = []
    for ws in (True, False):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        call = w4.GroupedCall([(X, pw, sd, Y)], workspace=ws)
        assert (call.ws_bytes > 0) == ws
        note(f"bf16 windows M={M} N={N} K={K} outliers={outl} workspace={call.ws_bytes}")
        call()
        outs.append(bf16_host(Y))
    assert np.array_equal(outs[0], outs[1])
    if not outl:
        q = oracle.quantize(W, s)
        check(outs[0], oracle.gemm(bf16_bits_to_f64(activations_bf16(22, M, M, K)), q.q,
                                   q.scales, q.zeros, s), f"prescaled M={M} N={N} K={K}")


def test_bf16_graph_replay_with_prescale():
    """A grouped bf16 call whose windowed problems use the prescale kernel (two launches
    per call, plus a tiled split-K problem and its reduction), captured in a HIP graph
    and replayed with eager work in between: every replay gives the eager bits."""
    torch = torch_cuda()
    items = []
    for i, (M, N, K) in enumerate([(9, 1024, 14336), (16, 272, 4096), (1, 272, 640),
                                   (64, 272, 4096)]):
        W = weights(23, i, N, K)
        s = awq_scales(23, i, K)
        pw = w4.w4a16_quantize_pack(to_dev(W), to_dev(s))
        X = bf16_dev(activations_bf16(23, i, M, K))
        items.append((X, pw, to_dev(s), torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    call = w4.GroupedCall(items)
    assert call.ws_bytes > 0
    call()
    eager = [bf16_host(it[3]).copy() for it in items]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph capture of a bf16 grouped call with prescaled windows")
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for it in items:
            it[3].fill_(float("nan"))
        call.ws.fill_(255)                     # the workspace holds nothing between calls
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for it, ref in zip(items, eager):
            assert np.array_equal(bf16_host(it[3]), ref), rep
