"""The entry points without a workspace argument (w4a16_gemm, w4a16_gemm_grouped)
split K through the library's shared scratch: the same bits as the grouped call with
a caller workspace, calls on two streams ordered by the library's event (no race),
and under stream capture the unsplit path."""
import ctypes

import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import (MAX_REL_BF16, REL_L2_BF16, assert_close, note, to_dev, to_host,
                               torch_cuda)
from workloads import activations, awq_scales, weights

pytestmark = pytest.mark.gpu

# (M, N, K, awq): each splits K with a workspace (few output blocks, long rows)
SHAPES = [(64, 528, 4096, False), (64, 48, 18944, True), (40, 272, 1152, True),
          (100, 256, 4096, True), (17, 1024, 2048, False)]


def case(i, M, N, K, awq):
    W = weights(31, i, N, K)
    s = awq_scales(31, i, K) if awq else None
    pw = w4.w4a16_quantize_pack(to_dev(W), None if s is None else to_dev(s))
    X = activations(31, i, M, K)
    return W, s, pw, X


def c_gemm(Xd, pw, sd, out, stream):
    """The C-ABI w4a16_gemm itself (no workspace argument)."""
    rc = w4.lib().w4a16_gemm(Xd.data_ptr(), pw.wq.data_ptr(), pw.scales.data_ptr(),
                             pw.zeros.data_ptr(), None if sd is None else sd.data_ptr(),
                             out.data_ptr(), Xd.shape[0], pw.N, pw.K, ctypes.c_void_p(stream))
    assert rc == 0, rc


def test_gemm_uses_the_workspace_split():
    torch = torch_cuda()
    st = torch.cuda.current_stream().cuda_stream
    for i, (M, N, K, awq) in enumerate(SHAPES):
        W, s, pw, X = case(i, M, N, K, awq)
        Xd, sd = to_dev(X), None if s is None else to_dev(s)
        call = w4.GroupedCall([(Xd, pw, sd, torch.empty((M, N), dtype=torch.float16,
                                                        device="cuda"))])
        assert 0 < call.ws_bytes <= w4.SHARED_SCRATCH_BYTES, (M, N, K, call.ws_bytes)
        note(f"shared scratch gemm M={M} N={N} K={K} awq={awq}")
        call()
        want = to_host(call.items[0][3])
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        c_gemm(Xd, pw, sd, out, st)
        got = to_host(out)
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), (M, N, K)
        if i < 2:
            ref = oracle.quantize(W, s)
            assert_close(got, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"M={M} N={N}")


def test_grouped_without_workspace_matches_workspace_call():
    torch = torch_cuda()
    items = []
    for i, (M, N, K, awq) in enumerate(SHAPES):
        W, s, pw, X = case(i, M, N, K, awq)
        items.append((to_dev(X), pw, None if s is None else to_dev(s),
                      torch.empty((M, N), dtype=torch.float16, device="cuda")))
    note("shared scratch grouped call")
    ws = w4.GroupedCall(items)
    ws()
    want = [to_host(it[3]).copy() for it in items]
    for it in items:
        it[3].fill_(float("nan"))
    w4.GroupedCall(items, workspace=False)()
    for it, w in zip(items, want):
        assert np.array_equal(to_host(it[3]).view(np.uint16), w.view(np.uint16))


def test_calls_on_two_streams_do_not_race():
    """Alternating calls on two streams, no synchronisation between them: each waits for
    the previous one's use of the shared scratch, so every output equals the call run
    alone."""
    torch = torch_cuda()
    M, N, K = 64, 48, 18944
    _, s, pw, _ = case(1, M, N, K, True)
    sd = to_dev(s)
    xs = [to_dev(activations(32, j, M, K)) for j in range(6)]
    want = []
    for Xd in xs:
        out = torch.empty((M, N), dtype=torch.float16, device="cuda")
        c_gemm(Xd, pw, sd, out, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want.append(to_host(out).copy())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    note("shared scratch two streams")
    for rep in range(3):
        for j, (Xd, out) in enumerate(zip(xs, outs)):
            c_gemm(Xd, pw, sd, out, streams[j % 2].cuda_stream)
        torch.cuda.synchronize()
        for j, (out, w) in enumerate(zip(outs, want)):
            assert np.array_equal(to_host(out).view(np.uint16), w.view(np.uint16)), (rep, j)
            out.fill_(float("nan"))
        torch.cuda.synchronize()


def test_capture_takes_the_unsplit_path():
    """Under stream capture the call does not use the shared scratch: a captured graph
    replays the unsplit path's bits (w4a16_gemm_path, automatic kernel choice) every
    time, with eager work between the replays."""
    torch = torch_cuda()
    M, N, K = 64, 528, 4096
    _, s, pw, X = case(0, M, N, K, False)
    Xd = to_dev(X)
    want = to_host(w4.w4a16_gemm_path(Xd, pw, None, w4.PATH_AUTO)).copy()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        c_gemm(Xd, pw, None, out, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("shared scratch under capture")
    with torch.cuda.graph(g):
        c_gemm(Xd, pw, None, out, torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint16), want.view(np.uint16)), rep


def test_bf16_and_int8_without_workspace_match_workspace_call():
    """bf16 activations (INT4 codes) and INT8 codes (fp16 activations): the DMA-staged
    tiled kernels take X * s from the shared scratch when the call has no workspace,
    with the same bits as the call with one; the outputs match the oracle."""
    torch = torch_cuda()
    items, refs = [], []
    for i, (M, N, K, awq, bf, bits) in enumerate([(64, 528, 4096, True, True, 4),
                                                  (100, 256, 4096, True, True, 4),
                                                  (64, 528, 4096, True, False, 8),
                                                  (100, 48, 18944, False, False, 8)]):
        W = weights(33, i, N, K)
        s = awq_scales(33, i, K) if awq else None
        sd = None if s is None else to_dev(s)
        pw = w4.w4a16_quantize_pack(to_dev(W), sd, mode=w4.QUANT_ASYM8 if bits == 8 else w4.QUANT_ASYM)
        Xd = to_dev(activations(33, i, M, K))
        dt = torch.bfloat16 if bf else torch.float16
        Xd = Xd.to(dt)
        items.append((Xd, pw, sd, torch.empty((M, N), dtype=dt, device="cuda")))
        refs.append((W, s, bits, Xd.float().cpu().numpy().astype(np.float64)))
    note("shared scratch: bf16 and INT8 grouped call")
    call = w4.GroupedCall(items)
    assert call.ws_bytes > 0
    call()
    want = [it[3].float().cpu().numpy().copy() for it in items]
    for it in items:
        it[3].fill_(float("nan"))
    w4.GroupedCall(items, workspace=False)()
    for it, w, (W, s, bits, X) in zip(items, want, refs):
        got = it[3].float().cpu().numpy()
        assert np.array_equal(got, w), (it[0].shape, bits)
        ref = oracle.quantize(W, s, bits=bits)
        tol = (REL_L2_BF16, MAX_REL_BF16) if it[0].dtype == torch.bfloat16 else ()
        assert_close(got, oracle.gemm(X, ref.q, ref.scales, ref.zeros, s), f"bits={bits}", *tol)
