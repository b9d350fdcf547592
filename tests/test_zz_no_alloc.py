"""w4a16_gemm_grouped_static (the entry point for callers that cannot allocate) against
w4a16_gemm_grouped_ws with a caller workspace of the queried size: the same kernels with
the same splits, so the outputs must be the same bits.  Two calls in a row through the C
ABI, the second with a smaller input, so the static scratch is reused with a smaller
need; then the oracle on sampled outputs, as for any grouped call."""
import ctypes

import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, note, to_dev, to_host, torch_cuda
from workloads import activations, config_by_name, weight_rows, weights

pytestmark = pytest.mark.gpu


def _layer(cfg, rows_cap=None):
    out = []
    for mi, mat in enumerate(cfg.matrices):
        N = mat.N if rows_cap is None else min(mat.N, rows_cap)
        W = weights(cfg.weight_key, mi, mat.N, mat.K, threads=16)[:N]
        out.append((mi, N, mat.K, w4.w4a16_quantize_pack(to_dev(W), None)))
    return out


def _call_both(cfg, packed, M):
    """One call each of the static and the workspace entry point on the same problems,
    straight through the C ABI; returns (static outputs, workspace outputs)."""
    torch = torch_cuda()
    L = w4.lib()
    Xs = [to_dev(activations(cfg.weight_key, mi, M, K)) for mi, N, K, _ in packed]
    Ya = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
          for _, N, _, _ in packed]
    Yb = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
          for _, N, _, _ in packed]

    def problems(Ys):
        arr = (w4.Problem * len(packed))()
        for i, ((mi, N, K, pw), X, Y) in enumerate(zip(packed, Xs, Ys)):
            arr[i] = w4.Problem(X.data_ptr(), pw.wq.data_ptr(), pw.scales.data_ptr(),
                                pw.zeros.data_ptr(), None, Y.data_ptr(), M, N, K,
                                None, None, None, 0, 4)
        return arr
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pa = problems(Ya)
    need = ctypes.c_size_t()
    assert L.w4a16_gemm_workspace_size(pa, len(packed), ctypes.byref(need)) == 0
    assert need.value <= w4.STATIC_SCRATCH_BYTES
    note(f"{cfg.name} M={M}: static call, workspace need {need.value} bytes")
    assert L.w4a16_gemm_grouped_static(pa, len(packed), st) == 0
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
    pb = problems(Yb)
    note(f"{cfg.name} M={M}: workspace call")
    assert L.w4a16_gemm_grouped_ws(pb, len(packed), ctypes.c_void_p(ws.data_ptr()), need.value,
                                   st) == 0
    torch.cuda.synchronize()
    return [to_host(y) for y in Ya], [to_host(y) for y in Yb], need.value


def test_static_matches_workspace_two_calls():
    cfg = config_by_name("qwen2_7b_batched_decode")
    packed = _layer(cfg)
    needs = []
    for M in (64, 32):           # the second call is smaller and needs less scratch
        Ya, Yb, need = _call_both(cfg, packed, M)
        needs.append(need)
        for (mi, N, K, pw), a, b in zip(packed, Ya, Yb):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (M, mi)
        # and the oracle on sampled rows of one matrix per call
        mi, N, K, _ = packed[6]
        rows = np.arange(16 * 7, 16 * 9)
        ref = oracle.quantize(weight_rows(cfg.weight_key, mi, N, K, 16 * 7, 16 * 9), None)
        X = activations(cfg.weight_key, mi, M, K)
        assert_close(Ya[6][:, rows], oracle.gemm(X, ref.q, ref.scales, ref.zeros, None),
                     f"static M={M}")
    assert needs[0] > needs[1] > 0


def test_static_without_split_needs_no_scratch():
    """A call that splits nothing (decode shapes) runs without touching the scratch."""
    cfg = config_by_name("llama3_8b_decode")
    packed = _layer(cfg, rows_cap=1024)
    Ya, Yb, need = _call_both(cfg, packed, 1)
    assert need == 0
    for a, b in zip(Ya, Yb):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
