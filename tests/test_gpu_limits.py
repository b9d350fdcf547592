"""The largest shape the boundary accepts: packed codes just under 2 GiB - 1 MiB.

W = 32736 x 131072 (N*K/2 = 2,145,386,496 bytes, G = 1024 groups, 2046 row
blocks): every 32-bit byte offset the kernels form (group-major tile and
metadata offsets, row offsets of X) is near its largest here.  The rows the
oracle checks (first, last and sampled row blocks) come from the seeded
generator and are written into a device matrix whose other rows torch fills
with random values; every tile packs on its own and every output row depends
only on its own weight row, so the checks are exact at this size.  Packing is
compared byte for byte on the sampled row blocks (codes and metadata runs),
and the GEMM on sampled outputs at M = 1 (streaming, K windows), M = 16 and
M = 33 (tiled, split-K).
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, h16_bits, note, to_dev, to_host, torch_cuda
from workloads import activations, awq_scales, weight_rows

pytestmark = pytest.mark.gpu

N, K = 32736, 131072
KEY, MAT = 21, 0


def test_largest_accepted_shape():
    torch = torch_cuda()
    assert N * K // 2 < 2 * 1024 ** 3 - 1024 ** 2
    G, NB = K // 128, N // 16
    blocks = [0, 1, 977, NB - 1]
    note(f"limits: fill W {N}x{K} on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    W = torch.empty((N, K), dtype=torch.float16, device="cuda")
    W.normal_(0.0, 0.02, generator=gen)
    Wr = np.concatenate([weight_rows(KEY, MAT, N, K, 16 * b, 16 * b + 16) for b in blocks])
    for j, b in enumerate(blocks):
        W[16 * b:16 * b + 16].copy_(torch.from_numpy(Wr[16 * j:16 * j + 16]))
    s = awq_scales(KEY, MAT, K)
    sd = to_dev(s)
    note("limits: pack")
    pw = w4.w4a16_quantize_pack(W, sd)
    del W
    torch.cuda.synchronize()
    ref = oracle.quantize(Wr, s)
    wq, sc, zr = pw.wq, pw.scales, pw.zeros
    for j, b in enumerate(blocks):
        idx = torch.tensor([(g * NB + b) for g in range(G)], device="cuda")
        got = wq.view(-1, 1024)[idx].reshape(-1)
        assert np.array_equal(to_host(got), oracle.pack_codes(ref.q[16 * j:16 * j + 16])), \
            f"codes of row block {b}"
        qidx = torch.tensor([(u * NB + b) for u in range(G // 4)], device="cuda")
        for buf, vals in ((sc, ref.scales), (zr, ref.zeros)):
            got = to_host(buf.view(-1, 64)[qidx].reshape(-1))
            assert np.array_equal(h16_bits(got), h16_bits(oracle.pack_meta(vals[16 * j:16 * j + 16]))), \
                f"metadata of row block {b}"
    rows = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in blocks])
    rng = np.random.default_rng(21)
    for M in (1, 16, 33):
        X = activations(KEY, MAT, M, K)
        note(f"limits: gemm M={M} (path {w4.w4a16_select_path(M, N, K)})")
        Y = to_host(w4.w4a16_gemm(to_dev(X), pw, sd))
        ns = rng.choice(len(rows), size=24, replace=False)
        Yref = oracle.gemm(X, ref.q[ns], ref.scales[ns], ref.zeros[ns], s)
        assert_close(Y[:, rows[ns]], Yref, f"limits M={M}")
        assert np.isfinite(Y.astype(np.float32)).all()
    del pw
    torch.cuda.empty_cache()
