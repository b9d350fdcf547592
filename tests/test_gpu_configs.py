"""Full-size workloads: every matrix of the five problem configurations, packed on the
GPU and multiplied at each configuration's batch sizes, one matrix per call, with the
kernel the library's dispatch picks.  (The benchmark runs each decode, verify and
batched layer as one grouped call of all seven matrices; those exact calls are checked
in test_gpu_grouped_layers.py.  The 70B prefill matrices are timed one call each, as
here.)

The oracle cannot run a whole 70B-shaped layer in seconds, so it checks samples
it computes on its own: whole 16-row blocks of the packed buffers (first, last
and random ones; rows are quantized independently, so the oracle quantizes just
those rows, regenerated from the seeded generator), and the outputs Y[m][n] for
sampled rows n of those blocks and sampled batch rows m.
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, h16_bits, note, to_dev, to_host, torch_cuda
from workloads import CONFIGS, activations, awq_scales, weight_rows, weights

pytestmark = pytest.mark.gpu

CASES = [(cfg.index, mi) for cfg in CONFIGS for mi in range(len(cfg.matrices))]


def sample_blocks(N, rng, count=3):
    nb = N // 16
    picks = {0, nb - 1}
    while len(picks) < min(nb, count + 2):
        picks.add(int(rng.integers(0, nb)))
    return sorted(picks)


def sample_rows(M, rng, count=24):
    if M <= count:
        return np.arange(M)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, count, replace=False)]))


@pytest.mark.parametrize("ci,mi", CASES, ids=[f"cfg{c + 1}-{CONFIGS[c].matrices[m].name}"
                                             for c, m in CASES])
def test_config_matrix(ci, mi):
    torch = torch_cuda()
    cfg = CONFIGS[ci]
    mat = cfg.matrices[mi]
    N, K = mat.N, mat.K
    rng = np.random.default_rng([ci, mi])
    note(f"config {cfg.name} matrix {mat.name} {N}x{K}: generate + pack")
    W = weights(cfg.weight_key, mi, N, K, threads=16)
    s = awq_scales(cfg.weight_key, mi, K) if cfg.awq else None
    Wd = to_dev(W)
    sd = None if s is None else to_dev(s)
    del W
    pw = w4.w4a16_quantize_pack(Wd, sd)
    del Wd
    wq, sc, zr = to_host(pw.wq), to_host(pw.scales), to_host(pw.zeros)

    G, NB = K // 128, N // 16
    blocks = sample_blocks(N, rng)
    rows = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in blocks])
    Wr = np.concatenate([weight_rows(cfg.weight_key, mi, N, K, 16 * b, 16 * b + 16)
                         for b in blocks])
    ref = oracle.quantize(Wr, s)
    # A 16-row block packed on its own is its G tiles back to back; in the whole
    # buffer (group-major) tile g of row block b sits at (g * NB + b) * 1024.
    for j, b in enumerate(blocks):
        qb = ref.q[16 * j:16 * j + 16]
        got = np.concatenate([wq[(g * NB + b) * 1024:(g * NB + b + 1) * 1024] for g in range(G)])
        assert np.array_equal(got, oracle.pack_codes(qb)), f"packed codes differ in row block {b}"
    assert np.array_equal(h16_bits(oracle.unpack_meta(sc, N, K)[rows]), h16_bits(ref.scales))
    assert np.array_equal(h16_bits(oracle.unpack_meta(zr, N, K)[rows]), h16_bits(ref.zeros))
    Gq = oracle.meta_groups(K) // 4
    for j, b in enumerate(blocks):   # whole metadata runs of the sampled row blocks, padding included
        got = np.concatenate([sc[(u * NB + b) * 64:(u * NB + b + 1) * 64] for u in range(Gq)])
        refb = oracle.pack_meta(ref.scales[16 * j:16 * j + 16])
        assert np.array_equal(h16_bits(got), h16_bits(refb))

    for M in cfg.Ms:
        note(f"config {cfg.name} matrix {mat.name} M={M}: gemm "
             f"(path {w4.w4a16_select_path(M, N, K)})")
        X = activations(cfg.weight_key, mi, M, K, outliers=cfg.act_outliers)
        Y = to_host(w4.w4a16_gemm(to_dev(X), pw, sd))
        assert Y.shape == (M, N)
        ms = sample_rows(M, rng)
        ns = rng.choice(len(rows), size=min(len(rows), 48), replace=False)
        Yref = oracle.gemm(X[ms], ref.q[ns], ref.scales[ns], ref.zeros[ns], s)
        assert_close(Y[np.ix_(ms, rows[ns])], Yref, f"{cfg.name}/{mat.name} M={M}")
        # every output is finite, not only the sampled ones
        assert np.isfinite(Y.astype(np.float32)).all()
        del Y
    del pw
    torch.cuda.empty_cache()
