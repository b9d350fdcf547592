"""Full-size grouped launches: the exact calls the benchmark times, checked against the oracle.

The benchmark runs a whole layer as one grouped call (``GroupedCall``: all seven
full-size matrices, with the workspace the library asks for) at each batch size:
the Llama-3-8B-shaped layer at M = 1 (decode) and M = 2, 5, 9 (speculative verify),
and the Qwen2-7B-shaped layer at M = 16, 64, 256 (batched decode); the same layer at
M = 24, 40 and 80 covers the tiled kernel's 32-, 48- and 96-row tiles.  A grouped launch
chooses its K split, its X * s staging (whole rows, K windows, or both in one launch)
and its split-K partials from the whole set of problems, so its summation order can
differ from a one-problem call of the same matrix; this file checks the grouped call
itself.  The oracle quantizes sampled 16-row blocks of every matrix on its own (rows
are quantized independently; the blocks are regenerated from the seeded generator)
and computes Y for sampled rows n of those blocks and sampled batch rows m.
"""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import assert_close, note, to_dev, to_host, torch_cuda
from workloads import activations, awq_scales, config_by_name, weight_rows, weights

pytestmark = pytest.mark.gpu

CASES = [("llama3_8b_decode", 1), ("llama3_8b_verify", 2), ("llama3_8b_verify", 5),
         ("llama3_8b_verify", 9), ("qwen2_7b_batched_decode", 16),
         ("qwen2_7b_batched_decode", 64), ("qwen2_7b_batched_decode", 256),
         ("qwen2_7b_batched_decode", 24), ("qwen2_7b_batched_decode", 40),
         ("qwen2_7b_batched_decode", 80)]

_PACKED = {}


def packed_layer(cfg):
    """The layer's seven matrices packed on the GPU (cached per weight key: the decode
    and verify configurations share the 8B layer's weights)."""
    if cfg.weight_key not in _PACKED:
        _PACKED.clear()
        torch = torch_cuda()
        torch.cuda.empty_cache()
        mats = []
        for mi, mat in enumerate(cfg.matrices):
            note(f"{cfg.name}: pack {mat.name} {mat.N}x{mat.K}")
            W = weights(cfg.weight_key, mi, mat.N, mat.K, threads=16)
            s = awq_scales(cfg.weight_key, mi, mat.K) if cfg.awq else None
            sd = None if s is None else to_dev(s)
            pw = w4.w4a16_quantize_pack(to_dev(W), sd)
            del W
            mats.append((mat, pw, s, sd))
        _PACKED[cfg.weight_key] = mats
    return _PACKED[cfg.weight_key]


def sample_blocks(N, rng, count=2):
    nb = N // 16
    picks = {0, nb - 1}
    while len(picks) < min(nb, count + 2):
        picks.add(int(rng.integers(0, nb)))
    return sorted(picks)


@pytest.mark.parametrize("name,M", CASES, ids=[f"{n}-M{m}" for n, m in CASES])
def test_grouped_layer_call(name, M):
    torch = torch_cuda()
    cfg = config_by_name(name)
    mats = packed_layer(cfg)
    items = []
    for mi, (mat, pw, s, sd) in enumerate(mats):
        X = to_dev(activations(cfg.weight_key, mi, M, mat.K, outliers=cfg.act_outliers))
        Y = torch.empty((M, mat.N), dtype=torch.float16, device="cuda")
        items.append((X, pw, sd, Y))
    call = w4.GroupedCall(items, stream=torch.cuda.current_stream().cuda_stream)
    note(f"{name} M={M}: one grouped call of {len(items)} problems, workspace "
         f"{call.ws_bytes} bytes, path {w4.w4a16_select_path(M, mats[0][0].N, mats[0][0].K)}")
    call()
    rng = np.random.default_rng([cfg.index, M])
    for mi, (mat, pw, s, sd) in enumerate(mats):
        Y = to_host(items[mi][3])
        assert np.isfinite(Y.astype(np.float32)).all(), f"{mat.name}: non-finite output"
        blocks = sample_blocks(mat.N, rng)
        rows = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in blocks])
        Wr = np.concatenate([weight_rows(cfg.weight_key, mi, mat.N, mat.K, 16 * b, 16 * b + 16)
                             for b in blocks])
        ref = oracle.quantize(Wr, s)
        X = activations(cfg.weight_key, mi, M, mat.K, outliers=cfg.act_outliers)
        ms = np.arange(M) if M <= 24 else np.unique(
            np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
        Yref = oracle.gemm(X[ms], ref.q, ref.scales, ref.zeros, s)
        assert_close(Y[np.ix_(ms, rows)], Yref, f"{name}/{mat.name} M={M} (grouped)")
    # the same call again gives the same bits (fixed-order reductions)
    first = [to_host(it[3]).copy() for it in items]
    call()
    for mi, it in enumerate(items):
        assert np.array_equal(to_host(it[3]).view(np.uint16), first[mi].view(np.uint16))
