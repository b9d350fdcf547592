"""GPU packer vs the fp64 oracle: packed codes, scales and zero points must be bit-exact."""
import numpy as np
import pytest

import oracle
import weight_only_int4_group_amd as w4
from tests.gpu_helpers import h16_bits, note, to_dev, to_host, torch_cuda
from workloads import awq_scales, weights

pytestmark = pytest.mark.gpu


def gpu_pack(W, s, mode=w4.QUANT_ASYM):
    torch_cuda()
    pw = w4.w4a16_quantize_pack(to_dev(W), None if s is None else to_dev(s), mode=mode)
    return to_host(pw.wq), to_host(pw.scales), to_host(pw.zeros)


GRANULARITY = {w4.QUANT_ASYM: "group", w4.QUANT_ASYM_CHANNEL: "channel",
               w4.QUANT_ASYM_TENSOR: "tensor"}


def oracle_quant(W, s, mode):
    if mode == w4.QUANT_SYM:
        return oracle.quantize_symmetric(W, s)
    return oracle.quantize(W, s, GRANULARITY[mode])


def check_exact(W, s, tag, mode=w4.QUANT_ASYM):
    note(f"pack {tag} N={W.shape[0]} K={W.shape[1]} awq={s is not None} mode={mode}")
    wq, sc, z = gpu_pack(W, s, mode)
    ref = oracle_quant(W, s, mode)
    assert np.array_equal(h16_bits(sc), h16_bits(oracle.pack_meta(ref.scales))), tag
    assert np.array_equal(h16_bits(z), h16_bits(oracle.pack_meta(ref.zeros))), tag
    assert np.array_equal(wq, oracle.pack_codes(ref.q)), tag


MODES = [w4.QUANT_ASYM, w4.QUANT_SYM, w4.QUANT_ASYM_CHANNEL, w4.QUANT_ASYM_TENSOR]


@pytest.mark.parametrize("mode", MODES)
def test_pack_gemv_1024(mode):
    check_exact(weights(0, 0, 1024, 1024), None, "1024x1024", mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 640), (1024, 4096)])
def test_pack_awq_shapes(N, K, mode):
    check_exact(weights(1, 9, N, K), awq_scales(1, 9, K), f"awq {N}x{K}", mode)


@pytest.mark.parametrize("mode", [w4.QUANT_ASYM_CHANNEL, w4.QUANT_ASYM_TENSOR])
def test_pack_coarse_granularity_across_range_passes(mode):
    """More rows than one pass of the packer's row-range scratch (32768 rows): the
    channel and tensor ranges are formed pass by pass, and the row holding the tensor's
    extreme value sits in the second pass."""
    rng = np.random.default_rng(12)
    N, K = 32768 + 4096 + 48, 256
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[N - 5, 200] = np.float16(0.75)                    # the tensor's largest weight
    W[33000, 17] = np.float16(-0.5)                     # and its least
    s = awq_scales(1, 9, K)
    check_exact(W, s, "two range passes", mode)
    # the same packer call again on a different (smaller) matrix: nothing carries over
    check_exact(W[:4096 + 32], s, "after two range passes", mode)


@pytest.mark.parametrize("mode", MODES)
def test_pack_edge_groups(mode):
    rng = np.random.default_rng(11)
    N, K = 64, 1024
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    W[0:16, 0:128] = 0                                  # all-zero group
    W[16, 128:256] = np.float16(-0.0)                   # signed zeros only
    W[17, 256:384] = 3.0                                # constant positive group
    W[18, 256:384] = -3.0                               # constant negative group
    W[19, 384:512] = np.float16(6e-8)                   # subnormal weights -> tiny scale
    W[20, 512:640] = rng.standard_normal(128).astype(np.float16) * np.float16(1e-5)
    W[21, 640:768] = np.float16(60000.0)                # near the top of fp16
    W[22, 768:896] *= 500                               # outlier-heavy group
    W[23, 896:1024] = np.linspace(-1, 1, 128).astype(np.float16)  # ties land on .5
    check_exact(W, None, "edge groups", mode)
    s = np.exp(rng.uniform(-1, 1, K)).astype(np.float16)   # keeps 60000 / s in range
    check_exact(W, s, "edge groups + awq", mode)


def test_pack_symmetric_on_grid_exact():
    # weights on the signed -7..7 grid (with +-7 in every group) come back exactly
    rng = np.random.default_rng(6)
    N, K, G = 32, 256, 2
    c = rng.integers(-7, 8, size=(N, G, 128))
    c[:, :, 0], c[:, :, 1] = 7, -7
    scale = np.ldexp(rng.integers(64, 128, size=(N, G)).astype(np.float64),
                     rng.integers(-16, -8, size=(N, G)))
    W = (c * scale[:, :, None]).reshape(N, K).astype(np.float16)
    wq, sc, zz = gpu_pack(W, None, w4.QUANT_SYM)
    assert np.array_equal(oracle.unpack_meta(sc, N, K).astype(np.float64), scale)
    assert np.all(oracle.unpack_meta(zz, N, K) == 8)
    assert np.array_equal(oracle.unpack_codes(wq, N, K).astype(np.int64) - 8, c.reshape(N, K))


def test_pack_on_grid_exact():
    # weights on the quantization grid are reconstructed exactly (pin P2's input family)
    rng = np.random.default_rng(5)
    N, K, G = 32, 256, 2
    q = rng.integers(0, 16, size=(N, G, 128))
    q[:, :, 0], q[:, :, 1] = 0, 15
    z = rng.integers(0, 16, size=(N, G))
    scale = np.ldexp(rng.integers(64, 128, size=(N, G)).astype(np.float64),
                     rng.integers(-16, -8, size=(N, G)))
    W = ((q - z[:, :, None]) * scale[:, :, None]).reshape(N, K).astype(np.float16)
    wq, sc, zz = gpu_pack(W, None)
    assert np.array_equal(oracle.unpack_meta(sc, N, K).astype(np.float64), scale)
    assert np.array_equal(oracle.unpack_meta(zz, N, K).astype(np.int64), z)
    assert np.array_equal(oracle.unpack_codes(wq, N, K), q.reshape(N, K).astype(np.uint8))


@pytest.mark.parametrize("bad", ["nan_w", "inf_w", "zero_s", "neg_s", "inf_s"])
def test_pack_rejects_nonfinite(bad):
    N, K = 32, 256
    W = weights(0, 3, N, K)
    s = np.ones(K, np.float16)
    if bad == "nan_w":
        W[5, 7] = np.nan
    elif bad == "inf_w":
        W[31, 255] = np.inf
    elif bad == "zero_s":
        s[100] = 0
    elif bad == "neg_s":
        s[3] = -1
    else:
        s[200] = np.inf
    note(f"pack rejects {bad}")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_quantize_pack(to_dev(W), to_dev(s))
    assert e.value.status == -4


def test_pack_rejects_scale_overflow():
    N, K = 16, 128
    W = np.zeros((N, K), np.float16)
    W[3, 0], W[3, 1] = np.float16(60000), np.float16(-60000)
    s = np.full(K, np.float16(0.05))          # W/s spans 2.4e6: range/15 > 65504
    note("pack rejects scale overflow")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_quantize_pack(to_dev(W), to_dev(s))
    assert e.value.status == -5
