"""The C-ABI library: it loads without a GPU, exports what include/w4a16.h declares,
and validates every argument on the host before any HIP call.

Only calls that fail validation are made here (no compute happens without a GPU).
"""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

import weight_only_int4_group_amd as w4
from oracle.accounting import packed_sizes as oracle_sizes

HEADER = os.path.join(ROOT, "include", "w4a16.h")
V = ctypes.c_void_p
A16 = V(1 << 20)        # a 16-byte aligned stand-in address (never dereferenced)
ODD = V((1 << 20) + 2)  # a misaligned one


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(w4a16_\w+)\s*\(", text, re.M)))


def status_constants():
    text = open(HEADER).read()
    return {name: int(val) for name, val in re.findall(r"(W4A16_E?\w+)\s*=\s*(-?\d+)", text)}


def test_library_exports_every_declared_function():
    L = w4.lib()
    names = declared_functions()
    assert len(names) >= 6
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(w4.EXPORTED_SYMBOLS)
    assert w4.w4a16_version() >= 100


def test_status_codes_match_header():
    consts = status_constants()
    for code, name in w4.STATUS.items():
        assert consts[name] == code
    for code in w4.STATUS:
        assert w4.w4a16_strerror(code) and w4.w4a16_strerror(code) != "unknown status"
    assert w4.w4a16_strerror(12345) == "unknown status"


@pytest.mark.parametrize("N,K", [(1024, 1024), (16, 128), (14336, 4096), (4096, 14336),
                                 (18944, 3584), (28672, 8192)])
def test_packed_sizes(N, K):
    wq, sc, z = w4.w4a16_packed_sizes(N, K)
    assert (wq, sc, z) == oracle_sizes(N, K)
    assert wq == N * K // 2 and sc == z == 2 * N * (-(-(K // 128) // 4) * 4)


@pytest.mark.parametrize("N,K", [(0, 128), (16, 0), (8, 128), (16, 64), (17, 128), (16, 200),
                                 (-16, 128), (1 << 25, 128), (65536, 65536)])
def test_packed_sizes_rejects(N, K):
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_packed_sizes(N, K)
    assert e.value.status == -1


def test_packed_sizes_null_outputs():
    assert w4.lib().w4a16_packed_sizes(16, 128, None, None, None) == -1
    assert w4.lib().w4a16_packed_sizes_mode(16, 128, 0, None, None, None) == -1


@pytest.mark.parametrize("N,K", [(16, 128), (14336, 4096), (4096, 14336), (18944, 3584)])
def test_packed_sizes_per_mode(N, K):
    """INT4 modes share one size; INT8 codes take a byte per weight, same metadata."""
    wq4, sc, z = oracle_sizes(N, K)
    for mode in (w4.QUANT_ASYM, w4.QUANT_SYM, w4.QUANT_ASYM_CHANNEL, w4.QUANT_ASYM_TENSOR):
        assert w4.w4a16_packed_sizes(N, K, mode) == (wq4, sc, z)
    assert w4.w4a16_packed_sizes(N, K, w4.QUANT_ASYM8) == (N * K, sc, z)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_packed_sizes(N, K, 5)
    assert e.value.status == -3


def test_packed_sizes_int8_limit():
    # 32768 x 65536 INT4 codes fit the limit (1 GiB); as INT8 bytes (2 GiB) they do not
    assert w4.w4a16_packed_sizes(32768, 65536)[0] == 1 << 30
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_packed_sizes(32768, 65536, w4.QUANT_ASYM8)
    assert e.value.status == -1


def gemm_rc(X=A16, Wq=A16, sc=A16, z=A16, s=None, Y=A16, M=1, N=16, K=128, path=0):
    return w4.lib().w4a16_gemm_path(X, Wq, sc, z, s, Y, M, N, K, path, None)


def pack_rc(W=A16, s=None, N=16, K=128, Wq=A16, sc=A16, z=A16):
    return w4.lib().w4a16_quantize_pack(W, s, N, K, Wq, sc, z, None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=100), -1), (dict(K=0), -1), (dict(N=8), -1), (dict(N=0), -1), (dict(M=-1), -1),
    (dict(M=1 << 23), -1), (dict(X=None), -1), (dict(Wq=None), -1), (dict(sc=None), -1),
    (dict(z=None), -1), (dict(Y=None), -1), (dict(X=ODD), -2), (dict(Y=ODD), -2),
    (dict(s=ODD), -2), (dict(Wq=ODD), -2), (dict(path=7), -3), (dict(path=-1), -3),
])
def test_gemm_validation(kw, code):
    assert gemm_rc(**kw) == code


def test_gemm_empty_batch_is_a_noop():
    # M = 0: nothing to read or write, the pointers may be NULL, no HIP call is made
    assert gemm_rc(X=None, Y=None, M=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), -1), (dict(Wq=None), -1), (dict(sc=None), -1), (dict(z=None), -1),
    (dict(N=24), -1), (dict(K=192), -1), (dict(N=0), -1), (dict(W=ODD), -2), (dict(s=ODD), -2),
    (dict(z=ODD), -2),
])
def test_pack_validation(kw, code):
    assert pack_rc(**kw) == code


def test_select_path():
    sel = w4.w4a16_select_path
    for M in (1, 2, 5, 9, 16):
        assert sel(M, 4096, 4096) == w4.PATH_SKINNY
    for M in (64, 256, 4096):
        assert sel(M, 4096, 4096) == w4.PATH_TILED


def test_grouped_validation():
    L = w4.lib()
    assert L.w4a16_gemm_grouped(None, 0, None) == 0          # nothing to do
    assert L.w4a16_gemm_grouped(None, 2, None) == -1         # NULL array
    assert L.w4a16_gemm_grouped(None, -1, None) == -1
    good = w4.Problem(A16, A16, A16, A16, None, A16, 0, 16, 128)   # M = 0: valid no-op
    bad_k = w4.Problem(A16, A16, A16, A16, None, A16, 1, 16, 100)
    bad_al = w4.Problem(ODD, A16, A16, A16, None, A16, 1, 16, 128)
    arr = (w4.Problem * 3)(good, good, good)
    assert L.w4a16_gemm_grouped(arr, 3, None) == 0           # all empty: no HIP call
    arr = (w4.Problem * 3)(good, bad_k, good)
    assert L.w4a16_gemm_grouped(arr, 3, None) == -1
    arr = (w4.Problem * 2)(bad_al, good)
    assert L.w4a16_gemm_grouped(arr, 2, None) == -2


def ws_size(*problems):
    L = w4.lib()
    arr = (w4.Problem * len(problems))(*problems)
    nb = ctypes.c_size_t(12345)
    rc = L.w4a16_gemm_workspace_size(arr, len(problems), ctypes.byref(nb))
    return rc, nb.value


def test_workspace_size():
    """Host-only size query: zero where K is not split (streaming-path problems, grids
    that fill the GPU), S fp32 [M][N] slabs where it is."""
    P = w4.Problem
    assert ws_size(P(A16, A16, A16, A16, None, A16, 9, 4096, 14336)) == (0, 0)
    assert ws_size(P(A16, A16, A16, A16, None, A16, 4096, 8192, 8192)) == (0, 0)
    # 64 x 272 output: three 64 x 128 blocks (the DMA-staged kernel's M <= 64 shape)
    # x 32 groups, far fewer than the GPU's block slots, so K is cut into ranges of
    # the minimum 8 groups: 4 splits
    rc, nb = ws_size(P(A16, A16, A16, A16, None, A16, 64, 272, 4096))
    assert rc == 0 and nb == 4 * 64 * 272 * 4
    # a problem with M = 0 and a streaming one add nothing
    rc2, nb2 = ws_size(P(A16, A16, A16, A16, None, A16, 64, 272, 4096),
                       P(A16, A16, A16, A16, None, A16, 0, 16, 128),
                       P(A16, A16, A16, A16, None, A16, 1, 4096, 4096))
    assert (rc2, nb2) == (0, nb)
    # bf16 streaming problems: room for bf16(X * s) [M][K] and fp32 group sums [M][G]
    pb = P(A16, A16, A16, A16, None, A16, 9, 4096, 14336)
    pb.dtype = w4.DTYPE_BF16
    a256 = lambda n: -(-n // 256) * 256
    assert ws_size(pb) == (0, a256(9 * 14336 * 2) + a256(9 * 112 * 4))
    # launches share the workspace in stream order: the larger need counts
    rc3, nb3 = ws_size(pb, P(A16, A16, A16, A16, None, A16, 64, 272, 4096))
    assert rc3 == 0 and nb3 == max(nb, a256(9 * 14336 * 2) + a256(9 * 112 * 4))
    L = w4.lib()
    arr = (P * 1)(P(A16, A16, A16, A16, None, A16, 64, 272, 4096))
    assert L.w4a16_gemm_workspace_size(arr, 1, None) == -1
    assert ws_size(P(A16, A16, A16, A16, None, A16, 64, 272, 100))[0] == -1


def test_split_counts_whole_rounds():
    """K splits of a grouped tiled call are chosen by whole rounds of resident
    workgroups (host-only, through the workspace size).  Qwen2-7B-shaped layer, fp16
    activations and INT4 codes, so the launches take the DMA-staged tiled kernel:
    at M = 64 its 64 x 128 blocks (388 of them) of two K slices, two workgroups per
    CU (512 slots): 30-group ranges split only down (5 ways), 500 workgroups in one
    round.  At M = 256 its 128 x 256 blocks with two per CU (512 slots): 30-group
    ranges split only down (5 ways), 500 workgroups."""
    P = w4.Problem
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584),
              (18944, 3584), (3584, 18944)]

    def layer(M):
        return [P(A16, A16, A16, A16, None, A16, M, N, K) for N, K in shapes]

    splits64 = [1, 1, 1, 1, 1, 1, 5]
    rc, nb = ws_size(*layer(64))
    assert rc == 0 and nb == 5 * 64 * 3584 * 4
    assert sum(s * -(-N // 128) for s, (N, _) in zip(splits64, shapes)) == 500
    splits256 = [1, 1, 1, 1, 1, 1, 5]
    rc, nb = ws_size(*layer(256))
    assert rc == 0 and nb == 5 * 256 * 3584 * 4
    assert sum(s * 2 * -(-N // 256) for s, (N, _) in zip(splits256, shapes)) == 500
    # prefill-sized calls fill the GPU without splitting
    assert ws_size(P(A16, A16, A16, A16, None, A16, 4096, 28672, 8192)) == (0, 0)
    # with an AWQ s the DMA kernel's workspace also holds the prescaled X * s
    a256 = lambda n: -(-n // 256) * 256
    assert ws_size(P(A16, A16, A16, A16, A16, A16, 4096, 28672, 8192)) == (0, a256(4096 * 8192 * 2))


def test_grouped_ws_validation():
    L = w4.lib()
    good = w4.Problem(A16, A16, A16, A16, None, A16, 0, 16, 128)
    arr = (w4.Problem * 1)(good)
    assert L.w4a16_gemm_grouped_ws(arr, 1, None, 0, None) == 0
    assert L.w4a16_gemm_grouped_ws(arr, 1, ODD, 1 << 20, None) == -2   # misaligned workspace
    assert L.w4a16_gemm_grouped_ws(None, 1, None, 0, None) == -1


def test_grouped_static_rejects_calls_beyond_its_scratch():
    """w4a16_gemm_grouped_static checks the workspace a call needs against its static
    scratch on the host, before any HIP call: the 70B prefill layer as one grouped call
    needs far more than 64 MiB (k and v split, with fp32 partials of 4096 x 1024)."""
    L = w4.lib()
    P = w4.Problem
    shapes = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192),
              (28672, 8192), (8192, 28672)]
    arr = (P * 7)(*[P(A16, A16, A16, A16, A16, A16, 4096, N, K) for N, K in shapes])
    rc, need = ws_size(*arr)
    assert rc == 0 and need > w4.STATIC_SCRATCH_BYTES
    assert L.w4a16_gemm_grouped_static(arr, 7, None) == -7
    assert w4.w4a16_strerror(-7) != "unknown status"
    # validation comes first, as for the other grouped entry points
    assert L.w4a16_gemm_grouped_static(None, 2, None) == -1
    bad = (P * 1)(P(ODD, A16, A16, A16, None, A16, 1, 16, 128))
    assert L.w4a16_gemm_grouped_static(bad, 1, None) == -2
    empty = (P * 1)(P(A16, A16, A16, A16, None, A16, 0, 16, 128))
    assert L.w4a16_gemm_grouped_static(empty, 1, None) == 0   # M = 0: nothing to do


def test_quantize_mode_validation():
    L = w4.lib()
    # unknown mode: rejected before anything else, without a GPU call
    assert L.w4a16_quantize_pack_mode(A16, None, 16, 128, 5, A16, A16, A16, None) == -3
    assert L.w4a16_quantize_pack_mode(A16, None, 16, 128, -1, A16, A16, A16, None) == -3
    # known modes validate shapes and alignment like w4a16_quantize_pack
    for mode in (w4.QUANT_ASYM, w4.QUANT_SYM, w4.QUANT_ASYM_CHANNEL, w4.QUANT_ASYM_TENSOR,
                 w4.QUANT_ASYM8):
        assert L.w4a16_quantize_pack_mode(A16, None, 16, 100, mode, A16, A16, A16, None) == -1
        assert L.w4a16_quantize_pack_mode(ODD, None, 16, 128, mode, A16, A16, A16, None) == -2


def test_spec_verify_workspace_size():
    # per sequence: two 8-byte sums per 4096-id chunk and the first rejection (4 bytes),
    # rounded up to 256 bytes
    assert w4.w4a16_spec_verify_workspace_size(64, 4, 128256) == -(-(64 * 32 * 16 + 64 * 4) // 256) * 256
    assert w4.w4a16_spec_verify_workspace_size(1, 0, 1) == 256
    assert w4.w4a16_spec_verify_workspace_size(0, 4, 32000) == 0
    for B, K, Vv in ((-1, 4, 10), (1, -1, 10), (1, 4, 0), (1, 1025, 10), (1 << 20, 1024, 1 << 20),
                     (1 << 22, 0, 1 << 14)):
        with pytest.raises(w4.W4A16Error):
            w4.w4a16_spec_verify_workspace_size(B, K, Vv)
    L = w4.lib()
    assert L.w4a16_spec_verify_workspace_size(1, 1, 1, None) == -1


def test_spec_verify_validation():
    L = w4.lib()
    A4 = V((1 << 20) + 4)   # 4-byte aligned
    ODD1 = V((1 << 20) + 1)
    WS = V(1 << 24)         # 256-byte aligned
    big = 1 << 20

    def call(pt=A4, pd=A4, dr=A4, ua=A4, us=A4, B=2, K=4, Vv=32000, ws=WS, wsb=big,
             na=A4, tk=A4):
        return L.w4a16_spec_verify(pt, pd, dr, ua, us, B, K, Vv, ws, wsb, na, tk, None)

    # shapes: B, K >= 0, V >= 1, K <= 1024, B and V <= 2^24, B (K+1) V <= 2^40,
    # B * ceil(V / 4096) < 2^24
    assert call(B=-1) == -1
    assert call(K=-1) == -1
    assert call(Vv=0) == -1
    assert call(K=1025) == -1
    assert call(Vv=(1 << 24) + 1) == -1
    assert call(B=(1 << 24) + 1) == -1
    assert call(B=1 << 20, K=1024, Vv=1 << 20) == -1
    assert call(B=1 << 22, K=0, Vv=1 << 14) == -1
    # an empty batch is a no-op, whatever the pointers
    assert call(B=0, pt=None, us=None, na=None, tk=None, ws=None, wsb=0) == 0
    # required pointers
    for name in ("pt", "us", "na", "tk", "ws", "pd", "dr", "ua"):
        assert call(**{name: None}) == -1, name
    # a workspace smaller than w4a16_spec_verify_workspace_size
    need = w4.w4a16_spec_verify_workspace_size(2, 4, 32000)
    assert call(wsb=need - 1) == -1
    # 4-byte alignment of every buffer, 256 of the workspace
    for name in ("pt", "pd", "dr", "ua", "us", "na", "tk"):
        assert call(**{name: ODD1}) == -2, name
    assert call(ws=V((1 << 24) + 128)) == -2
    # with K = 0 the draft buffers are not read and may be NULL (or misaligned)
    assert call(K=0, pd=None, dr=None, ua=None, pt=ODD1) == -2


def test_outlier_pack_validation():
    L = w4.lib()
    A4 = V((1 << 20) + 4)
    WS = V(1 << 24)
    need = w4.w4a16_outlier_workspace_size(32, 256)
    assert need >= 32 * 256 // 8

    def call(W=A16, s=None, N=32, K=256, mode=0, count=8, wq=A16, sc=A16, z=A16, rp=A4, col=A4,
             val=A4, ws=WS, wsb=need):
        return L.w4a16_quantize_pack_outliers(W, s, N, K, mode, count, wq, sc, z, rp, col, val,
                                              ws, wsb, None)

    assert call(mode=5) == -3
    assert call(N=8) == -1 and call(K=100) == -1          # shapes as the plain packer
    assert call(count=-1) == -1 and call(count=32 * 256 + 1) == -1
    assert call(wsb=need - 1) == -1
    for name in ("W", "wq", "sc", "z", "rp", "ws"):
        assert call(**{name: None}) == -1, name
    assert call(col=None) == -1 and call(val=None) == -1
    assert call(W=ODD) == -2 and call(rp=V((1 << 20) + 2)) == -2
    assert call(col=V((1 << 20) + 2)) == -2 and call(val=V((1 << 20) + 1)) == -2
    assert call(ws=V((1 << 24) + 128)) == -2
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_outlier_workspace_size(30, 256)
    assert w4.page_outlier_count(4096, 4096) == 16777


def test_grouped_outlier_fields_validation():
    L = w4.lib()
    A4 = V((1 << 20) + 4)

    def prob(**kw):
        p = w4.Problem(A16, A16, A16, A16, None, A16, 1, 32, 256)
        for k, v in kw.items():
            setattr(p, k, v.value if isinstance(v, ctypes.c_void_p) else v)
        return p

    arr = (w4.Problem * 1)(prob(o_row_ptr=A4))            # only one of three set
    assert L.w4a16_gemm_grouped(arr, 1, None) == -1
    arr = (w4.Problem * 1)(prob(o_row_ptr=V((1 << 20) + 2), o_col=A4, o_val=A4))
    assert L.w4a16_gemm_grouped(arr, 1, None) == -2
    arr = (w4.Problem * 1)(prob(o_row_ptr=A4, o_col=A4, o_val=V((1 << 20) + 1)))
    assert L.w4a16_gemm_grouped(arr, 1, None) == -2


def test_grouped_dtype_validation():
    L = w4.lib()
    p = w4.Problem(A16, A16, A16, A16, None, A16, 1, 32, 256)
    p.dtype = 2
    arr = (w4.Problem * 1)(p)
    assert L.w4a16_gemm_grouped(arr, 1, None) == -3
    assert ctypes.sizeof(w4.Problem) == 104


def test_grouped_code_width_validation():
    L = w4.lib()
    A4 = V((1 << 20) + 4)

    def rc(**kw):
        p = w4.Problem(A16, A16, A16, A16, None, A16, 1, 32, 256)
        for k, v in kw.items():
            setattr(p, k, v.value if isinstance(v, ctypes.c_void_p) else v)
        return L.w4a16_gemm_grouped((w4.Problem * 1)(p), 1, None)

    for bits in (1, 2, 3, 5, 16, -4):
        assert rc(wbits=bits) == -3, bits
    assert rc(wbits=8, o_row_ptr=A4, o_col=A4) == -1            # outliers: all three or none
    assert rc(wbits=8, dtype=w4.DTYPE_BF16, X=ODD) == -2        # bf16 with INT8 is validated
    assert rc(wbits=8, N=32768, K=65536) == -1                  # 2 GiB of INT8 codes
    assert rc(wbits=8, K=100) == -1
    assert rc(wbits=8, X=ODD) == -2


def test_bf16_bit_helpers_match_torch():
    import numpy as np
    import torch
    from workloads import bf16_bits_to_f64, to_bf16_bits
    x = np.random.default_rng(3).standard_normal(4096).astype(np.float32) * 50
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]      # ties round to even
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_bf16_bits(x), want)
    assert np.array_equal(bf16_bits_to_f64(want),
                          torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_scratch_sizes_match_header():
    """The binding's copies of the header's scratch sizes."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "w4a16.h")).read()
    for name, val in (("W4A16_STATIC_SCRATCH_BYTES", w4.STATIC_SCRATCH_BYTES),
                      ("W4A16_SHARED_SCRATCH_BYTES", w4.SHARED_SCRATCH_BYTES)):
        m = re.search(r"#define " + name + r" \(\(size_t\)(\d+) << (\d+)\)", hdr)
        assert m and int(m.group(1)) << int(m.group(2)) == val


def test_gemm_without_workspace_validates_first():
    """w4a16_gemm and w4a16_gemm_grouped take the shared scratch only after the same
    host-side validation: bad arguments return before any HIP call (no GPU here)."""
    L = w4.lib()
    assert L.w4a16_gemm(A16, A16, A16, A16, None, A16, 64, 272, 100, None) == -1   # K % 128
    assert L.w4a16_gemm(ODD, A16, A16, A16, None, A16, 64, 272, 128, None) == -2   # alignment
    assert L.w4a16_gemm(A16, A16, A16, A16, None, A16, 0, 272, 128, None) == 0     # empty batch
    bad = (w4.Problem * 1)(w4.Problem(A16, A16, A16, A16, None, A16, 64, 270, 128))
    assert L.w4a16_gemm_grouped(bad, 1, None) == -1
