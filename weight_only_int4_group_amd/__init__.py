"""Weight-only INT4 per-group quantization (W4A16) for AMD Instinct MI355X.

Thin ctypes binding over ``libw4a16.so`` (C ABI in ``include/w4a16.h``).  The
binding only marshals arguments: it checks tensor dtypes/devices, allocates
outputs with torch (device memory and streams are torch's), and passes raw
pointers and the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.

    from weight_only_int4_group_amd import w4a16_quantize_pack, w4a16_gemm
    pw = w4a16_quantize_pack(W, s)        # W: fp16 [N][K] cuda, s: fp16 [K] or None
    Y = w4a16_gemm(X, pw, s)              # X: fp16 [M][K] cuda -> Y: fp16 [M][N]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from .build import LIB_PATH as _BUILT_LIB

# the in-tree build; W4A16_LIB names another build of the same sources (the
# host-sanitized one, for CPU runs of the validation tests)
LIB_PATH = os.environ.get("W4A16_LIB") or _BUILT_LIB

__all__ = [
    "W4A16Error", "PackedWeight", "GROUP", "PATH_AUTO", "PATH_SKINNY", "PATH_TILED",
    "PATH_SKINNY_WINDOW", "QUANT_ASYM", "QUANT_SYM", "QUANT_ASYM_CHANNEL", "QUANT_ASYM_TENSOR",
    "QUANT_ASYM8",
    "lib",
    "w4a16_packed_sizes", "w4a16_quantize_pack", "w4a16_gemm", "w4a16_gemm_path",
    "w4a16_select_path", "w4a16_strerror", "w4a16_version", "EXPORTED_SYMBOLS",
    "w4a16_gemm_grouped", "GroupedCall", "w4a16_spec_verify",
    "w4a16_spec_verify_workspace_size", "SpecVerifyCall", "w4a16_quantize_pack_outliers",
    "w4a16_outlier_workspace_size", "page_outlier_count", "DTYPE_F16", "DTYPE_BF16",
    "w4a16_quantize_pack_gptq", "w4a16_gemm_grouped_static", "STATIC_SCRATCH_BYTES",
    "SHARED_SCRATCH_BYTES",
]

GROUP = 128
PATH_AUTO, PATH_SKINNY, PATH_TILED, PATH_SKINNY_WINDOW = 0, 1, 2, 3
QUANT_ASYM, QUANT_SYM, QUANT_ASYM_CHANNEL, QUANT_ASYM_TENSOR, QUANT_ASYM8 = 0, 1, 2, 3, 4
DTYPE_F16, DTYPE_BF16 = 0, 1
STATUS = {0: "W4A16_OK", -1: "W4A16_EINVAL", -2: "W4A16_EALIGN", -3: "W4A16_EUNSUPPORTED",
          -4: "W4A16_ENONFINITE", -5: "W4A16_ERANGE", -6: "W4A16_EHIP", -7: "W4A16_ESCRATCH"}
STATIC_SCRATCH_BYTES = 64 << 20   # W4A16_STATIC_SCRATCH_BYTES
SHARED_SCRATCH_BYTES = 32 << 20   # W4A16_SHARED_SCRATCH_BYTES
EXPORTED_SYMBOLS = ("w4a16_packed_sizes", "w4a16_packed_sizes_mode", "w4a16_quantize_pack",
                    "w4a16_quantize_pack_mode",
                    "w4a16_gemm",
                    "w4a16_gemm_path", "w4a16_gemm_grouped", "w4a16_gemm_grouped_ws",
                    "w4a16_gemm_grouped_static",
                    "w4a16_gemm_workspace_size", "w4a16_outlier_workspace_size",
                    "w4a16_gptq_workspace_size", "w4a16_quantize_pack_gptq",
                    "w4a16_quantize_pack_outliers", "w4a16_spec_verify",
                    "w4a16_spec_verify_workspace_size", "w4a16_select_path",
                    "w4a16_strerror", "w4a16_version")


class Problem(ctypes.Structure):
    """Mirror of the C struct w4a16_problem."""
    _fields_ = [("X", ctypes.c_void_p), ("Wq", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("s", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("o_row_ptr", ctypes.c_void_p), ("o_col", ctypes.c_void_p),
                ("o_val", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("wbits", ctypes.c_int32)]


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({w4a16_strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4a16.so (built in-tree by ``weight_only_int4_group_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m weight_only_int4_group_amd.build` (needs hipcc)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    L.w4a16_packed_sizes.argtypes = [i64, i64, sz, sz, sz]
    L.w4a16_packed_sizes_mode.argtypes = [i64, i64, ctypes.c_int, sz, sz, sz]
    L.w4a16_quantize_pack.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp]
    L.w4a16_quantize_pack_mode.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp, vp, vp, vp]
    L.w4a16_gemm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    L.w4a16_gemm_path.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    L.w4a16_gemm_grouped.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, vp]
    L.w4a16_gemm_grouped_ws.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, vp,
                                        ctypes.c_size_t, vp]
    L.w4a16_gemm_workspace_size.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, sz]
    L.w4a16_gemm_grouped_static.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, vp]
    L.w4a16_spec_verify.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp,
                                    vp, vp]
    L.w4a16_spec_verify_workspace_size.argtypes = [i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    L.w4a16_outlier_workspace_size.argtypes = [i64, i64, sz]
    L.w4a16_quantize_pack_outliers.argtypes = [vp, vp, i64, i64, ctypes.c_int, i64, vp, vp, vp,
                                               vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.w4a16_gptq_workspace_size.argtypes = [i64, i64, i64, sz]
    L.w4a16_quantize_pack_gptq.argtypes = [vp, vp, i64, i64, vp, i64, ctypes.c_double, vp, vp, vp,
                                           vp, ctypes.c_size_t, vp]
    L.w4a16_select_path.argtypes = [i64, i64, i64]
    L.w4a16_strerror.argtypes = [ctypes.c_int]
    L.w4a16_strerror.restype = ctypes.c_char_p
    L.w4a16_version.argtypes = []
    for name in ("w4a16_packed_sizes", "w4a16_packed_sizes_mode", "w4a16_quantize_pack",
                 "w4a16_quantize_pack_mode",
                 "w4a16_gemm", "w4a16_gemm_path",
                 "w4a16_gemm_grouped", "w4a16_gemm_grouped_ws", "w4a16_gemm_workspace_size",
                 "w4a16_gemm_grouped_static",
                 "w4a16_spec_verify", "w4a16_spec_verify_workspace_size", "w4a16_select_path",
                 "w4a16_outlier_workspace_size", "w4a16_quantize_pack_outliers",
                 "w4a16_gptq_workspace_size", "w4a16_quantize_pack_gptq",
                 "w4a16_version"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def w4a16_strerror(status: int) -> str:
    return lib().w4a16_strerror(status).decode()


def w4a16_version() -> int:
    return lib().w4a16_version()


def w4a16_packed_sizes(N: int, K: int, mode: int = QUANT_ASYM) -> tuple:
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().w4a16_packed_sizes_mode(N, K, mode, ctypes.byref(a), ctypes.byref(b),
                                       ctypes.byref(c))
    if rc:
        raise W4A16Error(rc, "w4a16_packed_sizes")
    return a.value, b.value, c.value


def w4a16_select_path(M: int, N: int, K: int) -> int:
    return lib().w4a16_select_path(M, N, K)


@dataclass
class PackedWeight:
    """Packed weight: INT4 codes (uint8, N*K/2 bytes) or, with wbits = 8, INT8 codes (N*K
    bytes), and the fp16 scale and zero-point buffers (flat, in the 4-group-quad layout
    of include/w4a16.h); with fp16 outliers
    (w4a16_quantize_pack_outliers) also their row pointers (int32 [N+1]), columns
    (int32) and values (fp16)."""
    wq: "object"
    scales: "object"
    zeros: "object"
    N: int
    K: int
    o_row_ptr: "object" = None
    o_col: "object" = None
    o_val: "object" = None
    wbits: int = 4      # 8: INT8 codes (QUANT_ASYM8)

    def outlier_ptrs(self):
        """(row_ptr, col, val) device pointers, or three None without outliers."""
        if self.o_row_ptr is None or self.o_col is None or self.o_col.numel() == 0:
            return None, None, None
        torch = _torch()
        return (_dev_ptr(self.o_row_ptr, "o_row_ptr", torch.int32, self.N + 1),
                _dev_ptr(self.o_col, "o_col", torch.int32),
                _dev_ptr(self.o_val, "o_val", torch.float16, self.o_col.numel()))


def _torch():
    import torch
    return torch


def _stream_handle(dev):
    return ctypes.c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def _dev_ptr(t, name, dtype=None, numel=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def w4a16_quantize_pack(W, s=None, out: PackedWeight | None = None,
                        mode: int = QUANT_ASYM) -> PackedWeight:
    """Quantize fp16 W[N][K] (AWQ scale s[K] or None) into a PackedWeight (blocks).
    mode: QUANT_ASYM (w4a16_quantize_pack), QUANT_SYM (signed -7..7 grid),
    QUANT_ASYM_CHANNEL or QUANT_ASYM_TENSOR (one scale per row or per tensor), or
    QUANT_ASYM8 (INT8 codes, one byte per weight)."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N][K]")
    N, K = W.shape
    wq_b, sc_b, z_b = w4a16_packed_sizes(N, K, mode)
    if out is None:
        out = PackedWeight(torch.empty(wq_b, dtype=torch.uint8, device=W.device),
                           torch.empty(sc_b // 2, dtype=torch.float16, device=W.device),
                           torch.empty(z_b // 2, dtype=torch.float16, device=W.device),
                           N, K, wbits=8 if mode == QUANT_ASYM8 else 4)
    rc = lib().w4a16_quantize_pack_mode(
        _dev_ptr(W, "W", torch.float16), _dev_ptr(s, "s", torch.float16, K), N, K, mode,
        _dev_ptr(out.wq, "wq", torch.uint8, wq_b),
        _dev_ptr(out.scales, "scales", torch.float16, sc_b // 2),
        _dev_ptr(out.zeros, "zeros", torch.float16, z_b // 2), _stream_handle(W.device))
    if rc:
        raise W4A16Error(rc, "w4a16_quantize_pack")
    out.wbits = 8 if mode == QUANT_ASYM8 else 4
    return out


def page_outlier_count(N: int, K: int) -> int:
    """The 0.1% share of an N x K matrix kept in fp16 by the mhpq.cn notes (sec.2.2),
    rounded to the nearest integer."""
    return (N * K + 500) // 1000


def w4a16_outlier_workspace_size(N: int, K: int) -> int:
    n = ctypes.c_size_t()
    rc = lib().w4a16_outlier_workspace_size(N, K, ctypes.byref(n))
    if rc:
        raise W4A16Error(rc, "w4a16_outlier_workspace_size")
    return n.value


def w4a16_quantize_pack_outliers(W, s=None, count: int | None = None,
                                 mode: int = QUANT_ASYM) -> PackedWeight:
    """Keep the `count` largest |W / s| of fp16 W[N][K] in fp16 (default: the 0.1% share)
    and quantize the rest into a PackedWeight that carries the outliers."""
    torch = _torch()
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N][K]")
    N, K = W.shape
    if count is None:
        count = page_outlier_count(N, K)
    wq_b, sc_b, z_b = w4a16_packed_sizes(N, K, mode)
    dev = W.device
    pw = PackedWeight(torch.empty(wq_b, dtype=torch.uint8, device=dev),
                      torch.empty(sc_b // 2, dtype=torch.float16, device=dev),
                      torch.empty(z_b // 2, dtype=torch.float16, device=dev), N, K,
                      torch.empty(N + 1, dtype=torch.int32, device=dev),
                      torch.empty(max(count, 1), dtype=torch.int32, device=dev)[:count],
                      torch.empty(max(count, 1), dtype=torch.float16, device=dev)[:count],
                      8 if mode == QUANT_ASYM8 else 4)
    ws = torch.empty(w4a16_outlier_workspace_size(N, K), dtype=torch.uint8, device=dev)
    rc = lib().w4a16_quantize_pack_outliers(
        _dev_ptr(W, "W", torch.float16), _dev_ptr(s, "s", torch.float16, K), N, K, mode, count,
        _dev_ptr(pw.wq, "wq", torch.uint8, wq_b),
        _dev_ptr(pw.scales, "scales", torch.float16, sc_b // 2),
        _dev_ptr(pw.zeros, "zeros", torch.float16, z_b // 2),
        _dev_ptr(pw.o_row_ptr, "o_row_ptr", torch.int32, N + 1),
        ctypes.c_void_p(pw.o_col.data_ptr()), ctypes.c_void_p(pw.o_val.data_ptr()),
        _dev_ptr(ws, "workspace", torch.uint8), ws.numel(), _stream_handle(dev))
    if rc:
        raise W4A16Error(rc, "w4a16_quantize_pack_outliers")
    return pw


def w4a16_quantize_pack_gptq(W, s, Xcal, damp: float = 0.01) -> PackedWeight:
    """GPTQ quantize-and-pack of fp16 W[N][K] (AWQ s[K] or None) with fp16 calibration
    activations Xcal[n][K]: the packed format of w4a16_quantize_pack."""
    torch = _torch()
    if W.dim() != 2 or Xcal.dim() != 2 or Xcal.shape[1] != W.shape[1]:
        raise ValueError("W must be [N][K] and Xcal [n][K]")
    N, K = W.shape
    n = Xcal.shape[0]
    wq_b, sc_b, z_b = w4a16_packed_sizes(N, K)
    dev = W.device
    pw = PackedWeight(torch.empty(wq_b, dtype=torch.uint8, device=dev),
                      torch.empty(sc_b // 2, dtype=torch.float16, device=dev),
                      torch.empty(z_b // 2, dtype=torch.float16, device=dev), N, K)
    nb = ctypes.c_size_t()
    rc = lib().w4a16_gptq_workspace_size(N, K, n, ctypes.byref(nb))
    if rc:
        raise W4A16Error(rc, "w4a16_gptq_workspace_size")
    ws = torch.empty(nb.value, dtype=torch.uint8, device=dev)
    rc = lib().w4a16_quantize_pack_gptq(
        _dev_ptr(W, "W", torch.float16), _dev_ptr(s, "s", torch.float16, K), N, K,
        _dev_ptr(Xcal, "Xcal", torch.float16), n, float(damp),
        _dev_ptr(pw.wq, "wq", torch.uint8, wq_b),
        _dev_ptr(pw.scales, "scales", torch.float16, sc_b // 2),
        _dev_ptr(pw.zeros, "zeros", torch.float16, z_b // 2),
        _dev_ptr(ws, "workspace", torch.uint8), ws.numel(), _stream_handle(dev))
    if rc:
        raise W4A16Error(rc, "w4a16_quantize_pack_gptq")
    return pw


def w4a16_gemm_path(X, pw: PackedWeight, s=None, path: int = PATH_AUTO, out=None):
    """Y[M][N] = X[M][K] . dequant(pw)^T (fp16), on the current stream, asynchronously.
    (Without fp16 outliers: the forced-path entry point does not take them.)"""
    torch = _torch()
    if pw.outlier_ptrs()[0] is not None:
        raise ValueError("w4a16_gemm_path takes no fp16 outliers; use w4a16_gemm")
    if pw.wbits != 4:
        raise ValueError("w4a16_gemm_path takes INT4 codes only; use w4a16_gemm")
    if X.dim() != 2 or X.shape[1] != pw.K:
        raise ValueError("X must be [M][K] with K matching the packed weight")
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float16, device=X.device)
    elif tuple(out.shape) != (M, pw.N):
        raise ValueError("out must be [M][N]")
    rc = lib().w4a16_gemm_path(
        _dev_ptr(X, "X", torch.float16), _dev_ptr(pw.wq, "wq", torch.uint8),
        _dev_ptr(pw.scales, "scales", torch.float16), _dev_ptr(pw.zeros, "zeros", torch.float16),
        _dev_ptr(s, "s", torch.float16, pw.K), _dev_ptr(out, "out", torch.float16),
        M, pw.N, pw.K, path, _stream_handle(X.device))
    if rc:
        raise W4A16Error(rc, "w4a16_gemm")
    return out


def w4a16_gemm(X, pw: PackedWeight, s=None, out=None):
    """Y[M][N] = X[M][K] . dequant(pw)^T through the grouped entry point with a workspace,
    so large-M calls may split K across workgroups.  X (and Y) fp16 or bf16."""
    torch = _torch()
    if X.dim() != 2 or X.shape[1] != pw.K:
        raise ValueError("X must be [M][K] with K matching the packed weight")
    if out is None:
        out = torch.empty((X.shape[0], pw.N), dtype=X.dtype, device=X.device)
    GroupedCall([(X, pw, s, out)])()
    return out


class GroupedCall:
    """A prepared w4a16_gemm_grouped_ws call: the problem array is marshalled and the
    workspace (w4a16_gemm_workspace_size bytes, a torch tensor owned by this object)
    allocated once, so each call is a single C call on the current stream (for
    captured or repeated launches over the same buffers).  Items are (X,
    PackedWeight, s or None, Y).  Calls of one object must not overlap in time on
    different streams, since they share the workspace.  With ``static=True`` the call
    goes to w4a16_gemm_grouped_static instead: no workspace is allocated here, the
    library's own static scratch serves (all such calls on a GPU share it).  With
    ``workspace=False`` it goes to w4a16_gemm_grouped, which takes no workspace
    argument (the library's event-ordered shared scratch serves when it fits).  A
    uint8 device tensor as ``workspace`` is used instead of a new one (calls that
    share it must not overlap in time)."""

    def __init__(self, items, stream=None, workspace=True, static=False):
        torch = _torch()
        self.items = list(items)  # keep the tensors alive
        # a fixed HIP stream (e.g. torch.cuda.current_stream().cuda_stream) saves
        # looking up torch's current stream on every call
        self.stream = None if stream is None else ctypes.c_void_p(stream)
        self.array = (Problem * len(self.items))()
        for i, (X, pw, s, Y) in enumerate(self.items):
            if X.dim() != 2 or X.shape[1] != pw.K or tuple(Y.shape) != (X.shape[0], pw.N):
                raise ValueError(f"problem {i}: X must be [M][K] and Y [M][N]")
            if X.dtype not in (torch.float16, torch.bfloat16):
                raise TypeError(f"problem {i}: X must be float16 or bfloat16")
            self.array[i] = Problem(
                _dev_ptr(X, "X", X.dtype),
                _dev_ptr(pw.wq, "wq", torch.uint8, pw.N * pw.K * pw.wbits // 8),
                _dev_ptr(pw.scales, "scales", torch.float16),
                _dev_ptr(pw.zeros, "zeros", torch.float16), _dev_ptr(s, "s", torch.float16, pw.K),
                _dev_ptr(Y, "Y", X.dtype), X.shape[0], pw.N, pw.K, *pw.outlier_ptrs(),
                DTYPE_BF16 if X.dtype == torch.bfloat16 else DTYPE_F16, pw.wbits)
        self.device = self.items[0][0].device if self.items else None
        self.ws, self.ws_ptr, self.ws_bytes = None, None, 0
        self.static = static
        self.use_ws = workspace is not False
        if self.use_ws and self.items and not static:
            nb = ctypes.c_size_t()
            rc = lib().w4a16_gemm_workspace_size(self.array, len(self.items), ctypes.byref(nb))
            if rc:
                raise W4A16Error(rc, "w4a16_gemm_workspace_size")
            if nb.value:
                if isinstance(workspace, torch.Tensor):  # a caller's buffer, shared by calls
                    if (not workspace.is_cuda or workspace.dtype != torch.uint8
                            or not workspace.is_contiguous() or workspace.numel() < nb.value):
                        raise ValueError(f"workspace must be a contiguous uint8 device tensor "
                                         f"of at least {nb.value} bytes")
                    self.ws = workspace
                else:
                    self.ws = torch.empty(nb.value, dtype=torch.uint8, device=self.device)
                self.ws_ptr, self.ws_bytes = self.ws.data_ptr(), nb.value

    def __call__(self):
        if not self.items:
            return
        st = self.stream if self.stream is not None else _stream_handle(self.device)
        if self.static:
            rc = lib().w4a16_gemm_grouped_static(self.array, len(self.items), st)
            if rc:
                raise W4A16Error(rc, "w4a16_gemm_grouped_static")
            return
        if not self.use_ws:
            rc = lib().w4a16_gemm_grouped(self.array, len(self.items), st)
            if rc:
                raise W4A16Error(rc, "w4a16_gemm_grouped")
            return
        rc = lib().w4a16_gemm_grouped_ws(self.array, len(self.items), self.ws_ptr,
                                         self.ws_bytes, st)
        if rc:
            raise W4A16Error(rc, "w4a16_gemm_grouped_ws")


def w4a16_gemm_grouped(items):
    """Several independent Y = X . dequant(pw)^T in as few launches as possible.
    items: list of (X, PackedWeight, s or None); returns the list of Y tensors."""
    torch = _torch()
    full = [(X, pw, s, torch.empty((X.shape[0], pw.N), dtype=X.dtype, device=X.device))
            for (X, pw, s) in items]
    GroupedCall(full)()
    return [it[3] for it in full]


def w4a16_gemm_grouped_static(items):
    """w4a16_gemm_grouped with the library's static scratch as the workspace (no device
    allocation by the library; outputs are allocated here).  items: list of (X,
    PackedWeight, s or None); returns the list of Y tensors."""
    torch = _torch()
    full = [(X, pw, s, torch.empty((X.shape[0], pw.N), dtype=X.dtype, device=X.device))
            for (X, pw, s) in items]
    GroupedCall(full, static=True)()
    return [it[3] for it in full]


def w4a16_spec_verify_workspace_size(B: int, K: int, V: int) -> int:
    n = ctypes.c_size_t()
    rc = lib().w4a16_spec_verify_workspace_size(B, K, V, ctypes.byref(n))
    if rc:
        raise W4A16Error(rc, "w4a16_spec_verify_workspace_size")
    return n.value


class SpecVerifyCall:
    """A prepared w4a16_spec_verify call over fixed buffers: shapes are checked, pointers
    marshalled and the workspace allocated once, so each call is a single C call (two
    kernel launches) on the stream.

    p_target fp32 [B][K+1][V], p_draft fp32 [B][K][V], draft int32 [B][K], u_accept fp32
    [B][K], u_sample fp32 [B] (device tensors).  Each call writes n_accepted and token,
    int32 [B] each: the number of accepted drafts and the token drawn after them (-1 if
    the row it is drawn from has no mass).  `workspace` (uint8 device tensor of at least
    w4a16_spec_verify_workspace_size bytes) is allocated when not given; calls sharing a
    workspace must not overlap in time on different streams."""

    def __init__(self, p_target, p_draft, draft, u_accept, u_sample, out=None, workspace=None,
                 stream=None):
        torch = _torch()
        if p_target.dim() != 3:
            raise ValueError("p_target must be [B][K+1][V]")
        B, K1, V = p_target.shape
        K = K1 - 1
        if K < 0:
            raise ValueError("p_target needs at least one position")
        if tuple(p_draft.shape) != (B, K, V) or tuple(draft.shape) != (B, K) \
                or tuple(u_accept.shape) != (B, K) or tuple(u_sample.shape) != (B,):
            raise ValueError("p_draft [B][K][V], draft [B][K], u_accept [B][K], u_sample [B]")
        ws_bytes = w4a16_spec_verify_workspace_size(B, K, V)
        dev = p_target.device
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        elif workspace.numel() < ws_bytes:
            raise ValueError(f"workspace needs {ws_bytes} bytes")
        if out is None:
            out = (torch.empty(B, dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev))
        self.out = out
        self.keep = (p_target, p_draft, draft, u_accept, u_sample, workspace)
        self.device = dev
        self.stream = None if stream is None else ctypes.c_void_p(stream)
        self.args = (
            _dev_ptr(p_target, "p_target", torch.float32),
            _dev_ptr(p_draft, "p_draft", torch.float32),
            _dev_ptr(draft, "draft", torch.int32), _dev_ptr(u_accept, "u_accept", torch.float32),
            _dev_ptr(u_sample, "u_sample", torch.float32), B, K, V,
            _dev_ptr(workspace, "workspace", torch.uint8), workspace.numel(),
            _dev_ptr(out[0], "n_accepted", torch.int32, B),
            _dev_ptr(out[1], "token", torch.int32, B))

    def __call__(self):
        st = self.stream if self.stream is not None else _stream_handle(self.device)
        rc = lib().w4a16_spec_verify(*self.args, st)
        if rc:
            raise W4A16Error(rc, "w4a16_spec_verify")
        return self.out


def w4a16_spec_verify(p_target, p_draft, draft, u_accept, u_sample, out=None, workspace=None):
    """Speculative-sampling verification of B sequences on the current stream; returns
    (n_accepted, token).  Arguments as for SpecVerifyCall."""
    return SpecVerifyCall(p_target, p_draft, draft, u_accept, u_sample, out, workspace)()
