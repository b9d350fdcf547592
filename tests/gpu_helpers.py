"""Shared pieces of the GPU parity tests: device setup, tolerance, packed-byte views."""
import sys

import numpy as np
import pytest

# Output tolerance for the fp16 dequantize-matmul against the fp64 oracle:
# relative L2 error <= 1e-3 and every element within 5e-3 * max|y_ref|.
# Error budget behind it: X * s rounded to fp16 (unit roundoff 2^-11), the
# tiled path's fp16 dequantized weight (2^-11), fp32 accumulation, and the
# final fp16 rounding of Y (2^-11): independent relative errors of about
# 3e-4 rms in total, a third of the bound.
REL_L2 = 1e-3
MAX_REL = 5e-3
# bf16 activations (X and Y in bf16): the same three roundings (X * s, the tiled
# kernel's dequantized weight, Y) at bf16's unit roundoff 2^-8 instead of fp16's
# 2^-11, so both bounds scale by 8.
REL_L2_BF16 = 8e-3
MAX_REL_BF16 = 4e-2


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def note(msg):
    """Name the case before a GPU step, so a fault leaves a trace."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def errors(Y, Yref):
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    d = Y - Yref
    nref = np.linalg.norm(Yref)
    mref = np.abs(Yref).max(initial=0.0)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mx = np.abs(d).max(initial=0.0) / mref if mref > 0 else np.abs(d).max(initial=0.0)
    return rel, mx


def assert_close(Y, Yref, tag="", rel_l2=REL_L2, max_rel=MAX_REL):
    assert np.all(np.isfinite(np.asarray(Y, dtype=np.float64))), f"{tag}: non-finite output"
    rel, mx = errors(Y, Yref)
    assert rel <= rel_l2 and mx <= max_rel, f"{tag}: rel-L2 {rel:.3e}, max-rel {mx:.3e}"
    return rel, mx


def h16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)
