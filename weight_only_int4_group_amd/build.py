"""Compile the HIP sources under csrc/ into libw4a16.so (gfx950), in-tree.

Run as ``python -m weight_only_int4_group_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libw4a16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ("api.hip", "pack.hip", "skinny.hip", "tiled.hip", "spec.hip", "outliers.hip",
           "gptq.hip")
# the plain streaming-read and MFMA-only kernels the benchmark times as its
# bandwidth and matrix-core ceilings:
# its own small library, not part of the W4A16 ABI
CEILING_SOURCES = ("stream_read.hip", "mfma_peak.hip")
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libw4a16_ceiling.so")
# host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the library
# (device code unchanged), for running the argument-validation tests on a CPU
HOSTSAN_LIB_PATH = os.path.join(PKG_DIR, "libw4a16_hostsan.so")
HOST_SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-omit-frame-pointer -g").split()
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # plain (non-packed) fp32 ALU ops only; hipcc's host pass warns that it
        # does not know this device feature, which is harmless
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(sources, out, extra, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *compile_flags(), *srcs, *extra, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH, and the benchmark's streaming-read kernel into
    CEILING_LIB_PATH (always recompiles); returns LIB_PATH."""
    _compile(SOURCES, LIB_PATH, ["-ldl"], verbose)
    _compile(CEILING_SOURCES, CEILING_LIB_PATH, [], verbose)
    return LIB_PATH


def build_host_sanitized(verbose: bool = False) -> str:
    """Compile the library with ASan and UBSan on its host code into HOSTSAN_LIB_PATH.
    Load it with the sanitizer runtime preloaded (the Python interpreter itself is
    not instrumented) and W4A16_LIB pointing at it; its device code is the
    ordinary build's."""
    _compile(SOURCES, HOSTSAN_LIB_PATH, ["-ldl", *HOST_SANITIZE_FLAGS], verbose)
    return HOSTSAN_LIB_PATH


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv[1:]:
        print(build_host_sanitized(verbose=True))
    else:
        print(build(verbose=True))
