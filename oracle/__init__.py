"""CPU oracle for weight-only INT4 per-group quantization and the dequantize-matmul.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the HIP path is checked against.  Only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it; the library ``weight_only_int4_group_amd`` never does, and this package
never imports the library.  Both sides draw their inputs from ``workloads``.

Sources (web pages; cited by page, section and table/equation):
  * [discosf] discosf.com news 6284891, a tutorial on quantization, speculative
    sampling and PD disaggregation in nano-vllm.  Section 2.1: a quantizer maps
    a float range onto an integer range with a scale and a zero point; the
    per-group granularity (e.g. 128 elements per group) is the usual choice for
    4-bit GPTQ/AWQ.  Section 2.2: 70B weights are about 140 GB in FP16, 70 GB in
    INT8, 35 GB in INT4.  Section 2.3: scale and zero point travel with the
    weights; the loader either dequantizes or feeds low-precision operators.
  * [aiwing] aiwing.uk, chapter 22 (advanced inference optimisation), section
    22.3: the bytes-per-parameter table (FP32 4, FP16 2, INT8 1, INT4 0.5,
    INT2 0.25; a 7B model is 28/14/7/3.5/1.75 GB); weight-only quantization
    either dequantizes to FP16 then multiplies, or uses a mixed-precision
    kernel; the AWQ equation W_hat = quant(W / s) * s with s the per-channel
    activation magnitude; weights can be quantized offline.
  * [mhpq] mhpq.cn news 1188791, practitioner notes.  Section 2.1: a 1024x1024
    weight matrix in INT4 takes a quarter of its FP16 size.  Section 2.2: the
    top 0.1% of the weights by magnitude go to an FP16 sub-tensor, merged with
    the INT4 rest by a where(mask, ...).

Readings taken where the pages are silent (each one is listed with its reason
in the design notes of the repository):
  R1 asymmetric unsigned 4-bit codes 0..15 with a zero point;
  R2 groups are 128 consecutive input features of one output row;
  R3 the range of a group is its min and max, widened to include 0;
  R4 scale = (max - min) / 15;  R5 the scale is rounded UP to fp16;
  R6 the zero point is the integer z = rint(-min / scale), stored as fp16,
     and dequantization is (q - z) * scale;
  R7 q = clamp(rint(W' / scale) + z, 0, 15), rint ties to even, applied before
     adding z;  R8 W' = W / s is one correctly rounded fp64 division;
  R9 an all-zero group has scale 0, zero point 0 and codes 0; non-finite W or
     s, or s <= 0, is an error; a scale that overflows fp16 is an error.
The symmetric variant (``quantize_symmetric``, the signed -7..7 grid of [mhpq]
sec.2.1) takes R2, R5, R7's ties, R8 and R9's errors as they are, with
scale = max|W'| / 7 rounded up, signed codes rint(W' / scale) stored + 8 and a
constant zero point 8 (an all-zero group: scale 0, codes 8).
``quantize(..., bits=8)`` is the INT8 (W8A16) variant: codes 0..255 under the same
readings, packed one byte per weight in 2048-byte tiles (``pack_codes8``).
``quantize(..., granularity="channel" | "tensor")`` are the coarser granularities of
[discosf] sec.2.1 (one scale per output channel, or per tensor): the range of
R3 is taken over the row or the whole tensor, and every group slot of the
packed metadata repeats that scale and zero point.
``gptq.quantize_gptq`` is the GPTQ alternative producer of aiwing.uk sec.22.3 (Hessian
H = 2 X^T X from calibration activations, error compensation along each row); its
readings Q1-Q5 are in that module.
The outlier side path (``outliers``, [mhpq] sec.2.2) keeps the largest |W / s|
in fp16 and quantizes the rest with those positions set to 0; its readings
O1-O5 are in that module.
Pins: every function here is checked by tests against facts the pages or the
mathematics fix (bound, grid reconstruction, byte counts, brute force in exact
rationals, integer special case); see tests/test_oracle_*.py.
"""
from .quantizer import (GRANULARITIES, GROUP, QMAX, SYM_QMAX, SYM_ZERO, NonFiniteInput, OracleError,
                        QuantResult, ScaleOverflow, quantize, quantize_symmetric, round_up_fp16)
from .layout import (META_QUAD, TILE_BYTES, TILE_BYTES8, TILE_ROWS, byte_address8, meta_groups,
                     meta_index, nibble_address, pack_codes, pack_codes8, pack_meta, unpack_codes,
                     unpack_codes8, unpack_meta)
from .matmul import dequantize, gemm
from . import accounting, exact, gptq, outliers, spec

__all__ = [
    "GRANULARITIES", "GROUP", "QMAX", "NonFiniteInput", "OracleError", "QuantResult", "ScaleOverflow",
    "quantize", "quantize_symmetric", "SYM_QMAX", "SYM_ZERO", "round_up_fp16", "META_QUAD", "TILE_BYTES", "TILE_ROWS", "meta_groups",
    "meta_index", "nibble_address",
    "pack_codes", "pack_meta", "unpack_codes", "unpack_meta", "dequantize", "gemm",
    "TILE_BYTES8", "byte_address8", "pack_codes8", "unpack_codes8",
    "accounting", "exact", "gptq", "outliers", "spec",
]
