"""Byte accounting of weight formats.

Bytes per parameter follow the aiwing.uk ch.22 sec.22.3 table (FP32 4, FP16/BF16
2, INT8 1, INT4 0.5, INT2 0.25) and the discosf.com tutorial sec.2.2 sizes; the
group metadata adds one fp16 scale and one fp16 zero point per 128 weights.
TEST INFRASTRUCTURE: see the package docstring for who may import this.
"""
from __future__ import annotations

from fractions import Fraction

BITS = {"fp32": 32, "fp16": 16, "bf16": 16, "int8": 8, "int4": 4, "int2": 2}


def bytes_per_param(fmt: str) -> Fraction:
    return Fraction(BITS[fmt], 8)


def weight_bytes(params: int, fmt: str) -> Fraction:
    """Bytes of the bare weights of ``params`` parameters in ``fmt`` (no metadata)."""
    return params * bytes_per_param(fmt)


def int4_group_bytes(params: int, group: int = 128, meta_bits: int = 32) -> Fraction:
    """INT4 codes plus one fp16 scale and one fp16 zero point (32 bits) per group."""
    return Fraction(params * 4, 8) + Fraction(params * meta_bits, 8 * group)


def packed_sizes(N: int, K: int) -> tuple:
    """(code bytes, scale bytes, zero-point bytes) of one packed [N][K] matrix; the
    metadata holds the groups of a row rounded up to a multiple of 4."""
    if N % 16 or K % 128:
        raise ValueError("N must be a multiple of 16 and K of 128")
    groups = N * (-(-(K // 128) // 4) * 4)
    return N * K // 2, 2 * groups, 2 * groups
