"""Seeded synthetic workloads: the five problem configurations and their input generators.

This package holds shapes and random inputs only.  It contains none of the
quantization or matmul arithmetic, so the CPU oracle (``oracle/``) and the HIP
path (``weight_only_int4_group_amd``) can both draw their inputs from it without
sharing any of the method's code.
"""
from .configs import CONFIGS, Config, Matrix, config_by_name
from .synth import (activations, activations_bf16, awq_scales, bf16_bits_to_f64, to_bf16_bits,
                    weights, weight_rows)

__all__ = ["CONFIGS", "Config", "Matrix", "config_by_name", "activations", "activations_bf16",
           "bf16_bits_to_f64", "to_bf16_bits", "awq_scales",
           "weights", "weight_rows"]
