"""The five problem configurations (shapes, batch sizes M, which inputs carry an AWQ scale).

A weight matrix is stored like a linear layer's weight: ``W[N][K]`` (output
features x input features), and the product is ``Y[M][N] = X[M][K] . W_hat^T``.
Quantization groups are 128 consecutive input features of one output row.

Shapes:
  * 1024 x 1024 single GEMV -- the 1024x1024 matrix used as the worked example
    in the mhpq.cn practitioner notes, section 2.1 (INT4 footprint is a quarter
    of FP16).
  * Llama-3-8B-shaped decoder layer (hidden 4096, kv 1024, intermediate 14336),
    decode (M=1) and speculative-verify (M = draft length + 1 in {2, 5, 9}).
    The verify batch follows the aiwing.uk chapter 22, section 22.1 description
    of the target model checking all draft positions in one forward pass.
  * Qwen2-7B-shaped layer (hidden 3584, kv 512, intermediate 18944) at batched
    decode M in {16, 64, 256}.
  * 70B-shaped layer (hidden 8192, kv 1024, intermediate 28672) at prefill
    M=4096; the discosf.com tutorial, section 1.1, describes prefill as one
    large compute-bound matmul and decode as a bandwidth-bound weight stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int  # output features (rows of W)
    K: int  # input features (columns of W); a multiple of 128


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    Ms: tuple
    matrices: tuple
    awq: bool             # an AWQ per-input-channel scale s is present
    act_outliers: bool    # 1% of activation channels scaled by 20
    weight_key: int       # generator key for W and s (verify reuses the decode layer's weights)
    description: str = field(default="", compare=False)

    @property
    def weight_count(self) -> int:
        return sum(m.N * m.K for m in self.matrices)


def _layer(hidden: int, kv: int, inter: int) -> tuple:
    return (
        Matrix("q", hidden, hidden),
        Matrix("k", kv, hidden),
        Matrix("v", kv, hidden),
        Matrix("o", hidden, hidden),
        Matrix("gate", inter, hidden),
        Matrix("up", inter, hidden),
        Matrix("down", hidden, inter),
    )


_L8B = _layer(4096, 1024, 14336)
_QWEN = _layer(3584, 512, 18944)
_L70B = _layer(8192, 1024, 28672)

CONFIGS = (
    Config(0, "gemv_1024", (1,), (Matrix("w", 1024, 1024),), awq=False, act_outliers=False,
           weight_key=0, description="single 1024x1024 GEMV, M=1, s=1"),
    Config(1, "llama3_8b_decode", (1,), _L8B, awq=True, act_outliers=False, weight_key=1,
           description="Llama-3-8B-shaped decoder layer, M=1, AWQ s ~ LogNormal(0, 0.5)"),
    Config(2, "llama3_8b_verify", (2, 5, 9), _L8B, awq=True, act_outliers=False, weight_key=1,
           description="8B layer at speculative-verify batch M = draft length + 1"),
    Config(3, "qwen2_7b_batched_decode", (16, 64, 256), _QWEN, awq=False, act_outliers=False,
           weight_key=3, description="Qwen2-7B-shaped layer, batched decode, no AWQ scale"),
    Config(4, "llama_70b_prefill", (4096,), _L70B, awq=True, act_outliers=True, weight_key=4,
           description="70B-shaped layer, prefill M=4096, AWQ s, 1% activation channels x20"),
)


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
