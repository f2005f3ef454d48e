"""Seeded synthetic inputs for the block-wise int4 matmul workloads.

This module only draws random numbers: it holds none of the method's
arithmetic, so the CPU oracle and the HIP path can share it.  The draws give
the operands directly in their stored form (ONNX MatMulNBits byte layout for
codes and zero points, fp16/fp32 for activations and scales):

* codes: uniform random bytes ``u8[N, k_blocks, group/2]``.  Every nibble of a
  uniform byte is uniform on 0..15 and independent of the others, which is the
  stated code distribution.
* zero points: uniform random bytes ``u8[N, ceil(k_blocks/2)]`` (nibbles
  uniform on 0..15), or absent (the default zero point 8 applies).
* scales: continuous uniform in [lo, hi] in fp64, rounded once (RNE) to the
  storage dtype.
* activations: standard normal times sigma in fp64, rounded once (RNE) to the
  activation dtype.

Seeds are tuples fed to ``numpy.random.default_rng`` (PCG64).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group: int
    act_dtype: str            # "f16" | "f32"
    scale_dtype: str          # "f16" | "f32"
    scale_range: Tuple[float, float]
    zero_points: bool
    sigma: float = 1.0
    fused_gate_up: bool = False
    seed: Tuple[int, ...] = (0,)

    @property
    def k_blocks(self) -> int:
        return (self.K + self.group - 1) // self.group


# The five measured workloads, named by what they are.
TINY_GEMV = Workload("tiny GEMV M=1 K=256 N=256 g=32 f32", 1, 256, 256, 32,
                     "f32", "f32", (0.005, 0.02), False, seed=(1,))
DECODE_GEMV = Workload("decode GEMV M=1 K=4096 N=4096 g=32 f16 asym-zp", 1, 4096, 4096, 32,
                       "f16", "f16", (0.005, 0.02), True, seed=(2,))
GATE_UP_SWIGLU = Workload("fused gate/up SwiGLU M=1 K=4096 N=11008 g=128 f16", 1, 4096, 11008, 128,
                          "f16", "f16", (0.002, 0.01), False, fused_gate_up=True, seed=(3,))
SMALL_M_GEMM = Workload("small-M GEMM K=4096 N=14336 g=64 f16 asym-zp", 16, 4096, 14336, 64,
                        "f16", "f16", (0.005, 0.02), True, seed=(4,))
PREFILL_GEMM = Workload("prefill GEMM M=2048 K=4096 N=14336 g=128 f16 asym-zp", 2048, 4096, 14336, 128,
                        "f16", "f16", (0.002, 0.01), True, sigma=0.5, seed=(5,))
# The next measured workload: the MLP's down projection at M=1 (tall and
# skinny, K > N), the step after the fused gate/up.
DOWN_PROJ_GEMV = Workload("down-projection GEMV M=1 K=11008 N=4096 g=128 f16", 1, 11008, 4096, 128,
                          "f16", "f16", (0.002, 0.01), False, seed=(6,))
# Int8 activations (accuracy_level 4): fp32 activations, scales and outputs;
# the decode shape with block 32 and no zero points (the symmetric form the
# pages give their own int8 GEMV), and the prefill shape.
ACC4_DECODE = Workload("int8-activation decode GEMV M=1 K=4096 N=4096 g=32 f32 sym", 1, 4096, 4096, 32,
                       "f32", "f32", (0.005, 0.02), False, seed=(7,))
ACC4_PREFILL = Workload("int8-activation prefill GEMM M=2048 K=4096 N=14336 g=128 f32 asym-zp", 2048, 4096,
                        14336, 128, "f32", "f32", (0.002, 0.01), True, seed=(8,))
SMALL_M_VALUES = (2, 4, 8, 16)


@dataclass
class Weight:
    N: int
    K: int
    group: int
    packed: np.ndarray                 # u8 [N, k_blocks, group/2]
    scales: np.ndarray                 # f16 | f32 [N, k_blocks]
    zero_points: Optional[np.ndarray]  # u8 [N, ceil(k_blocks/2)] or None


def _np_dtype(name: str):
    return {"f16": np.float16, "f32": np.float32}[name]


def weight(N: int, K: int, group: int, scale_dtype: str, scale_range, zero_points: bool,
           seed: Tuple[int, ...]) -> Weight:
    kb = (K + group - 1) // group
    packed = np.random.default_rng(seed + (1,)).integers(
        0, 256, size=(N, kb, group // 2), dtype=np.uint8)
    lo, hi = scale_range
    scales = np.random.default_rng(seed + (2,)).uniform(lo, hi, size=(N, kb)).astype(
        _np_dtype(scale_dtype))
    zp = None
    if zero_points:
        zp = np.random.default_rng(seed + (3,)).integers(
            0, 256, size=(N, (kb + 1) // 2), dtype=np.uint8)
    return Weight(N, K, group, packed, scales, zp)


def activation(M: int, K: int, dtype: str, sigma: float, seed: Tuple[int, ...]) -> np.ndarray:
    a = np.random.default_rng(seed + (0,)).standard_normal((M, K)) * sigma
    return a.astype(_np_dtype(dtype))


def workload_weights(w: Workload):
    """The weight(s) of a workload: one Weight, or (gate, up) when fused."""
    if w.fused_gate_up:
        return (weight(w.N, w.K, w.group, w.scale_dtype, w.scale_range, w.zero_points, w.seed + (0,)),
                weight(w.N, w.K, w.group, w.scale_dtype, w.scale_range, w.zero_points, w.seed + (1,)))
    return weight(w.N, w.K, w.group, w.scale_dtype, w.scale_range, w.zero_points, w.seed)


def workload_activation(w: Workload, M: Optional[int] = None) -> np.ndarray:
    M = w.M if M is None else M
    return activation(M, w.K, w.act_dtype, w.sigma, w.seed + (M,))
