"""Seeded synthetic inputs for the W2A8 linear layer.

This module only draws random numbers and shapes them into arrays. It holds
none of the layer's arithmetic (no ternarization, packing, quantization,
matmul or scaling), so both the CPU oracle and the GPU path can consume its
arrays without sharing any of the method's code.

The workloads follow the benchmark page "如何编译 BitNet W2A8 CUDA 内核并用
test.py 运行 GEMV 加速测试" (section "运行 test.py 做 GEMV 基准测试"): random
int8 activations and random weights, M=1, at its eight (N, K) shapes, plus
the two further shapes it names under "限制与注意事项".  Distributions and
seeds are fixed here so every test, the smoke check and the benchmark draw
the same arrays.

Generator: numpy ``default_rng(seed)`` (PCG64).  Activations are drawn first,
then weights.  Large weight matrices are drawn in row blocks of
``ROW_BLOCK`` rows so memory stays bounded; the block size is part of the
recipe (the same seed always yields the same matrix).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 4096

# The eight GEMV shapes (N, K) of the benchmark page's test script, in its order.
SWEEP_SHAPES = [
    (2560, 2560), (3840, 2560), (13824, 2560), (2560, 6912),
    (3200, 3200), (4800, 3200), (3200, 10240), (20480, 3200),
]
# The two further shapes the kernel source specialises (same page, "限制与注意事项").
LARGE_SHAPES = [(5120, 27648), (55296, 5120)]
# One GPU's share of each large matrix split over 8 GPUs: 55296 rows / 8, and
# 27648 along K / 8 (same value distribution as the large shapes).
SHARD_SHAPES = [(6912, 5120), (5120, 3456)]
# Prefill shapes for the batched product.
GEMM_SHAPES = [(13824, 2560), (2560, 6912)]
GEMM_MS = [8, 128, 512]


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def int8_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """int8 uniform on [-127, 127] (both ends included)."""
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def ternary_uniform(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 matrix [n, k] with values in {-1, 0, 1}, each with probability 1/3."""
    out = np.empty((n, k), dtype=np.int8)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        out[r0:r1] = rng.integers(-1, 2, size=(r1 - r0, k), dtype=np.int8)
    return out


def ternary_sparse(rng: np.random.Generator, n: int, k: int,
                   p_neg: float = 0.2, p_pos: float = 0.2) -> np.ndarray:
    """int8 matrix [n, k]: u ~ U[0,1); -1 if u < p_neg, +1 if u < p_neg + p_pos, else 0."""
    out = np.empty((n, k), dtype=np.int8)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        u = rng.random((r1 - r0, k))
        blk = np.zeros(u.shape, dtype=np.int8)
        blk[u < p_neg + p_pos] = 1
        blk[u < p_neg] = -1
        out[r0:r1] = blk
    return out


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even) and return the 16-bit patterns.

    This is the data type conversion of the activations themselves (the inputs
    are bf16 tensors), not a step of the layer.  NaN inputs are not produced by
    any generator here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gemv_case(n: int, k: int, seed: int, sparse: bool = False):
    """M=1 case: returns (x int8 [k], W int8 [n, k]).

    sparse=False: W entries -1/0/+1 each with probability 1/3.
    sparse=True : P(-1) = P(+1) = 0.2, P(0) = 0.6 (the two large shapes).
    """
    rng = _rng(seed)
    x = int8_uniform(rng, (k,))
    w = ternary_sparse(rng, n, k) if sparse else ternary_uniform(rng, n, k)
    return x, w


def gemv_a4_case(n: int, k: int, seed: int, sparse: bool = False):
    """M=1 case with int4 activations: returns (q int8 [k] uniform in -8..7,
    W int8 [n, k] as in gemv_case)."""
    rng = _rng(seed)
    q = rng.integers(-8, 8, size=(k,), dtype=np.int8)
    w = ternary_sparse(rng, n, k) if sparse else ternary_uniform(rng, n, k)
    return q, w


def gemm_case(m: int, n: int, k: int, seed: int):
    """Batched case: returns (X int8 [m, k], W int8 [n, k]) with uniform ternary W."""
    rng = _rng(seed)
    x = int8_uniform(rng, (m, k))
    w = ternary_uniform(rng, n, k)
    return x, w


def linear_case(m: int, n: int, k: int, seed: int, outlier_p: float = 0.01,
                outlier_mul: float = 10.0, w_std: float = 0.02):
    """Full linear-layer case.

    Activations: standard normal fp32 [m, k]; a fraction ``outlier_p`` of the
    entries (mask u < outlier_p) is multiplied by ``outlier_mul``; then rounded
    to bf16 (returned as uint16 bit patterns).
    Weights: fp32 [n, k] normal with mean 0 and standard deviation ``w_std``.
    Returns (x_bf16_bits uint16 [m, k], W fp32 [n, k]).
    """
    rng = _rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    mask = rng.random((m, k)) < outlier_p
    x[mask] *= np.float32(outlier_mul)
    xb = fp32_to_bf16_bits(x)
    w = np.empty((n, k), dtype=np.float32)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        w[r0:r1] = rng.normal(0.0, w_std, size=(r1 - r0, k)).astype(np.float32)
    return xb, w


# Seeds of the named workloads.
SEED_SMALL = 1                      # N = K = 2560
SWEEP_SEEDS = list(range(11, 19))   # one per sweep shape, in order
LARGE_SEEDS = [21, 22]
SHARD_SEEDS = [51, 52]
LINEAR_SEEDS = {1: 31, 128: 32}
GEMM_SEEDS = {  # shape-major, then M
    (GEMM_SHAPES[0], 8): 41, (GEMM_SHAPES[0], 128): 42, (GEMM_SHAPES[0], 512): 43,
    (GEMM_SHAPES[1], 8): 44, (GEMM_SHAPES[1], 128): 45, (GEMM_SHAPES[1], 512): 46,
}
