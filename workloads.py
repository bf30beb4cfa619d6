"""Seeded synthetic inputs for the binary XNOR-popcount path.

This module is shared by both sides of every parity check (the HIP path and the
CPU oracle) and by the benchmark.  It holds random draws, shapes and the
workload descriptions only: no step of the binary method's arithmetic (sign,
packing, popcount, scaling, thresholds) lives here.

Seeds follow ``seed = 1000 * workload + tensor_index``; every draw uses numpy's
PCG64 ``default_rng``.  fp32 normals come from ``standard_normal(dtype=float32)``
and U(0,1) from ``random(dtype=float32)``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "normal_f32", "uniform01_f32", "random_words", "bn_params", "edge_values", "inject_edge_values",
    "WORKLOADS", "seed_for",
]


def seed_for(workload: int, tensor_index: int) -> int:
    return 1000 * workload + tensor_index


def normal_f32(seed: int, shape) -> np.ndarray:
    """fp32 samples of N(0, 1)."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def uniform01_f32(seed: int, shape) -> np.ndarray:
    """fp32 samples of U(0, 1)."""
    return np.random.default_rng(seed).random(shape, dtype=np.float32)


def random_words(seed: int, shape) -> np.ndarray:
    """Uniformly random 32-bit words (uint32): packed operands with every bit
    pattern, for cases where the bits themselves are the input."""
    return np.random.default_rng(seed).integers(0, 2**32, size=shape, dtype=np.uint32)


def bn_params(seed: int, n: int):
    """BatchNorm parameters of one binary hidden layer.

    gamma ~ U(0.5, 1.5) and beta ~ N(0, 0.1) (0.1 read as the standard
    deviation); running mean 0, running variance 1 and eps 1e-5 are the usual
    initial statistics, since the workload states none.
    """
    g = np.random.default_rng(seed)
    gamma = g.uniform(0.5, 1.5, n).astype(np.float32)
    beta = g.normal(0.0, 0.1, n).astype(np.float32)
    mean = np.zeros(n, dtype=np.float32)
    var = np.ones(n, dtype=np.float32)
    eps = np.float32(1e-5)
    return gamma, beta, mean, var, eps


def edge_values() -> np.ndarray:
    """IEEE-754 single values at which a sign test is easy to get wrong."""
    bits = np.array([
        0x00000000,  # +0.0
        0x80000000,  # -0.0
        0x7FC00000,  # quiet NaN
        0xFFC00000,  # negative quiet NaN
        0x7F800001,  # signalling NaN payload
        0x7F800000,  # +inf
        0xFF800000,  # -inf
        0x00000001,  # smallest positive denormal
        0x80000001,  # smallest negative denormal
        0x007FFFFF,  # largest positive denormal
        0x807FFFFF,  # largest negative denormal
        0x00800000,  # FLT_MIN
        0x80800000,  # -FLT_MIN
        0x7F7FFFFF,  # FLT_MAX
        0xFF7FFFFF,  # -FLT_MAX
        0x3F800000,  # 1.0
        0xBF800000,  # -1.0
    ], dtype=np.uint32)
    return bits.view(np.float32)


def inject_edge_values(x: np.ndarray, seed: int, fraction: float = 0.01,
                       finite_only: bool = False) -> np.ndarray:
    """Return a copy of ``x`` with a seeded fraction of entries replaced by
    values from :func:`edge_values` (finite ones only if asked)."""
    vals = edge_values()
    if finite_only:
        vals = vals[np.isfinite(vals)]
    g = np.random.default_rng(seed)
    y = np.array(x, dtype=np.float32, copy=True)
    flat = y.reshape(-1)
    n = max(1, int(flat.size * fraction))
    idx = g.choice(flat.size, size=min(n, flat.size), replace=False)
    flat[idx] = vals[g.integers(0, vals.size, size=idx.size)]
    return y


# The five workloads, with the shapes the timing and the parity tests use.
WORKLOADS = {
    1: dict(name="single binary linear layer", M=64, N=256, K=1000),
    2: dict(name="binary MLP batch 1024", batch=1024, d_in=784, hidden=4096,
            n_hidden=3, d_out=10),
    3: dict(name="batch-1 binary GEMV",
            shapes=[dict(N=11008, K=4096), dict(N=4096, K=11008)]),
    4: dict(name="large binary GEMM",
            shapes=[dict(M=8192, N=8192, K=8192), dict(M=16384, N=16384, K=16384)]),
    5: dict(name="binary 3x3 conv block (im2col XNOR GEMM + fp32 residual)",
            shapes=[dict(B=256, H=56, W=56, C=64, Cout=64),
                    dict(B=256, H=14, W=14, C=256, Cout=256)]),
}
