"""Seeded synthetic inputs shared by the CPU oracle, the tests and the benchmark.

This module only draws random numbers and lays them out in memory; it holds
none of the method's arithmetic (no rounding to 16-bit formats, no products).
Both sides of every parity check receive the same fp32 arrays from here and
each applies its own quantisation.

Seeds: workload ``k`` draws operand ``i`` from ``numpy.random.default_rng``
(PCG64) seeded with ``1000*k + i``; operand indices are A=1, B=2 (GEMMs),
Q=1, K=2, V=3 (attention); the outlier positions of operand i use
operand index 90 + i (91 for A, 92 for B).

Distributions follow the workloads the pages describe:
  * uniform[-1, 1] operands for the small single GEMM and the block-repeat
    spike (Warp issue #1965, "Spike" section);
  * normal(0, 1) operands for the dense 4096^3 GEMM, padded leading dimension
    filled with NaN so that any read of the padding poisons the result
    (tensor-core layout explainer, paragraph on leading dimensions);
  * normal(0, 1) with 1% of entries multiplied by 1e4 for the split-precision
    GEMM, to stress cancellation;
  * normal(0, sigma=1/sqrt(128)) for the attention-shaped pair (Strata PR #800,
    2,048 queries, 32,768 keys, head dim 128).
"""
from __future__ import annotations

import numpy as np

A_OP, B_OP, Q_OP, K_OP, V_OP, OUTLIER_OP = 1, 2, 1, 2, 3, 9


def seed_for(workload: int, operand: int) -> int:
    return 1000 * int(workload) + int(operand)


def rng(workload: int, operand: int) -> np.random.Generator:
    return np.random.default_rng(seed_for(workload, operand))


def uniform(shape, workload: int, operand: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """fp32 uniform[lo, hi) array."""
    return rng(workload, operand).uniform(lo, hi, size=shape).astype(np.float32)


def normal(shape, workload: int, operand: int, sigma: float = 1.0) -> np.ndarray:
    """fp32 normal(0, sigma) array; ``sigma`` is the standard deviation."""
    return (rng(workload, operand).standard_normal(size=shape) * sigma).astype(np.float32)


def with_outliers(x: np.ndarray, workload: int, operand: int, frac: float = 0.01,
                  scale: float = 1e4) -> np.ndarray:
    """Copy of ``x`` with exactly round(frac * x.size) positions, drawn uniformly
    without replacement, multiplied by ``scale`` in fp32."""
    out = np.array(x, dtype=np.float32, copy=True)
    n = int(round(frac * out.size))
    if n:
        pos = rng(workload, OUTLIER_OP * 10 + operand).choice(out.size, size=n, replace=False)
        flat = out.reshape(-1)
        flat[pos] = flat[pos] * np.float32(scale)
    return out


def pad_columns(x: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Embed a 2-D array of shape (rows, cols) in storage of shape (rows, ld),
    filling columns cols..ld-1 with ``fill`` (NaN by default)."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    out = np.full((rows, ld), fill, dtype=np.float32)
    out[:, :cols] = x
    return out


def asymmetric_ints(shape, workload: int, operand: int, lo: int, hi: int) -> np.ndarray:
    """fp32 array of distinct integers drawn from [lo, hi] without repetition
    (zero excluded), so that a transposed or half-swapped layout cannot match
    by coincidence."""
    n = int(np.prod(shape))
    pool = np.array([v for v in range(lo, hi + 1) if v != 0], dtype=np.int64)
    if n > pool.size:
        raise ValueError("not enough distinct integers in range")
    vals = rng(workload, operand).choice(pool, size=n, replace=False)
    return vals.astype(np.float32).reshape(shape)


# ---- the five workloads -------------------------------------------------------

def gemm_small(m: int = 256, n: int = 256, k: int = 256):
    """Single fp16 GEMM: A (m x k) row-major, B stored column-major as Bt (n x k);
    uniform[-1, 1] fp32 before rounding."""
    a = uniform((m, k), 1, A_OP)
    bt = uniform((n, k), 1, B_OP)
    return a, bt


def block_repeat(tm: int = 64, tn: int = 64, tk: int = 64, m: int = 2048, n: int = 2048):
    """Block-repeat spike: A (m x tk) row-major, B stored column-major as Bt (n x tk)."""
    a = uniform((m, tk), 2, A_OP)
    bt = uniform((n, tk), 2, B_OP)
    return a, bt


def gemm_dense(m: int = 4096, n: int = 4096, k: int = 4096, pad: int = 64):
    """Dense GEMM: A row-major (m x k) in storage (m, k+pad); B column-major,
    stored as Bt (n x k) in storage (n, k+pad); normal(0, 1); NaN padding."""
    a = pad_columns(normal((m, k), 3, A_OP), k + pad)
    bt = pad_columns(normal((n, k), 3, B_OP), k + pad)
    return a, bt


def gemm_split(m: int = 4096, n: int = 4096, k: int = 4096):
    """Split-precision GEMM: fp32 normal(0, 1) with 1% outliers x1e4; A row-major
    (m x k), B column-major stored as Bt (n x k)."""
    a = with_outliers(normal((m, k), 4, A_OP), 4, A_OP)
    bt = with_outliers(normal((n, k), 4, B_OP), 4, B_OP)
    return a, bt


def attention(nq: int = 2048, nk: int = 32768, d: int = 128):
    """Attention-shaped pair: Q (nq x d), K (nk x d), V (nk x d), all row-major,
    fp32 normal(0, 1/sqrt(128))."""
    s = 1.0 / np.sqrt(128.0)
    return normal((nq, d), 5, Q_OP, s), normal((nk, d), 5, K_OP, s), normal((nk, d), 5, V_OP, s)
