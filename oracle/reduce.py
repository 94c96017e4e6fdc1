"""Mean of the per-rank gradient contributions (oracle; test infrastructure only).

[DPZ] s3.1 (equations for L_r, g_r and g): with equal local batches, the same
starting weights and a per-sample loss, the mean over ranks of the local mean
gradients equals the full-batch mean gradient; this mean is what data
parallelism must deliver to every rank. [L5] s3 (ZeRO-1/2, step 1): a
reduce-scatter leaves each rank only its own 1/N slice of it.
[L5] s7.5 (MixedPrecisionPolicy with reduce_dtype=float32): the reduction
happens in fp32.

Two forms are given:
  * mean_exact: the sum taken in fp64 (exact for bf16 inputs whenever the
    exponent spread of one column is below ~45 bits), divided by N and rounded
    once to fp32 -- the definition.
  * mean_seq32: the fp32 arithmetic of one particular order -- a running sum
    over ranks in ascending order, started from rank 0's value, then one fp32
    division by N. The pages leave the order open (reading: this one); any
    other order is also a correct reduction within the stated bound.
"""
from __future__ import annotations

import numpy as np


def decode_rows(rows: np.ndarray) -> np.ndarray:
    """[N, n] contributions as fp32: uint16 rows are bf16 patterns (exact decode)."""
    rows = np.asarray(rows)
    if rows.ndim != 2:
        raise ValueError("rows must be [N, n]")
    if rows.dtype == np.uint16:
        return (rows.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if rows.dtype == np.float32:
        return rows
    raise ValueError("rows must be uint16 (bf16 patterns) or float32")


def mean_exact(rows) -> np.ndarray:
    c = decode_rows(rows).astype(np.float64)
    n = c.shape[0]
    if n < 1:
        raise ValueError("need at least one contribution")
    return (c.sum(axis=0) / n).astype(np.float32)


def mean_seq32(rows) -> np.ndarray:
    c = decode_rows(rows)
    n = c.shape[0]
    if n < 1:
        raise ValueError("need at least one contribution")
    s = c[0].copy()
    for r in range(1, n):
        s = (s + c[r]).astype(np.float32)
    return (s / np.float32(n)).astype(np.float32)


def abs_mean(rows) -> np.ndarray:
    """(sum_r |c_r|) / N in fp64: the scale of the reduction's rounding error."""
    c = decode_rows(rows).astype(np.float64)
    return np.abs(c).sum(axis=0) / c.shape[0]


def sumsq(g) -> float:
    """Sum of squares of the reduced shard, in fp64 ([DPZ] s6: a global
    gradient norm needs the partial of every shard; this is one shard's)."""
    g64 = np.asarray(g, dtype=np.float64)
    return float(np.dot(g64, g64))
