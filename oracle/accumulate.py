"""Gradient accumulation over micro-batches and global-norm clipping (oracle;
test infrastructure only).

What the pages fix:
  * [L5] s3 (key conclusion under ZeRO-1/2): with gradient accumulation ZeRO-1
    sums each rank's full local gradient over the micro-batches and
    reduce-scatters once after the last one, while ZeRO-2 keeps no full
    gradient and reduce-scatters every micro-batch, accumulating its own 1/N.
  * [L5] s2 (note under the equations): the fp32 accumulation buffer costs 4P
    per rank for ZeRO-0/1 (it is the full gradient) and 4P/N for ZeRO-2/3.
  * [DPZ] s6 (global operations must know about shards): a global
    gradient-norm clip needs a reduction across shards; each rank's local
    gradient yields only a partial.

Readings where the pages are silent:
  * the accumulated gradient is the mean over the K micro-batches (each
    micro-batch's loss is a mean), applied as a factor `scale` = 1/K;
  * ZeRO-2 order: per micro-batch, mean over ranks (ascending-rank fp32 sum,
    one division by N), then times scale, then added to the fp32 accumulator
    (the first micro-batch initialises it);
  * ZeRO-1 order: each rank adds its micro-batch gradients into an fp32
    buffer in micro-batch order, then the buffers are reduced (ascending-rank
    sum, division by N) and multiplied by scale;
  * clipping follows the common definition (PyTorch's clip_grad_norm_):
    norm = sqrt(sum of squares over all shards), coefficient =
    max_norm / (norm + 1e-6), capped at 1 (a NaN norm gives a NaN
    coefficient), and the gradient is multiplied by it before AdamW.
"""
from __future__ import annotations

import math

import numpy as np

from . import reduce

CLIP_EPS = 1e-6


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _scaled(u, scale):
    """Multiply by scale in fp32; a scale of exactly 1 leaves the values untouched."""
    s = np.float32(scale)
    return u if s == np.float32(1.0) else (u * s).astype(np.float32)


def zero2_accumulate(rows_per_microbatch, scale=1.0) -> np.ndarray:
    """Sharded accumulation: reduce each micro-batch, then add into the fp32 shard."""
    acc = None
    for rows in rows_per_microbatch:
        u = _scaled(reduce.mean_seq32(rows), scale)
        acc = u.copy() if acc is None else (acc + u).astype(np.float32)
    return acc


def zero1_accumulate(rows_per_microbatch, scale=1.0) -> np.ndarray:
    """Unsharded accumulation: each rank sums its local gradients in fp32, then one reduce."""
    local = None
    for rows in rows_per_microbatch:
        c = reduce.decode_rows(rows)
        local = c.copy() if local is None else (local + c).astype(np.float32)
    return _scaled(reduce.mean_seq32(_f32(local)), scale)


def exact_mean_over_microbatches(rows_per_microbatch) -> np.ndarray:
    """fp64 sum of every contribution of every micro-batch over N*K, rounded once."""
    tot = None
    count = 0
    for rows in rows_per_microbatch:
        c = reduce.decode_rows(rows).astype(np.float64)
        s = c.sum(axis=0)
        tot = s if tot is None else tot + s
        count += c.shape[0]
    return (tot / count).astype(np.float32)


def global_norm(partials) -> float:
    """sqrt of the sum of per-shard sums of squares, added in the order given (fp64)."""
    total = 0.0
    for p in partials:
        total += float(p)
    return math.sqrt(total)


def clip_coefficient(partials, max_norm: float):
    """(coefficient as fp32, norm in fp64) from the shards' sums of squares."""
    norm = global_norm(partials)
    c = max_norm / (norm + CLIP_EPS)
    if c > 1.0:
        c = 1.0
    return np.float32(c), norm
