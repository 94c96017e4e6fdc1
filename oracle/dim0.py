"""Per-parameter dim-0 sharding (FSDP2) and its unshard copy-out (oracle; test
infrastructure only).

What the pages fix:
  * [L5] s7.2 point 1 and Fig. 5-5: FSDP2 keeps every parameter whole in shape
    and shards each one on its first dimension (DTensor Shard(0)); a rank's
    local shard of an [H, D] weight is [H/N, D].
  * [FZ3] s4 (FSDP1 vs FSDP2 table): each parameter is represented as a DTensor
    split along dim 0 over the DP mesh; unshard materialises the full local
    tensor from the gathered pieces, and the all-gather is a batched
    foreach_all_gather of many parameters.
  * [FZ3] s1 and s3: the all-gather result is copied out before compute.

Readings where the pages are silent:
  * when dim 0 does not divide by N, rank r holds rows [r*c, min((r+1)*c, d0))
    with c = ceil(d0/N) rows per rank, zero-padded to c rows (ranks past the
    end hold only padding) -- torch.chunk's split, padded to the first chunk;
  * a rank's shard of a unit is the concatenation of its padded per-parameter
    chunks in registration order (the all-gather input); the all-gather output
    holds the N ranks' shards one after the other;
  * a 0-d parameter is one row of one element.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dim0Layout:
    rows: tuple        # d0 of each parameter
    rowsize: tuple     # elements per dim-0 row
    chunk: tuple       # elements per rank of each parameter: ceil(d0/N) * rowsize
    local_offsets: tuple  # offset of each parameter's chunk inside a rank's shard
    local_total: int   # L: elements of one rank's shard
    world: int


def dim0_layout(shapes, world: int) -> Dim0Layout:
    if world < 1:
        raise ValueError("world size must be >= 1")
    rows, rs, chunk, loff = [], [], [], []
    t = 0
    for shp in shapes:
        shp = tuple(int(x) for x in shp)
        if any(x < 0 for x in shp):
            raise ValueError("dimensions must be non-negative")
        d0 = shp[0] if len(shp) else 1
        r = int(np.prod(shp[1:])) if len(shp) > 1 else 1
        c = -(-d0 // world) * r
        rows.append(d0)
        rs.append(r)
        chunk.append(c)
        loff.append(t)
        t += c
    return Dim0Layout(tuple(rows), tuple(rs), tuple(chunk), tuple(loff), t, world)


def valid(numel: int, chunk: int, rank: int) -> int:
    """Elements of a parameter's chunk on `rank` that are real (the rest is pad)."""
    return max(0, min(chunk, numel - rank * chunk))


def shard_dim0(params, world: int, rank: int, dtype=np.float32) -> np.ndarray:
    """Rank r's shard of the unit: its padded dim-0 chunk of every parameter, concatenated."""
    lay = dim0_layout([np.shape(p) for p in params], world)
    out = np.zeros(lay.local_total, dtype=dtype)
    for p, c, lo in zip(params, lay.chunk, lay.local_offsets):
        flat = np.asarray(p).ravel(order="C")
        v = valid(flat.size, c, rank)
        out[lo:lo + v] = flat[rank * c:rank * c + v]
    return out


def copy_out_dim0(gathered: np.ndarray, shapes, world: int):
    """Full parameters from the rank-major all-gather output; padding rows dropped."""
    lay = dim0_layout(shapes, world)
    if gathered.size < world * lay.local_total:
        raise ValueError("gathered buffer is shorter than N shards")
    outs = []
    for shp, c, lo in zip(shapes, lay.chunk, lay.local_offsets):
        n = int(np.prod(shp)) if len(shp) else 1
        flat = np.empty(n, dtype=gathered.dtype)
        for r in range(world):
            v = valid(n, c, r)
            base = r * lay.local_total + lo
            flat[r * c:r * c + v] = gathered[base:base + v]
        outs.append(flat.reshape(shp))
    return outs
