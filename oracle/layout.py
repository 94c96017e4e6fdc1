"""FlatParameter layout: flatten, pad, shard, pack and copy-out (oracle; test infrastructure only).

What the pages fix:
  * [L5] s7.1 point 1 and [ZvF] s3 (difference 1): all parameters of one wrapped
    unit are laid end to end in a single 1-D tensor, and that tensor is split
    along the data-parallel dimension.
  * [L5] s7.1 point 3: when the element count does not divide by the world size,
    the FlatParameter is padded at its end.
  * [LAF] s5.1 (flatten illustration) and the shard routine of [DPZ] s4.2: the
    split is even and contiguous, rank r holding the r-th chunk.
  * [L5] s7.1 point 1 (views assigned to each submodule's parameter) and
    [FZ3] s1/s3 (copy-out after the all-gather): unsharding hands each parameter
    its own slice of the gathered flat buffer.

Readings where the pages are silent:
  * order of parameters: registration order, each tensor in C (row-major) order;
  * no alignment padding between parameters, only the tail pad;
  * pad value +0.0;
  * the rank shard of an empty unit is empty.

Beyond the pages: `align` (default 1, the pages' layout) rounds the per-rank
slice S up to a multiple of `align` elements. The extra padding also sits at
the tail of the unit, so parameter offsets and every real element's value
are unchanged; only S, P and the rank boundaries r*S move.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Layout:
    offsets: tuple  # offset of parameter i inside the flat buffer
    total: int      # T = sum of element counts
    padded: int     # P = S * N
    shard: int      # S = ceil(T / N) rounded up to a multiple of align
    pad: int        # P - T, always in [0, N * align)
    world: int


def flat_layout(numels, world: int, align: int = 1) -> Layout:
    """Offsets are the exclusive prefix sum of element counts in list order."""
    if world < 1:
        raise ValueError("world size must be >= 1")
    if align < 1:
        raise ValueError("align must be >= 1")
    offsets = []
    t = 0
    for n in numels:
        n = int(n)
        if n < 0:
            raise ValueError("element counts must be non-negative")
        offsets.append(t)
        t += n
    s = -(-t // world)  # ceil(T / N)
    s = -(-s // align) * align  # up to a multiple of align
    p = s * world
    return Layout(tuple(offsets), t, p, s, p - t, world)


def flatten(params, world: int, dtype=None, align: int = 1) -> np.ndarray:
    """Concatenate C-order ravels of `params` and append zero padding up to P."""
    lay = flat_layout([np.asarray(p).size for p in params], world, align)
    if dtype is None:
        dtype = np.asarray(params[0]).dtype if params else np.float32
    flat = np.zeros(lay.padded, dtype=dtype)
    for off, p in zip(lay.offsets, params):
        a = np.asarray(p).ravel(order="C")
        flat[off:off + a.size] = a
    return flat


def shard_of(flat: np.ndarray, world: int, rank: int) -> np.ndarray:
    """Rank r's contiguous chunk [r*S, (r+1)*S) of a padded flat buffer."""
    if not 0 <= rank < world:
        raise ValueError("rank must lie in [0, world)")
    if flat.size % world:
        raise ValueError("flat buffer is not padded to a multiple of the world size")
    s = flat.size // world
    return flat[rank * s:(rank + 1) * s]


def pack_shard(params, world: int, rank: int, align: int = 1):
    """The rank's fp32 master shard plus zeroed Adam moments.

    Parameters may be fp32 arrays or bf16 patterns given as uint16 arrays; the
    latter are decoded exactly (the bf16 bits are the top half of an fp32).
    """
    decoded = []
    for p in params:
        a = np.asarray(p)
        if a.dtype == np.uint16:
            a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        decoded.append(a.astype(np.float32, copy=False))
    flat = flatten(decoded, world, dtype=np.float32, align=align)
    master = shard_of(flat, world, rank).copy()
    return master, np.zeros_like(master), np.zeros_like(master)


def copy_out(gathered: np.ndarray, shapes):
    """Per-parameter tensors cut from a gathered flat buffer; the tail pad is dropped."""
    sizes = [int(np.prod(s)) if len(s) else 1 for s in shapes]
    lay = flat_layout(sizes, 1)
    if gathered.size < lay.total:
        raise ValueError("gathered buffer is shorter than the unit")
    return [gathered[off:off + n].reshape(shape).copy()
            for off, n, shape in zip(lay.offsets, sizes, shapes)]


def flat_window(fetch, numels, f0: int, f1: int, dtype=np.float32) -> np.ndarray:
    """flat[f0:f1] of the padded FlatParameter without materialising the whole unit.

    `fetch(i, j0, j1)` returns elements [j0, j1) of parameter i (C order). Each
    position f is parameter i's element f - off_i for the i whose range holds
    it, and +0 past the last parameter (the tail pad).
    """
    lay = flat_layout(numels, 1)
    out = np.zeros(max(f1 - f0, 0), dtype=dtype)
    for i, (off, n) in enumerate(zip(lay.offsets, numels)):
        a, b = max(f0, off), min(f1, off + int(n))
        if a < b:
            out[a - f0:b - f0] = fetch(i, a - off, b - off)
    return out
