"""Per-rank model-state memory and per-step communication (oracle; test infrastructure only).

Exact rational arithmetic (fractions.Fraction); decimal GB (10^9 bytes).

What the pages fix:
  * [L5] s2 (equations for M0..M3) and [DPZ] s3.2-3.3: with bf16 parameters
    (2 B), bf16 gradients (2 B) and an fp32 optimizer state of k = 12 B
    (master, m, v), per-rank state is
        stage 0 (DDP):  2P + 2P + kP
        stage 1:        2P + 2P + kP/N
        stage 2:        2P + (2P + kP)/N
        stage 3:        (2P + 2P + kP)/N
    [ZvF] s2 states the same in GB for an "N B" model.
  * [L5] s2 (note under the equations): accumulating gradients in fp32 adds 4P
    to stages 0-1 (the gradient is held whole) and 4P/N to stages 2-3.
  * [L5] s3 and [DPZ] s3.4: per-step communication is 2P elements for DDP and
    ZeRO-1/2 (a reduce-scatter plus an all-gather, or one all-reduce) and 3P
    for ZeRO-3 (one more all-gather); each ring phase moves (N-1)/N of the
    buffer per rank.
  * The calculator exercise of [L5] raises ValueError for non-positive sizes
    or a stage outside 0..3; the same convention is kept.

Display: the pages print these with Python float formatting, i.e. the binary
value rounded half-to-even at the shown digit; `fmt` reproduces that.
"""
from __future__ import annotations

from fractions import Fraction

GB = 10 ** 9

# (replicated bytes, sharded bytes) per parameter for k = 12 -- the split used
# by the ledger script of [DPZ] s4.1.
SPLIT = {0: (16, 0), 1: (4, 12), 2: (2, 14), 3: (0, 16)}
NAMES = {0: "DDP", 1: "ZeRO-1", 2: "ZeRO-2", 3: "ZeRO-3"}


def _check(params, world, stage):
    if params <= 0 or world <= 0:
        raise ValueError("parameter count and world size must be positive")
    if stage not in (0, 1, 2, 3):
        raise ValueError("stage must be one of 0, 1, 2, 3")


def state_bytes(params, world: int, stage: int, k=12, fp32_grad_accum: bool = False) -> Fraction:
    """Per-rank model-state bytes (params, grads, optimizer state [+ fp32 accumulation])."""
    _check(params, world, stage)
    p = Fraction(params)
    n = Fraction(world)
    par, grad, opt = 2 * p, 2 * p, Fraction(k) * p
    extra = Fraction(0)
    if fp32_grad_accum:
        extra = 4 * p if stage <= 1 else 4 * p / n
    if stage == 0:
        base = par + grad + opt
    elif stage == 1:
        base = par + grad + opt / n
    elif stage == 2:
        base = par + (grad + opt) / n
    else:
        base = (par + grad + opt) / n
    return base + extra


def bytes_per_param(world: int, stage: int) -> Fraction:
    """Replicated + sharded/N bytes per parameter (k = 12)."""
    _check(1, world, stage)
    rep, sh = SPLIT[stage]
    return Fraction(rep) + Fraction(sh, world)


def saving_vs_ddp(world: int, stage: int) -> Fraction:
    return bytes_per_param(world, 0) / bytes_per_param(world, stage)


def comm_elements(params, stage: int) -> Fraction:
    """Elements moved per rank per step in the ideal bandwidth model."""
    _check(params, 1, stage)
    p = Fraction(params)
    return 3 * p if stage == 3 else 2 * p


def comm_bytes(params, stage: int, elem_bytes: int = 2) -> Fraction:
    return comm_elements(params, stage) * elem_bytes


def ring_phase(buffer_size, world: int) -> Fraction:
    """Per-rank volume of one reduce-scatter or all-gather phase of a ring."""
    if world <= 0:
        raise ValueError("world size must be positive")
    return Fraction(world - 1, world) * Fraction(buffer_size)


def to_gb(nbytes) -> Fraction:
    return Fraction(nbytes) / GB


def fmt(x, digits: int) -> str:
    """Python's fixed-point formatting of the binary float nearest to x."""
    return format(float(x), f".{digits}f")
