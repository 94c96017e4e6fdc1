"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and nothing else: it contains none of the
update's arithmetic (no layout, reduction, optimizer or rounding rule of the
method). Where an input must be bf16, the draw is converted by PyTorch's own
dtype conversion, a library routine that neither the oracle nor the HIP
library uses.

Recipe (stated once, used everywhere):
  * master theta ~ N(0, 0.02^2) in fp32,
  * each simulated rank's gradient contribution ~ N(0, (1e-3)^2), drawn in fp32
    and converted to bf16 (fp32 contributions are kept as drawn),
  * m = v = 0 before the first step.
Host draws use numpy's PCG64; device draws use torch's generator on the GPU.
"""
from __future__ import annotations

import numpy as np

THETA_SIGMA = 0.02
GRAD_SIGMA = 1e-3


def host_normal(seed: int, n: int, sigma: float) -> np.ndarray:
    """fp32 array of n draws from N(0, sigma^2), PCG64-seeded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(n, dtype=np.float64) * sigma).astype(np.float32)


def host_uniform(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(lo, hi, n).astype(np.float32)


def to_bf16_bits_via_torch(x: np.ndarray) -> np.ndarray:
    """Convert fp32 values to bf16 with torch's cast; return the uint16 patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_grad_rows(seed: int, world: int, n: int, dtype: str) -> np.ndarray:
    """[world, n] gradient contributions: uint16 bf16 patterns or fp32 values."""
    rows = np.stack([host_normal(seed * 1000 + r, n, GRAD_SIGMA) for r in range(world)])
    if dtype == "bf16":
        return to_bf16_bits_via_torch(rows.reshape(-1)).reshape(world, n)
    if dtype == "f32":
        return rows
    raise ValueError(f"unknown contribution dtype {dtype!r}")


def host_params(seed: int, numels, sigma: float = THETA_SIGMA):
    """One fp32 array per parameter, each seeded from (seed, index)."""
    return [host_normal(seed * 100003 + i, n, sigma) for i, n in enumerate(numels)]


# ---- device draws (GPU side of the same recipe; used at sizes the host cannot hold) ----

def device_generator(seed: int, device="cuda"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_normal(gen, n: int, sigma: float, out_dtype=None, device="cuda"):
    """Draw n fp32 N(0, sigma^2) values on the device, optionally converted by torch."""
    import torch

    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    x.mul_(sigma)
    if out_dtype is not None and out_dtype != torch.float32:
        x = x.to(out_dtype)
    return x
