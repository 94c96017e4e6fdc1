"""Helpers for the GPU parity tests: device inputs, host copies, tolerance checks.

The checks compare the HIP path with the CPU oracle on identical inputs (the
GPU's own input buffers copied to the host). Tolerances:
  * reduce: bit-exact against the ascending-rank fp32 order; within
    1e-6 * (sum_r |c_r|) / N of the exactly rounded mean;
  * AdamW: |d| <= 1e-6 * scale with the scales of oracle.adamw.error_scales
    (plain relative error wherever no cancellation occurs);
  * bf16 cast: bit-exact against round-to-nearest-even of the GPU's own fp32
    result, and within 1 bf16 ulp of the oracle's.
"""
import numpy as np
import torch

from oracle import adamw as oadamw
from oracle import bf16 as obf16
from oracle import reduce as oreduce
from synth import gen

REL = 1e-6
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def hparams(**kw):
    d = dict(HP)
    d.update(kw)
    return d


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: bf16 as uint16 patterns, fp32/fp64 as is."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def device_rows(seed: int, world: int, n: int, dtype: str, device="cuda"):
    """`world` separately allocated contribution buffers ~ N(0, 1e-6)."""
    g = gen.device_generator(seed, device)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [gen.device_normal(g, n, gen.GRAD_SIGMA, tdt, device) for _ in range(world)]


def device_state(seed: int, n: int, device="cuda", moments=True):
    g = gen.device_generator(seed, device)
    th = gen.device_normal(g, n, gen.THETA_SIGMA, None, device)
    if not moments:
        z = torch.zeros(n, device=device)
        return th, z, z.clone()
    m = gen.device_normal(g, n, 1e-4, None, device)
    v = gen.device_normal(g, n, 1e-6, None, device).abs_()
    return th, m, v


def check_mean(g_gpu: np.ndarray, rows_host: np.ndarray):
    seq = oreduce.mean_seq32(rows_host)
    assert np.array_equal(bits32(g_gpu), bits32(seq)), "reduce differs from the ascending-rank fp32 sum"
    ex = oreduce.mean_exact(rows_host).astype(np.float64)
    scale = oreduce.abs_mean(rows_host)
    err = np.abs(g_gpu.astype(np.float64) - ex)
    assert np.all(err <= REL * scale), f"max scaled err {np.max(err / np.maximum(scale, 1e-300))}"


def check_adamw(after, before, g, step, hp):
    """after/before: (theta, m, v) host fp32 arrays; g: host fp32 gradient used.
    Returns (oracle theta', theta' tolerance)."""
    hpo = oadamw.HParams(**hp)
    th1, m1, v1 = oadamw.adamw_step(before[0], before[1], before[2], g, step, hpo)
    st, sm, sv = oadamw.error_scales(before[0], before[1], g, step, hpo, m1, v1)
    for name, got, want, sc in (("theta", after[0], th1, st), ("m", after[1], m1, sm), ("v", after[2], v1, sv)):
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        bad = ~(err <= REL * sc)
        assert not bad.any(), f"{name}: {bad.sum()} elements off, max scaled {np.max(err / np.maximum(sc, 1e-300))}"
    return th1, REL * st


def check_bf16(b_gpu: np.ndarray, theta_gpu: np.ndarray, oracle):
    """Bit-exact RNE of the GPU's own theta', and within 1 bf16 ulp (plus the
    fp32 tolerance the cast input already carries) of the oracle's theta'."""
    theta_or, tol = oracle
    assert np.array_equal(b_gpu, obf16.to_bf16_bits(theta_gpu)), "bf16 cast is not RNE of the GPU's theta"
    d = np.abs(obf16.from_bf16_bits(b_gpu).astype(np.float64) - theta_or.astype(np.float64))
    assert np.all(d <= obf16.ulp(theta_or) + tol), "bf16 result more than 1 ulp from the oracle"


def max_scaled_adamw_error(after, before, g, step, hp):
    hpo = oadamw.HParams(**hp)
    th1, m1, v1 = oadamw.adamw_step(before[0], before[1], before[2], g, step, hpo)
    st, _, _ = oadamw.error_scales(before[0], before[1], g, step, hpo, m1, v1)
    return float(np.max(np.abs(after[0].astype(np.float64) - th1) / st))


GUARD_LENGTHS = [1, 7, 8, 15, 16, 23, 24, 25, 31, 32, 33, 40, 47, 63, 64, 100, 255, 256, 257, 1000,
                 2047, 8191, 8192, 8193, 20000, 70001]


def guarded_views(lengths, seed):
    """Destinations as views of one NaN-filled bf16 buffer, each starting at a
    different offset from the 16-byte grid, with guard gaps between them."""
    rng = np.random.default_rng(seed)
    starts, pos = [], 0
    for n in lengths:
        pos += 24 + int(rng.integers(0, 8))
        starts.append(pos)
        pos += n
    big = torch.full((pos + 24,), float("nan"), device="cuda", dtype=torch.bfloat16)
    views = [big[a:a + n] for a, n in zip(starts, lengths)]
    return big, views, starts


def check_guards(big, starts, lengths):
    """Every element of the buffer outside the views still holds the NaN fill."""
    mask = np.ones(big.numel(), dtype=bool)
    for a, n in zip(starts, lengths):
        mask[a:a + n] = False
    guard = host(big)[mask]
    nan_bits = np.uint16(torch.tensor(float("nan"), dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF)
    assert np.all(guard == nan_bits)
