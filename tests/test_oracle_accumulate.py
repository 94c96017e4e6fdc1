"""Pins of the oracle's micro-batch accumulation and global-norm clipping."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import accumulate, bf16, reduce
from synth import gen


def _dyadic_microbatches(world, k, b, d, seed):
    # per-sample linear loss l_i(w) = a_i . w: gradient a_i; small dyadic values
    # keep every sum exact in fp32
    rng = np.random.default_rng(seed)
    a = rng.integers(-64, 64, size=(k, world, b, d)) / 256.0
    local = a.mean(axis=2).astype(np.float32)  # [k, world, d]: each rank's micro-batch mean
    return a, [local[j] for j in range(k)]


def test_zero1_and_zero2_orders_equal_the_full_batch_gradient():
    # Lesson 5 s3: ZeRO-1 accumulates full local gradients and reduces once, ZeRO-2
    # reduces every micro-batch; with equal micro-batches both give the mean
    # gradient of all N*K*b samples (DP-and-ZeRO page s3.1 applied twice).
    world, k, b, d = 4, 4, 2, 64
    a, mbs = _dyadic_microbatches(world, k, b, d, 0)
    full = a.reshape(-1, d).mean(axis=0)
    z1 = accumulate.zero1_accumulate(mbs, scale=1.0 / k)
    z2 = accumulate.zero2_accumulate(mbs, scale=1.0 / k)
    assert np.array_equal(z1.astype(np.float64), full)
    assert np.array_equal(z2.astype(np.float64), full)
    assert np.array_equal(accumulate.exact_mean_over_microbatches(mbs).astype(np.float64), full)
    # bf16-exact inputs give the same
    mbs16 = [bf16.to_bf16_bits(m) for m in mbs]
    assert np.array_equal(accumulate.zero2_accumulate(mbs16, 1.0 / k).astype(np.float64), full)


def test_single_microbatch_is_the_plain_reduce():
    rows = gen.host_grad_rows(3, 8, 1001, "bf16")
    assert np.array_equal(accumulate.zero2_accumulate([rows]), reduce.mean_seq32(rows))
    assert np.array_equal(accumulate.zero1_accumulate([rows]), reduce.mean_seq32(rows))


def test_exact_mean_over_microbatches_is_rounded_once():
    mbs = [gen.host_grad_rows(10 + j, 3, 17, "f32") for j in range(3)]
    got = accumulate.exact_mean_over_microbatches(mbs)
    for i in range(17):
        q = sum(Fraction(float(m[r, i])) for m in mbs for r in range(3)) / 9
        err = abs(Fraction(float(got[i])) - q)
        assert err <= abs(q) * Fraction(1, 2 ** 23)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_both_orders_within_the_summation_bound(dtype):
    world, k = 8, 5
    mbs = [gen.host_grad_rows(20 + j, world, 4001, dtype) for j in range(k)]
    exact = np.stack([reduce.decode_rows(m).astype(np.float64) for m in mbs]).sum(axis=(0, 1)) / (world * k)
    absum = np.stack([np.abs(reduce.decode_rows(m).astype(np.float64)) for m in mbs]).sum(axis=(0, 1)) / (world * k)
    u = 2.0 ** -24
    for got in (accumulate.zero1_accumulate(mbs, 1.0 / k), accumulate.zero2_accumulate(mbs, 1.0 / k)):
        bound = (world + k + 2) * u * absum + u * np.abs(exact)
        assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)


def test_clip_matches_torch_clip_grad_norm():
    # the global norm assembled from per-shard partials equals the norm of the
    # whole gradient, and the clipped gradient equals torch's clip_grad_norm_
    world = 4
    g = gen.host_normal(5, 4000, 1e-3).astype(np.float64)
    shards = np.array_split(g, world)
    partials = [reduce.sumsq(s) for s in shards]
    for max_norm in (1e-3, 0.01, 1.0):
        coef, norm = accumulate.clip_coefficient(partials, max_norm)
        p = torch.nn.Parameter(torch.zeros(g.size, dtype=torch.float64))
        p.grad = torch.from_numpy(g.copy())
        total = torch.nn.utils.clip_grad_norm_([p], max_norm, foreach=False)
        assert abs(norm - float(total)) <= 1e-13 * float(total)
        want = p.grad.numpy()
        assert np.allclose(g * float(coef), want, rtol=1e-7, atol=0)  # coef is rounded to fp32
        assert (float(coef) == 1.0) == (max_norm >= norm)


def test_clip_nonfinite_and_order():
    coef, norm = accumulate.clip_coefficient([1.0, float("nan")], 1.0)
    assert np.isnan(coef) and np.isnan(norm)
    coef, norm = accumulate.clip_coefficient([4.0, 5.0], 1.0)
    assert norm == 3.0 and coef == np.float32(1.0 / (3.0 + 1e-6))
    coef, _ = accumulate.clip_coefficient([0.0], 1.0)
    assert coef == np.float32(1.0)
