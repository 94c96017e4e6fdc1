"""Pins of the oracle's gradient reduction (mean over ranks)."""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import bf16, reduce
from synth import gen

U32 = Fraction(1, 2 ** 24)  # unit roundoff of fp32


def _fp32_ulp(x: float) -> Fraction:
    x = abs(float(x))
    if x < 2.0 ** -126:
        return Fraction(1, 2 ** 149)
    e = math.frexp(x)[1] - 1
    return Fraction(2) ** (e - 23)


def _exact_mean(rows_f32):
    n = rows_f32.shape[0]
    return [sum(Fraction(float(rows_f32[r, k])) for r in range(n)) / n for k in range(rows_f32.shape[1])]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mean_exact_is_rounded_once(dtype):
    for world in (1, 2, 3, 4, 7, 8, 9):
        rows = gen.host_grad_rows(11 + world, world, 33, dtype)
        c = reduce.decode_rows(rows)
        got = reduce.mean_exact(rows)
        for k, q in enumerate(_exact_mean(c)):
            err = abs(Fraction(float(got[k])) - q)
            # correctly rounded (double rounding through fp64 can only matter
            # within 2^-29 relative of a halfway point)
            assert err <= _fp32_ulp(q) / 2 * (1 + Fraction(1, 2 ** 20)), (world, k)


def test_mean_seq32_order_is_ascending_from_rank0():
    one = np.float32(1.0)
    tiny = np.float32(2.0 ** -24)
    # 1 + 2^-24 is a tie that rounds back to 1, so adding the tiny values one at a
    # time after rank 0's 1.0 loses all of them ...
    rows = np.array([[one], [tiny], [tiny], [tiny]], dtype=np.float32)
    assert reduce.mean_seq32(rows)[0] == np.float32(0.25)
    # ... while summing the tiny values first keeps them: (2^-23 + 1) / 3 in fp32
    rows2 = np.array([[tiny], [tiny], [one]], dtype=np.float32)
    want = np.float32(np.float32(1.0 + 2.0 ** -23) / np.float32(3.0))
    assert reduce.mean_seq32(rows2)[0] == want
    # the exact mean sees every term in both cases
    assert reduce.mean_exact(rows)[0] == np.float32((1.0 + 3 * 2.0 ** -24) / 4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_seq32_within_recursive_summation_bound(dtype):
    # Higham, recursive summation: |s_hat - s| <= (n-1) u sum|x| (to first order);
    # then one more rounding for the division by N.
    for world in (2, 4, 8, 13, 64):
        rows = gen.host_grad_rows(5 + world, world, 257, dtype)
        c = reduce.decode_rows(rows).astype(np.float64)
        got = reduce.mean_seq32(rows).astype(np.float64)
        exact = c.sum(axis=0) / world
        bound = (world - 1) * float(U32) * np.abs(c).sum(axis=0) / world * (1 + 1e-6) + float(U32) * np.abs(got)
        assert np.all(np.abs(got - exact) <= bound + 1e-45)


def test_single_rank_and_identical_contributions():
    rows = gen.host_grad_rows(3, 1, 1000, "bf16")
    assert np.array_equal(reduce.mean_exact(rows).view(np.uint32), rows[0].astype(np.uint32) << 16)
    assert np.array_equal(reduce.mean_seq32(rows).view(np.uint32), rows[0].astype(np.uint32) << 16)
    for world in (2, 3, 5, 7, 8, 13, 63, 64):
        same = np.repeat(rows, world, axis=0)
        # k*c is exact in fp32 for k <= 64 and bf16 c, and the one correctly
        # rounded division of k*c by k returns c (dividing each term by k first
        # would not, for k other than a power of two)
        assert np.array_equal(reduce.mean_seq32(same), bf16.from_bf16_bits(rows[0]))
        assert np.array_equal(reduce.mean_exact(same), bf16.from_bf16_bits(rows[0]))


def test_exact_mean_is_order_free():
    rows = gen.host_grad_rows(9, 8, 500, "bf16")
    perm = np.random.default_rng(0).permutation(8)
    assert np.array_equal(reduce.mean_exact(rows), reduce.mean_exact(rows[perm]))


def _dyadic(rng, shape, bits=6):
    return (rng.integers(-(2 ** bits), 2 ** bits, size=shape) / 2.0 ** (bits + 2)).astype(np.float64)


def test_mean_of_rank_means_equals_full_batch_gradient_linear_loss():
    # DP-and-ZeRO page s3.1: with B samples split evenly over N ranks, the mean of
    # the local mean gradients equals the full-batch mean gradient. Per-sample
    # loss l_i(w) = a_i . w has gradient a_i.
    rng = np.random.default_rng(1)
    n_rank, b, d = 4, 4, 16
    a = _dyadic(rng, (n_rank * b, d))
    full = a.mean(axis=0)
    local = a.reshape(n_rank, b, d).mean(axis=1)  # dyadic, exact
    rows_bf16 = bf16.to_bf16_bits(local.astype(np.float32))
    assert np.array_equal(bf16.from_bf16_bits(rows_bf16).astype(np.float64), local)  # bf16-exact
    for rows in (local.astype(np.float32), rows_bf16):
        assert np.array_equal(reduce.mean_exact(rows).astype(np.float64), full)
        assert np.array_equal(reduce.mean_seq32(rows).astype(np.float64), full)


def test_mean_of_rank_means_equals_full_batch_gradient_least_squares():
    # l_i(w) = 1/2 (w . x_i - y_i)^2 has gradient (w . x_i - y_i) x_i
    rng = np.random.default_rng(2)
    n_rank, b, d = 4, 2, 8
    x = (rng.integers(-3, 4, size=(n_rank * b, d)) / 4.0)
    y = (rng.integers(-3, 4, size=n_rank * b) / 4.0)
    w = (rng.integers(-3, 4, size=d) / 4.0)
    per_sample = (x @ w - y)[:, None] * x  # exact small dyadics
    full = per_sample.mean(axis=0)
    local = per_sample.reshape(n_rank, b, d).mean(axis=1)
    assert np.array_equal(reduce.mean_exact(local.astype(np.float32)).astype(np.float64), full)
    assert np.array_equal(reduce.mean_seq32(local.astype(np.float32)).astype(np.float64), full)


def test_tail_batch_misweighting_breaks_equivalence():
    # DP-and-ZeRO page s9 experiment 4: when the last rank holds one sample and the
    # others two, the plain mean over ranks weights samples wrongly.
    a = np.array([[1.0], [2.0], [3.0], [4.0], [5.0], [6.0], [8.0]])
    sizes = [2, 2, 2, 1]
    local, i = [], 0
    for s in sizes:
        local.append(a[i:i + s].mean(axis=0))
        i += s
    local = np.array(local, dtype=np.float32)
    weighted = a.mean(axis=0)
    got = reduce.mean_exact(local).astype(np.float64)
    assert not np.array_equal(got, weighted)
    assert got[0] == (1.5 + 3.5 + 5.5 + 8.0) / 4 and weighted[0] == 29.0 / 7


def test_sumsq_matches_exact_sum():
    g = gen.host_normal(4, 4097, 1e-3)
    exact = sum(Fraction(float(x)) ** 2 for x in g)
    assert abs(Fraction(reduce.sumsq(g)) - exact) <= exact * Fraction(1, 10 ** 12)


def test_bad_rows():
    with pytest.raises(ValueError):
        reduce.decode_rows(np.zeros(4, np.float32))
    with pytest.raises(ValueError):
        reduce.decode_rows(np.zeros((2, 4), np.float64))


def test_abs_mean_hand_values():
    # The reduction's error scale (sum_r |c_r|) / N, worked by hand.
    # [1, -3]: (1 + 3) / 2 = 2, where |sum| / N would give 1 and sum|c| alone 4.
    got = reduce.abs_mean(np.array([[1.0], [-3.0]], dtype=np.float32))
    assert got.dtype == np.float64 and got.tolist() == [2.0]
    # three ranks, two columns: (1 + 3 + 5) / 3 = 3 and (2 + 4 + 0) / 3 = 2
    rows = np.array([[1.0, -2.0], [3.0, 4.0], [-5.0, 0.0]], dtype=np.float32)
    assert reduce.abs_mean(rows).tolist() == [3.0, 2.0]
    # bf16 patterns: 0x3f80 = 1.0, 0xc040 = -3.0, 0x4000 = 2.0, 0x8000 = -0.0
    rows16 = np.array([[0x3F80, 0x8000], [0xC040, 0x4000]], dtype=np.uint16)
    assert reduce.abs_mean(rows16).tolist() == [2.0, 1.0]


def test_abs_mean_special_cases():
    c = gen.host_grad_rows(21, 1, 300, "bf16")
    mag = np.abs(bf16.from_bf16_bits(c[0]).astype(np.float64))
    for world in (1, 2, 5, 64):
        # N identical contributions: the scale is |c| itself, whatever N
        assert np.array_equal(reduce.abs_mean(np.repeat(c, world, axis=0)), mag)
    # contributions of one sign: the scale is the magnitude of the exact mean
    rows = gen.host_grad_rows(22, 6, 300, "f32")
    pos = np.abs(rows)
    assert np.array_equal(reduce.abs_mean(pos), pos.astype(np.float64).sum(axis=0) / 6)
    # flipping the sign of any one rank leaves it unchanged; it bounds |mean|
    flipped = rows.copy()
    flipped[2] = -flipped[2]
    assert np.array_equal(reduce.abs_mean(flipped), reduce.abs_mean(rows))
    assert np.all(np.abs(reduce.mean_exact(rows).astype(np.float64)) <= reduce.abs_mean(rows) * (1 + 2.0 ** -23))
