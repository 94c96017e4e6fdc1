"""Pins of the oracle's fp32 -> bf16 rounding.

Checked against hand-worked bit patterns and against PyTorch's own CPU
conversion (a library round-to-nearest-even), which agrees on every non-NaN
input; NaN handling is fixed by the stated reading (quiet, sign kept).
"""
import numpy as np
import torch

from oracle import bf16


def _bits(vals):
    return np.array(vals, dtype=np.uint32).view(np.float32)


def test_hand_worked_patterns():
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0x3F808000: 0x3F80,  # 1 + 2^-8: exact tie, kept part even -> down
        0x3F818000: 0x3F82,  # 1 + 3*2^-8: tie, kept part odd -> up
        0x3F808001: 0x3F81,  # just above the tie -> up
        0x3F807FFF: 0x3F80,  # just below the tie -> down
        0xBF808001: 0xBF81,  # negative mirrors positive
        0x7F7FFFFF: 0x7F80,  # largest finite fp32 overflows to +inf
        0xFF7FFFFF: 0xFF80,
        0x7F800000: 0x7F80,  # +inf stays inf
        0x00000001: 0x0000,  # smallest subnormal rounds to +0
        0x80000001: 0x8000,  # ... and to -0 when negative
        0x00008000: 0x0000,  # subnormal tie, even -> down
        0x00018000: 0x0002,  # subnormal tie, odd -> up
        0x00000000: 0x0000,
        0x80000000: 0x8000,
    }
    got = bf16.to_bf16_bits(_bits(list(cases))).tolist()
    assert got == list(cases.values())


def test_nan_stays_quiet_nan():
    nans = [0x7FC00000, 0x7F800001, 0xFF800001, 0x7FBFFFFF, 0xFFFFFFFF]
    got = bf16.to_bf16_bits(_bits(nans))
    for src, b in zip(nans, got.tolist()):
        assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0  # NaN
        assert b & 0x0040  # quiet
        assert (b & 0x8000) == ((src >> 16) & 0x8000)  # sign kept
    assert got.tolist() == [0x7FC0, 0x7FC0, 0xFFC0, 0x7FFF, 0xFFFF]


def test_against_torch_on_many_patterns():
    rng = np.random.default_rng(123)
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    x = pats.view(np.float32)
    finite_or_inf = ~np.isnan(x)
    ours = bf16.to_bf16_bits(x[finite_or_inf])
    ref = torch.from_numpy(x[finite_or_inf].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_decode_is_exact_and_roundtrips():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16.from_bf16_bits(b)
    assert np.array_equal(f.view(np.uint32), b.astype(np.uint32) << 16)
    keep = ~np.isnan(f)
    assert np.array_equal(bf16.to_bf16_bits(f[keep]), b[keep])


def test_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8001, 0x7F7F], dtype=np.uint16)
    c = np.array([0x3F81, 0x3F7F, 0x8000, 0x0001, 0x7F80], dtype=np.uint16)
    assert bf16.ulp_distance(a, c).tolist() == [1, 1, 0, 2, 1]


def test_ulp_spacing():
    assert bf16.ulp(np.array([1.0, 1.5, 1.99, 2.0, -3.0, 0.0, 2.0 ** -130])).tolist() == [
        2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133]
    # adjacent bf16 values differ by exactly ulp
    b = np.arange(0x0080, 0x7F00, 37, dtype=np.uint16)
    lo, hi = bf16.from_bf16_bits(b).astype(np.float64), bf16.from_bf16_bits(b + 1).astype(np.float64)
    assert np.array_equal(hi - lo, bf16.ulp(lo))
