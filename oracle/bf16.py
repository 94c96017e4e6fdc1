"""fp32 <-> bf16 on bit patterns (oracle; test infrastructure only).

[L5] s3 step 2 and Fig. 5-4: after the local update each rank converts its
fp32 shard to BF16 in place before the all-gather; [LAF] s8.1-8.2: bf16 is the
compute/storage type of parameters, fp32 the master type. The pages do not fix
the rounding rule; the reading taken is IEEE round-to-nearest-even, with NaN
kept NaN (quiet bit forced, sign and top payload bits kept) and overflow going
to infinity.

bf16 is the top half of an fp32 pattern, so decoding is exact: value = u << 16.
"""
from __future__ import annotations

import numpy as np


def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16, returned as uint16 patterns.

    Round to nearest, ties to even, written out on the integers: keep the top
    16 bits, and round up when the dropped low half exceeds one half, or equals
    one half and the kept part is odd.
    """
    u = f32_bits(x).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (lo > half) | ((lo == half) & ((hi & np.uint64(1)) == np.uint64(1)))
    r = hi + round_up.astype(np.uint64)
    exp_all_ones = (u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)
    mant_nonzero = (u & np.uint64(0x007FFFFF)) != np.uint64(0)
    is_nan = exp_all_ones & mant_nonzero
    r = np.where(is_nan, hi | np.uint64(0x0040), r)
    return r.astype(np.uint16)


def from_bf16_bits(b) -> np.ndarray:
    """Exact decode of bf16 patterns to fp32."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in bf16 ulps between two finite bf16 patterns.

    Maps each pattern onto a monotone integer line (sign-magnitude to two's
    complement, +0 and -0 both to 0) so adjacent representable values differ
    by one.
    """
    def line(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)

    return np.abs(line(a_bits) - line(b_bits))


def ulp(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits): 2^(e-7) for a normal
    |x| in [2^e, 2^(e+1)), and 2^-133 (the subnormal spacing) below 2^-126."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)
