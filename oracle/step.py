"""The composed sharded update of one rank (oracle; test infrastructure only).

[L5] s3 (ZeRO-1/2, steps 1-3) and Fig. 5-4: the rank receives the reduced
gradient of its 1/N slice, updates its fp32 master/m/v slice locally, and
converts the result to BF16 for the all-gather. The all-gather buffer holds the
N slices rank-major, so rank r's bf16 slice lands at offset r*S
([LAF] s5.1 illustration).
"""
from __future__ import annotations

import numpy as np

from . import adamw, bf16, reduce


def sharded_step(rows, theta, m, v, step: int, hp: adamw.HParams, exact_mean: bool = True):
    """rows [N, S] (bf16 uint16 patterns or fp32) -> (g, theta', m', v', bf16 bits)."""
    g = reduce.mean_exact(rows) if exact_mean else reduce.mean_seq32(rows)
    th1, m1, v1 = adamw.adamw_step(theta, m, v, g, step, hp)
    return g, th1, m1, v1, bf16.to_bf16_bits(th1)
