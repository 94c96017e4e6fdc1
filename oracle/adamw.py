"""AdamW on the rank's fp32 master/m/v shard (oracle; test infrastructure only).

What the pages fix:
  * [L5] s3 (ZeRO-1/2 step 2) and s3 (ZeRO-3 item 4): each rank updates only
    its own 1/N of the fp32 optimizer state and master weights, locally, with
    no communication.
  * [L5] s2 and [DPZ] s3.2: the state is an fp32 master copy plus the first
    moment m and second moment v (k = 12 bytes per parameter); the optimizer is
    AdamW.
  * [DPZ] s4.2 (first-step simulator): m = (1 - b1) g, v = (1 - b2) g^2 from
    zero state, bias-corrected by 1 - b1 and 1 - b2, and the step
    theta - lr * m_hat / (sqrt(v_hat) + eps), eps outside the root.
  * [LAF] s8.2 step 6 gives the same update without bias correction (a
    simplified line); [LAF] s9.3 lists lr, beta1, beta2, epsilon, weight_decay.

Readings where the pages are silent (each one the standard published form):
  * weight decay is decoupled (Loshchilov and Hutter): theta is scaled by
    (1 - lr * wd) using the pre-step theta, not added to the gradient;
  * bias correction at step t uses 1 - b1^t and 1 - b2^t (Kingma and Ba);
  * every element gets the same decay (one parameter group).

Arithmetic: inputs are the fp32 stored values; everything is computed in fp64;
m' and v' are rounded to the state dtype (fp32 by default) and theta' is
computed from those rounded moments, then rounded once.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np


@dataclass(frozen=True)
class HParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def check_hparams(hp: HParams, step: int) -> None:
    for name in ("lr", "beta1", "beta2", "eps", "weight_decay"):
        if not math.isfinite(getattr(hp, name)):
            raise ValueError(f"{name} must be finite")
    if hp.lr < 0 or hp.eps < 0 or hp.weight_decay < 0:
        raise ValueError("lr, eps and weight_decay must be non-negative")
    if not (0.0 <= hp.beta1 < 1.0 and 0.0 <= hp.beta2 < 1.0):
        raise ValueError("betas must lie in [0, 1)")
    if step < 1:
        raise ValueError("step counts from 1")


def adamw_step(theta, m, v, g, step: int, hp: HParams, state_dtype=np.float32):
    """One AdamW step; returns (theta', m', v') in `state_dtype`."""
    check_hparams(hp, step)
    th = np.asarray(theta, dtype=np.float64)
    m0 = np.asarray(m, dtype=np.float64)
    v0 = np.asarray(v, dtype=np.float64)
    gg = np.asarray(g, dtype=np.float64)

    m1 = (hp.beta1 * m0 + (1.0 - hp.beta1) * gg).astype(state_dtype)
    v1 = (hp.beta2 * v0 + (1.0 - hp.beta2) * gg * gg).astype(state_dtype)

    bc1 = 1.0 - hp.beta1 ** step
    bc2 = 1.0 - hp.beta2 ** step
    m_hat = m1.astype(np.float64) / bc1
    v_hat = v1.astype(np.float64) / bc2
    update = hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
    th1 = (th * (1.0 - hp.lr * hp.weight_decay) - update).astype(state_dtype)
    return th1, m1, v1


def error_scales(theta, m, g, step: int, hp: HParams, m1, v1):
    """Per-element magnitudes the update's rounding errors scale with.

    m':     b1|m| + (1-b1)|g|           (the two terms summed, not their sum)
    v':     |v'|                         (both terms are non-negative)
    theta': |theta|(1 - lr wd) + lr (b1|m| + (1-b1)|g|) / (1 - b1^t) / (sqrt(v_hat) + eps)
            -- the decayed weight plus the step computed from the m'-term
            scale, since an fp32 m' carries an error proportional to its
            terms, which the step passes on even when m' itself cancels.
    A relative tolerance applied to these stays meaningful under cancellation
    and reduces to a plain relative error where none occurs.
    """
    th = np.abs(np.asarray(theta, dtype=np.float64))
    bc1 = 1.0 - hp.beta1 ** step
    bc2 = 1.0 - hp.beta2 ** step
    sm = hp.beta1 * np.abs(np.asarray(m, np.float64)) + (1 - hp.beta1) * np.abs(np.asarray(g, np.float64))
    sv = np.abs(np.asarray(v1, np.float64))
    m_hat_scale = np.maximum(sm, np.abs(np.asarray(m1, np.float64))) / bc1
    v_hat = np.asarray(v1, np.float64) / bc2
    st = th * (1.0 - hp.lr * hp.weight_decay) + hp.lr * m_hat_scale / (np.sqrt(v_hat) + hp.eps)
    return st, sm, sv
