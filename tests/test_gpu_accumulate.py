"""GPU parity of micro-batch accumulation (ZeRO-1 and ZeRO-2 orders) and of the
global-norm clip coefficient against the oracle."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from oracle import accumulate as oacc
from oracle import reduce as oreduce
from _gpu import bits32, check_adamw, check_bf16, device_rows, device_state, host, hparams

pytestmark = pytest.mark.gpu


def _zero2(mbs, n, scale, sumsq=False, offset=0):
    acc = torch.empty(n + offset, device="cuda")[offset:]
    s = torch.empty(1, device="cuda", dtype=torch.float64) if sumsq else None
    ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8) if sumsq else None
    for k, rows in enumerate(mbs):
        last = k == len(mbs) - 1
        zs.zs_accumulate_grads(rows, acc, scale=scale, first=(k == 0),
                               sumsq_out=s if last else None, workspace=ws if last else None)
    torch.cuda.synchronize()
    return host(acc), (float(s.item()) if sumsq else None)


# world sizes of each launch shape: one-wave (3, 5-7, 8, with reservations
# that change with N and the row type; 12 loading its rows in one batch),
# rank-major 8-wave (16, 64,
# 100; 30 with fp32 rows), rank-major with the last 1-3 ranks in a short second
# walk (30 and 31 with bf16 rows, 31, 33, 65)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("world", [3, 5, 6, 7, 8, 12, 16, 30, 31, 33, 64, 65, 100])
def test_zero2_accumulation_matches_oracle(dtype, world):
    n = 262144 + 5
    # four micro-batches (the sum of squares with the last), and one alone
    # (the sum of squares with the first call)
    for k, scale in ((4, 1.0 / 4), (4, 1.0 / 3), (4, 1.0), (1, 1.0 / 3), (1, 1.0)):
        mbs = [device_rows(900 + 10 * world + j, world, n, dtype) for j in range(k)]
        acc, ss = _zero2(mbs, n, scale, sumsq=True)
        want = oacc.zero2_accumulate([np.stack([host(r) for r in rows]) for rows in mbs], scale)
        assert np.array_equal(bits32(acc), bits32(want))
        ref = oreduce.sumsq(acc)
        assert abs(ss - ref) <= 1e-12 * ref


def test_zero2_accumulation_misaligned_accumulator():
    k, n, world = 3, 10001, 8
    mbs = [device_rows(950 + j, world, n, "bf16") for j in range(k)]
    acc, _ = _zero2(mbs, n, 1.0 / 3, offset=1)
    want = oacc.zero2_accumulate([np.stack([host(r) for r in rows]) for rows in mbs], 1.0 / 3)
    assert np.array_equal(bits32(acc), bits32(want))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero1_accumulation_matches_oracle(dtype):
    k, n, world = 4, 131072 + 3, 8
    mbs = [device_rows(970 + j, world, n, dtype) for j in range(k)]
    local = [torch.empty(n, device="cuda") for _ in range(world)]
    for j, rows in enumerate(mbs):
        for r in range(world):
            zs.zs_accumulate_local(rows[r], local[r], first=(j == 0))
    g = torch.empty(n, device="cuda")
    zs.zs_accumulate_grads(local, g, scale=1.0 / k, first=True)
    torch.cuda.synchronize()
    want = oacc.zero1_accumulate([np.stack([host(r) for r in rows]) for rows in mbs], 1.0 / k)
    assert np.array_equal(bits32(host(g)), bits32(want))
    # the local accumulators themselves, against the same fp32 sums
    for r in (0, world - 1):
        loc = None
        for rows in mbs:
            c = oreduce.decode_rows(np.stack([host(rows[r])]))[0]
            loc = c.copy() if loc is None else (loc + c).astype(np.float32)
        assert np.array_equal(bits32(host(local[r])), bits32(loc))


def test_both_orders_give_the_full_batch_gradient_on_dyadic_inputs():
    # Lesson 5 s3: accumulating before or after the reduce-scatter gives the same
    # gradient; with exactly representable inputs the GPU shows it bit for bit
    world, k, b, n = 8, 4, 2, 4096
    rng = np.random.default_rng(6)
    a = rng.integers(-64, 64, size=(k, world, b, n)) / 256.0
    local = a.mean(axis=2).astype(np.float32)
    full = a.reshape(-1, n).mean(axis=0)
    mbs = [[torch.from_numpy(local[j, r].copy()).cuda() for r in range(world)] for j in range(k)]
    z2, _ = _zero2(mbs, n, 1.0 / k)
    acc = [torch.empty(n, device="cuda") for _ in range(world)]
    for j in range(k):
        for r in range(world):
            zs.zs_accumulate_local(mbs[j][r], acc[r], first=(j == 0))
    z1 = torch.empty(n, device="cuda")
    zs.zs_accumulate_grads(acc, z1, scale=1.0 / k, first=True)
    torch.cuda.synchronize()
    assert np.array_equal(z2.astype(np.float64), full)
    assert np.array_equal(host(z1).astype(np.float64), full)


def test_clip_coefficient_and_clipped_step():
    world, n, max_norm = 4, 65536 + 3, 0.05
    shard_sumsq = torch.empty(world, device="cuda", dtype=torch.float64)
    ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8)
    grads = []
    for r in range(world):  # every simulated rank's reduced shard and its partial
        rows = device_rows(990 + r, 8, n, "bf16")
        g = torch.empty(n, device="cuda")
        zs.zs_reduce_grads(rows, g, sumsq_out=shard_sumsq[r:r + 1], workspace=ws)
        grads.append(g)
    coef = torch.empty(1, device="cuda")
    norm = torch.empty(1, device="cuda", dtype=torch.float64)
    zs.zs_clip_coefficient(shard_sumsq, max_norm, coef, norm)
    torch.cuda.synchronize()
    parts = host(shard_sumsq)
    want_coef, want_norm = oacc.clip_coefficient(parts, max_norm)
    assert abs(float(norm.item()) - want_norm) <= 1e-15 * want_norm
    assert abs(float(coef.item()) - float(want_coef)) <= np.spacing(np.float32(want_coef))
    assert float(coef.item()) < 1.0  # this case clips
    # the global norm equals the norm of all shards together
    allg = np.concatenate([host(g) for g in grads]).astype(np.float64)
    assert abs(want_norm - np.sqrt(np.dot(allg, allg))) <= 1e-12 * want_norm
    # AdamW with the coefficient as the device-side gradient scale
    th, m, v = device_state(995, n)
    before = tuple(host(t).copy() for t in (th, m, v))
    out = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    zs.zs_adamw_step(th, m, v, grads[0], step=2, grad_scale=coef, bf16_out=out, **hparams())
    torch.cuda.synchronize()
    g_scaled = (host(grads[0]) * np.float32(coef.item())).astype(np.float32)
    after = tuple(host(t) for t in (th, m, v))
    th_or = check_adamw(after, before, g_scaled, 2, hparams())
    check_bf16(host(out), after[0], th_or)


def test_clip_coefficient_edge_cases():
    coef = torch.empty(1, device="cuda")
    zs.zs_clip_coefficient(torch.tensor([1e-12, 2e-12], device="cuda", dtype=torch.float64), 1.0, coef)
    torch.cuda.synchronize()
    assert coef.item() == 1.0  # below the threshold: no clipping
    zs.zs_clip_coefficient(torch.tensor([1.0, float("nan")], device="cuda", dtype=torch.float64), 1.0, coef)
    torch.cuda.synchronize()
    assert np.isnan(coef.item())
