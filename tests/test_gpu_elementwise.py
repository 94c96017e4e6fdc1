"""GPU parity of the element-wise paths.

Every vector kernel moves 16-byte vectors (8-byte ones for bf16 rows), so each
entry point falls back to a lane-per-element kernel with the same arithmetic
when a pointer sits off that grid: a contribution row 2 bytes (bf16) or 4 bytes
(fp32) past it, fp32 state or an fp32 source 4 bytes past it. The pages fix
what is computed, not how it is laid out ("Lesson 5: ZeRO and FSDP" s3 and
s7.1: the reduce-scatter result, the local AdamW step and the BF16 copy of the
rank's slice), so the element-wise paths must give the vector paths' bits:
each case compares them with the oracle and, where two entry points compute
the same thing, bit for bit with each other, with and without the gradient
scale, the bf16 copy and the sum of squares.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from oracle import accumulate as oacc
from oracle import bf16 as obf16
from oracle import reduce as oreduce
from _gpu import bits32, check_adamw, check_bf16, check_mean, device_rows, device_state, host, hparams

pytestmark = pytest.mark.gpu

N = 70001  # several workgroups of the element-wise kernels and a ragged end


def _rows(seed, world, dtype, off):
    return [r[off:off + N] for r in device_rows(seed, world, N + 1, dtype)]


def _state(seed, off):
    return tuple(t[off:off + N] for t in device_state(seed, N + 1))


def _copy(state):
    """Copies at the same offset from the vector grid as the originals."""
    out = []
    for t in state:
        off = (t.data_ptr() - t.untyped_storage().data_ptr()) // 4
        c = torch.empty(N + 1, device="cuda")[off:off + N]
        c.copy_(t)
        out.append(c)
    return tuple(out)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("world", [3, 16])
@pytest.mark.parametrize("where", ["rows", "state"])
def test_single_pass_off_the_grid_is_bitwise_the_two_calls(dtype, world, where):
    # rows off the grid: the single pass goes element by element while the two
    # calls reduce element by element and run the vector AdamW; state off the
    # grid: both AdamW paths go element by element after a vector reduce
    rows = _rows(1200 + world, world, dtype, 1 if where == "rows" else 0)
    a = _state(1210 + world, 1 if where == "state" else 0)
    b = _copy(a)
    g = torch.empty(N, device="cuda")
    oa = torch.empty(N, device="cuda", dtype=torch.bfloat16)
    ob = torch.empty_like(oa)
    sc = torch.tensor([0.5], device="cuda")
    hp = hparams()
    before = tuple(host(t).copy() for t in a)
    for step, scale, cast in ((1, None, True), (2, sc, True), (3, None, False), (4, sc, False)):
        zs.zs_reduce_grads(rows, g)
        zs.zs_adamw_step(*a, g, step=step, grad_scale=scale, bf16_out=oa if cast else None, **hp)
        zs.zs_sharded_step(rows, *b, step=step, grad_scale=scale, bf16_out=ob if cast else None, **hp)
        if step == 1:  # the first step against the oracle
            torch.cuda.synchronize()
            rows_h = np.stack([host(r) for r in rows])
            check_mean(host(g), rows_h)
            after = tuple(host(t) for t in b)
            th_or = check_adamw(after, before, oreduce.mean_seq32(rows_h), 1, hp)
            check_bf16(host(ob), after[0], th_or)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(bits32(host(x)), bits32(host(y)))
    assert np.array_equal(host(oa), host(ob))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reduce_off_the_grid_with_sum_of_squares(dtype):
    rows = _rows(1230, 7, dtype, 1)
    g = torch.empty(N, device="cuda")
    s = torch.empty(1, device="cuda", dtype=torch.float64)
    ws = torch.empty(zs.zs_workspace_bytes(N), device="cuda", dtype=torch.uint8)
    zs.zs_reduce_grads(rows, g, sumsq_out=s, workspace=ws)
    torch.cuda.synchronize()
    gh = host(g)
    check_mean(gh, np.stack([host(r) for r in rows]))
    ref = oreduce.sumsq(gh)
    assert abs(s.item() - ref) <= 1e-12 * ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("where", ["rows", "acc"])
def test_accumulation_off_the_grid_every_flag(dtype, where):
    # ZeRO-2 accumulation over three micro-batches, first call and later calls,
    # scaled and unscaled, with the sum of squares on the last call and with or
    # without it on the first
    world, k = 5, 3
    mbs = [_rows(1240 + j, world, dtype, 1 if where == "rows" else 0) for j in range(k)]
    mbs_h = [np.stack([host(r) for r in rows]) for rows in mbs]
    for scale, sumsq_first in ((1.0, True), (1.0 / 3, True), (1.0, False), (1.0 / 3, False)):
        acc = torch.empty(N + 1, device="cuda")[(1 if where == "acc" else 0):][:N]
        s = torch.empty(1, device="cuda", dtype=torch.float64)
        ws = torch.empty(zs.zs_workspace_bytes(N), device="cuda", dtype=torch.uint8)
        for j, rows in enumerate(mbs):
            with_sumsq = j == k - 1 or (j == 0 and sumsq_first)
            zs.zs_accumulate_grads(rows, acc, scale=scale, first=(j == 0),
                                   sumsq_out=s if with_sumsq else None, workspace=ws if with_sumsq else None)
            if j == 0:
                torch.cuda.synchronize()
                first = host(acc).copy()
                assert np.array_equal(bits32(first), bits32(oacc.zero2_accumulate(mbs_h[:1], scale)))
                if sumsq_first:
                    ref = oreduce.sumsq(first)
                    assert abs(s.item() - ref) <= 1e-12 * ref
        torch.cuda.synchronize()
        got = host(acc)
        assert np.array_equal(bits32(got), bits32(oacc.zero2_accumulate(mbs_h, scale)))
        ref = oreduce.sumsq(got)
        assert abs(s.item() - ref) <= 1e-12 * ref


def test_cast_from_a_source_off_the_grid():
    src = device_state(1250, N + 1)[0][1:]
    out = torch.empty(N, device="cuda", dtype=torch.bfloat16)
    zs.zs_cast_for_gather(src, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), obf16.to_bf16_bits(host(src)))
