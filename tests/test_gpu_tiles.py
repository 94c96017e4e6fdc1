"""GPU parity where the rank walks' last round is split across the device.

The reduce, the single pass and the ZeRO-2 accumulation run their multi-group
shapes in tiles of `span` lane groups (4 elements each), one tile per
workgroup, except that the groups of the last round -- what is left after
the device's resident workgroups have each taken full tiles as often as
possible -- are spread evenly over all resident workgroups, in units of 64
groups, and each lane walks only as many groups as its tile holds. Those
tiles start and end inside the arrays, cover a varying number of groups per
lane, and leave some lanes of their last group idle. These cases size the
launch against the device so that the last round holds 1-2 units per
workgroup, about 6.5 groups per lane, or a nearly full tile, after zero, one
or two full rounds (with N = 31 and 33 the last 3 or 1 ranks take a second walk), and compare every element with the oracle's
ascending-rank fp32 mean ("Data parallelism and ZeRO memory sharding" s3.1)
and the ZeRO-2 sum ("Lesson 5: ZeRO and FSDP" s3, ZeRO-2 step 1), and the
single pass bit for bit with the two calls. Output buffers start as NaN, so a
group that no tile covers fails the comparison.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from oracle import accumulate as oacc
from oracle import reduce as oreduce
from _gpu import bits32, device_rows, device_state, host, hparams

pytestmark = pytest.mark.gpu

LDS_PER_CU = 160 * 1024  # gfx950


def _shape(world, dtype):
    """(lanes, groups per lane, resident workgroups per CU) of the multi-group
    shape the dispatch picks for `world` >= 16 contributions: the rank-major
    walk in 8-wave workgroups with 128 KiB of LDS (its last chunk of ranks
    short when the chunk, 4 bf16 or 2 fp32 rows, does not divide `world`)."""
    return 512, 16, LDS_PER_CU // (512 * 16 * 16)


def _sizes(world, dtype):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bs, g, per_cu = _shape(world, dtype)
    slots, span = cus * per_cu, bs * g
    rnd = slots * span  # groups of one full round
    groups = {
        "one round, 1-2 units per workgroup": slots * 64 * 3 // 2,
        "one round, 6.5 groups per lane": slots * bs * 13 // 2,
        "two rounds, the last nearly full": rnd + rnd * 97 // 100,
        "three rounds, 38 units in the last": 2 * rnd + 64 * 37 + 5,
    }
    return {k: 4 * v + 3 for k, v in groups.items()}  # a ragged tail of 3 elements


CASES = [(16, "bf16"), (64, "f32"), (33, "bf16"), (31, "bf16"), (33, "f32")]  # 31, 33: 3 and 1 ranks after the whole chunks


@pytest.mark.parametrize("world, dtype", CASES)
def test_reduce_and_single_pass_over_split_last_rounds(world, dtype):
    for i, (what, n) in enumerate(_sizes(world, dtype).items()):
        print(f"world {world} {dtype}: {what}, n = {n}", flush=True)
        rows = device_rows(7100 + 10 * world + i, world, n, dtype)
        g = torch.full((n,), float("nan"), device="cuda")
        s = torch.empty(1, device="cuda", dtype=torch.float64)
        ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8)
        zs.zs_reduce_grads(rows, g, sumsq_out=s, workspace=ws)
        torch.cuda.synchronize()
        gh = host(g)
        want = oreduce.mean_seq32(np.stack([host(r) for r in rows]))
        assert np.array_equal(bits32(gh), bits32(want)), what
        ref = oreduce.sumsq(gh)
        assert abs(s.item() - ref) <= 1e-12 * ref, what
        # the single pass against AdamW over that gradient, bit for bit
        a = device_state(7200 + i, n)
        b = tuple(t.clone() for t in a)
        oa = torch.full((n,), float("nan"), device="cuda", dtype=torch.bfloat16)
        ob = oa.clone()
        zs.zs_adamw_step(*a, g, step=2, bf16_out=oa, **hparams())
        zs.zs_sharded_step(rows, *b, step=2, bf16_out=ob, **hparams())
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), what
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), what
        del rows, a, b
        torch.cuda.empty_cache()


@pytest.mark.parametrize("world, dtype", CASES)
def test_accumulation_over_split_last_rounds(world, dtype):
    sizes = _sizes(world, dtype)
    for i, what in enumerate(("one round, 6.5 groups per lane", "three rounds, 38 units in the last")):
        n = sizes[what]
        print(f"world {world} {dtype}: {what}, n = {n}", flush=True)
        mbs = [device_rows(7300 + 10 * world + 2 * i + j, world, n, dtype) for j in range(2)]
        acc = torch.full((n,), float("nan"), device="cuda")
        s = torch.empty(1, device="cuda", dtype=torch.float64)
        ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8)
        zs.zs_accumulate_grads(mbs[0], acc, scale=0.5, first=True)
        zs.zs_accumulate_grads(mbs[1], acc, scale=0.5, sumsq_out=s, workspace=ws)
        torch.cuda.synchronize()
        got = host(acc)
        want = oacc.zero2_accumulate([np.stack([host(r) for r in rows]) for rows in mbs], 0.5)
        assert np.array_equal(bits32(got), bits32(want)), what
        ref = oreduce.sumsq(got)
        assert abs(s.item() - ref) <= 1e-12 * ref, what
        del mbs
        torch.cuda.empty_cache()
