"""GPU parity at the edges of the index and rank ranges.

* Buffers of more than 2^31 elements (an fp32 array of 8.6 GB): every kernel's
  element, byte and group offsets must be 64-bit. The step, the two-call path,
  the cast, pack and copy-out run on 2^31 + 12 elements and are checked on
  windows at the start, across the 2^31 boundary and at the end, with the
  whole-buffer properties (sum of squares, bitwise equality of the two paths)
  checked everywhere.
* World sizes above 64, up to the ABI's maximum of 256 contributions (the row
  table of the widest kernel instantiation).
"""
import math

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from oracle import accumulate as oacc
from oracle import bf16 as obf16
from oracle import reduce as oreduce
from synth import gen
from _gpu import bits32, check_adamw, check_bf16, check_mean, device_rows, host, hparams

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + 12
EDGE = 1 << 31


def _windows(n, width=32768):
    return [(0, width), (EDGE - width, min(n, EDGE + width)), (n - width, n)]


@pytest.mark.parametrize("world", [2, 16])  # the one-wave and the rank-major 8-wave shape
def test_step_beyond_2g_elements(world):
    n = BIG
    rows = device_rows(31000 + world, world, n, "bf16")
    g0 = gen.device_generator(31001)
    th = gen.device_normal(g0, n, gen.THETA_SIGMA)
    m = gen.device_normal(g0, n, 1e-4)
    v = gen.device_normal(g0, n, 1e-6).abs_()
    wins = _windows(n)
    before = [tuple(host(t[a:b]).copy() for t in (th, m, v)) for a, b in wins]
    hp = hparams()
    fused = tuple(t.clone() for t in (th, m, v))
    g = torch.empty(n, device="cuda")
    slot = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    fslot = torch.empty_like(slot)
    sumsq = torch.empty(1, device="cuda", dtype=torch.float64)
    ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8)
    zs.zs_reduce_grads(rows, g, sumsq_out=sumsq, workspace=ws)
    zs.zs_adamw_step(th, m, v, g, step=3, bf16_out=slot, **hp)
    zs.zs_sharded_step(rows, *fused, step=3, bf16_out=fslot, **hp)
    torch.cuda.synchronize()
    for (a, b), bef in zip(wins, before):
        rows_h = np.stack([host(r[a:b]) for r in rows])
        gw = host(g[a:b])
        check_mean(gw, rows_h)
        after = tuple(host(t[a:b]) for t in (th, m, v))
        th_or = check_adamw(after, bef, gw, 3, hp)
        check_bf16(host(slot[a:b]), after[0], th_or)
    for x, y in zip((th, m, v), fused):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(slot.view(torch.int16), fslot.view(torch.int16))
    del rows, fused, fslot, m, v
    # the fp64 sum of squares of all 2^31 + 12 reduced values on the host: the
    # oracle on 2^24-element chunks, whose partials fsum adds exactly (one
    # sequential fp64 dot over 2^31 values is itself off by a few parts in 1e12)
    chunk = 1 << 24
    ref = math.fsum(oreduce.sumsq(host(g[a:min(a + chunk, n)])) for a in range(0, n, chunk))
    assert abs(sumsq.item() - ref) <= 1e-12 * ref
    # the standalone cast over the same range
    zs.zs_cast_for_gather(th, slot)
    torch.cuda.synchronize()
    for a, b in wins:
        assert np.array_equal(host(slot[a:b]), obf16.to_bf16_bits(host(th[a:b])))
    del th, g, slot
    torch.cuda.empty_cache()


def test_pack_and_copy_out_beyond_2g_elements():
    # a unit of three parameters whose flat range passes 2^31: pack rank 0 of
    # world 1 (the whole flat buffer), then copy a gathered bf16 buffer out
    numels = [EDGE - 5000, 3000]  # the third parameter starts 2000 below 2^31
    numels.append(BIG - sum(numels))
    g0 = gen.device_generator(31100)
    params = [gen.device_normal(g0, k, gen.THETA_SIGMA) for k in numels]
    table = zs.ParamTable(params)
    offsets, total, padded, shard = zs.zs_flat_layout(numels, 1)
    assert total == BIG and shard == BIG
    master = torch.empty(shard, device="cuda")
    zs.zs_pack_shard(table, 1, 0, master)
    torch.cuda.synchronize()
    for a, b in _windows(BIG):
        want = np.empty(b - a, np.float32)
        for p, off, k in zip(params, offsets, numels):
            lo, hi = max(a, off), min(b, off + k)
            if lo < hi:
                want[lo - a:hi - a] = host(p[lo - off:hi - off])
        assert np.array_equal(bits32(host(master[a:b])), bits32(want))
    del params, table, master
    torch.cuda.empty_cache()

    gathered = gen.device_normal(g0, BIG, 1.0, torch.bfloat16)
    dst = [torch.empty(k, device="cuda", dtype=torch.bfloat16) for k in numels]
    zs.zs_copy_out(gathered, zs.ParamTable(dst))
    torch.cuda.synchronize()
    for d, off, k in zip(dst, offsets, numels):
        for a, b in ((0, min(k, 4096)), (max(0, k - 4096), k)):
            assert np.array_equal(host(d[a:b]), host(gathered[off + a:off + b]))
    # whole-buffer check on the device: the destinations concatenated are the source
    assert all(torch.equal(d.view(torch.int16), gathered[off:off + k].view(torch.int16))
               for d, off, k in zip(dst, offsets, numels))
    del gathered, dst
    torch.cuda.empty_cache()


@pytest.mark.parametrize("world", [65, 100, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_worlds(world, dtype):
    n = 65536 + 5
    rows = device_rows(32000 + world, world, n, dtype)
    rows_h = np.stack([host(r) for r in rows])
    g = torch.empty(n, device="cuda")
    zs.zs_reduce_grads(rows, g)
    torch.cuda.synchronize()
    check_mean(host(g), rows_h)
    assert np.array_equal(bits32(host(g)), bits32(oreduce.mean_seq32(rows_h)))
    # the single pass equals the two calls bit for bit
    g0 = gen.device_generator(32100 + world)
    a = (gen.device_normal(g0, n, gen.THETA_SIGMA), gen.device_normal(g0, n, 1e-4),
         gen.device_normal(g0, n, 1e-6).abs_())
    b = tuple(t.clone() for t in a)
    oa = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    ob = torch.empty_like(oa)
    zs.zs_adamw_step(*a, g, step=2, bf16_out=oa, **hparams())
    zs.zs_sharded_step(rows, *b, step=2, bf16_out=ob, **hparams())
    # ZeRO-2 accumulation over two micro-batches (the same rows twice)
    acc = torch.empty(n, device="cuda")
    zs.zs_accumulate_grads(rows, acc, scale=0.5, first=True)
    zs.zs_accumulate_grads(rows, acc, scale=0.5)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    want = oacc.zero2_accumulate([rows_h, rows_h], 0.5)
    assert np.array_equal(bits32(host(acc)), bits32(want))
