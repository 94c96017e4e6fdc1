"""GPU parity of FlatParameter pack and unshard copy-out: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from oracle import bf16 as obf16
from oracle import layout as olayout
from synth import gen, shapes
from _gpu import GUARD_LENGTHS, bits32, check_guards, guarded_views, host

pytestmark = pytest.mark.gpu


def _params(shape_list, seed, dtype=torch.float32):
    g = gen.device_generator(seed)
    return [gen.device_normal(g, shapes.numel(s), gen.THETA_SIGMA, dtype).reshape(s)
            for _, s in shape_list]


def _pack(params, world, rank, align=1):
    table = zs.ParamTable(params)
    _, total, padded, shard = zs.zs_flat_layout([p.numel() for p in params], world, align)
    master = torch.full((shard,), float("nan"), device="cuda")
    m = torch.full_like(master, 3.0)
    v = torch.full_like(master, 3.0)
    zs.zs_pack_shard(table, world, rank, master, m, v, align=align)
    torch.cuda.synchronize()
    return host(master), host(m), host(v)


@pytest.mark.parametrize("name,world", [("tiny", 4), ("tiny_ragged", 4), ("tiny_ragged", 3),
                                        ("tiny_ragged", 7), ("gpt2", 8), ("gpt2", 7), ("gpt2", 5)])
def test_pack_matches_oracle_every_rank(name, world):
    shp = shapes.WORKLOADS[name][0]()
    params = _params(shp, seed=sum(map(ord, name)) + world)
    host_params = [host(p).ravel() for p in params]
    ranks = range(world) if name != "gpt2" else (0, world // 2, world - 1)
    for r in ranks:
        master, m, v = _pack(params, world, r)
        want, _, _ = olayout.pack_shard(host_params, world, r)
        assert np.array_equal(bits32(master), bits32(want)), (name, world, r)
        assert not bits32(m).any() and not bits32(v).any()


@pytest.mark.parametrize("name,world,align", [("tiny_ragged", 3, 3), ("tiny_ragged", 7, 64), ("gpt2", 5, 64),
                                              ("gpt2", 8, 1000)])
def test_pack_with_aligned_slices_matches_oracle_every_rank(name, world, align):
    # slices rounded up to a multiple of `align` elements: each rank's master
    # is the oracle's, the padding past the unit +0
    shp = shapes.WORKLOADS[name][0]()
    params = _params(shp, seed=sum(map(ord, name)) + world + align)
    host_params = [host(p).ravel() for p in params]
    ranks = range(world) if name != "gpt2" else (0, world // 2, world - 1)
    for r in ranks:
        master, m, v = _pack(params, world, r, align)
        want, _, _ = olayout.pack_shard(host_params, world, r, align)
        assert master.size % align == 0
        assert np.array_equal(bits32(master), bits32(want)), (name, world, align, r)
        assert not bits32(m).any() and not bits32(v).any()


def test_pack_bf16_sources_widen_exactly():
    shp = shapes.tiny_ragged() + [("e", (1000,)), ("f", (9, 9))]
    params = _params(shp, seed=12, dtype=torch.bfloat16)
    hp = [host(p).ravel() for p in params]
    for world in (1, 4, 5):
        for r in range(world):
            master, _, _ = _pack(params, world, r)
            want, _, _ = olayout.pack_shard(hp, world, r)
            assert np.array_equal(bits32(master), bits32(want))


def test_pack_tiny_shard_is_param():
    params = _params(shapes.tiny(), seed=3)
    for r in range(4):
        master, _, _ = _pack(params, 4, r)
        assert np.array_equal(bits32(master), bits32(host(params[r]).ravel()))


def _copy_out_case(shape_list, seed, world):
    numels = shapes.numels(shape_list)
    _, total, padded, _ = zs.zs_flat_layout(numels, world)
    g = gen.device_generator(seed)
    gathered = gen.device_normal(g, padded, 1.0, torch.bfloat16)
    dst = [torch.full(s, float("nan"), device="cuda", dtype=torch.bfloat16) for _, s in shape_list]
    table = zs.ParamTable(dst)
    zs.zs_copy_out(gathered, table)
    torch.cuda.synchronize()
    want = olayout.copy_out(host(gathered), [s for _, s in shape_list])
    for d, w in zip(dst, want):
        assert np.array_equal(host(d), w)


@pytest.mark.parametrize("name,world", [("tiny_ragged", 4), ("tiny", 4), ("gpt2", 8), ("gpt2", 7)])
def test_copy_out_matches_oracle(name, world):
    _copy_out_case(shapes.WORKLOADS[name][0](), seed=21, world=world)


def test_copy_out_misaligned_offsets_and_tiny_params():
    # odd element counts put most parameters off the 16-byte grid of the flat buffer
    shp = [(f"p{i}", (n,)) for i, n in enumerate([1, 3, 5, 7, 9, 4097, 8191, 2, 16384, 13, 65537, 1])]
    _copy_out_case(shp, seed=22, world=3)


def test_copy_out_every_source_and_destination_shift():
    # every offset of source and destination from the 16-byte grid, with lengths
    # around the vector thresholds and the per-workgroup chunk
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.permutation(GUARD_LENGTHS * 3)]
    big, dst, starts = guarded_views(lengths, seed=32)
    numels = lengths
    _, total, padded, _ = zs.zs_flat_layout(numels, 1)
    gathered = gen.device_normal(gen.device_generator(33), padded, 1.0, torch.bfloat16)
    zs.zs_copy_out(gathered, zs.ParamTable(dst))
    torch.cuda.synchronize()
    want = olayout.copy_out(host(gathered), [(n,) for n in numels])
    offs = olayout.flat_layout(numels, 1).offsets
    assert {o % 8 for o in offs} == set(range(8)) and {a % 8 for a in starts} == set(range(8))
    for i, (d, w) in enumerate(zip(dst, want)):
        assert np.array_equal(host(d), w), (i, lengths[i], offs[i] % 8, starts[i] % 8)
    check_guards(big, starts, lengths)


def test_copy_out_llama8b_block_full():
    _copy_out_case(shapes.llama3_8b_block(), seed=23, world=8)


def test_copy_out_70b_block_full():
    # one 70B decoder block (855,654,400 elements, 9 tensors), as the benchmark times it
    _copy_out_case(shapes.llama_70b_block(), seed=24, world=64)


@pytest.mark.parametrize("align", [1, 64])
def test_roundtrip_pack_cast_gather_copy_out(align):
    # with lr = wd = 0, theta is unchanged, so the unsharded parameters come back
    # as the bf16 rounding of the originals, bit for bit; with slices rounded to
    # 64 elements every rank's slot starts on a 128-byte line (S = 24,887,962
    # by the pages' rule puts odd ranks' slots 4 bytes off an 8-byte boundary)
    shp = shapes.gpt2_small()
    world = 5
    params = _params(shp, seed=31)
    numels = [p.numel() for p in params]
    _, total, padded, shard = zs.zs_flat_layout(numels, world, align)
    table = zs.ParamTable(params)
    gather = torch.empty(padded, device="cuda", dtype=torch.bfloat16)
    if align == 64:
        assert all((gather.data_ptr() + 2 * r * shard) % 128 == 0 for r in range(world))
    for r in range(world):
        master = torch.empty(shard, device="cuda")
        m = torch.empty_like(master)
        v = torch.empty_like(master)
        zs.zs_pack_shard(table, world, r, master, m, v, align=align)
        zero_g = torch.zeros(shard, device="cuda")
        zs.zs_adamw_step(master, m, v, zero_g, step=1, lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8,
                         weight_decay=0.0, bf16_out=gather[r * shard:(r + 1) * shard])
    dst = [torch.empty(s, device="cuda", dtype=torch.bfloat16) for _, s in shp]
    zs.zs_copy_out(gather, zs.ParamTable(dst))
    torch.cuda.synchronize()
    for d, p in zip(dst, params):
        assert np.array_equal(host(d).ravel(), obf16.to_bf16_bits(host(p).ravel()))
    assert not host(gather)[total:].any()  # the tail pad gathered as +0


def test_pack_llama8b_full_windows_at_every_boundary():
    # the whole 8B list as fp32 parameters (32 GB); ranks 3 and 7, checked in
    # windows around every parameter boundary inside the shard plus random ones
    shp = shapes.llama3_8b()
    numels = shapes.numels(shp)
    world = 8
    g = gen.device_generator(41)
    params = [gen.device_normal(g, n, gen.THETA_SIGMA) for n in numels]
    lay = olayout.flat_layout(numels, world)
    table = zs.ParamTable(params)
    fetch = lambda i, a, b: host(params[i][a:b])  # noqa: E731
    rng = np.random.default_rng(0)
    for r in (3, world - 1):
        master = torch.empty(lay.shard, device="cuda")
        zs.zs_pack_shard(table, world, r, master)
        torch.cuda.synchronize()
        lo, hi = r * lay.shard, (r + 1) * lay.shard
        starts = [lo, hi - 4096] + [o - 2048 for o in lay.offsets if lo < o < hi]
        starts += [int(x) for x in rng.integers(lo, hi - 4096, size=16)]
        for f0 in starts:
            f0 = max(lo, min(f0, hi - 4096))
            want = olayout.flat_window(fetch, numels, f0, f0 + 4096)
            got = host(master[f0 - lo:f0 - lo + 4096])
            assert np.array_equal(bits32(got), bits32(want)), (r, f0)
        del master
    del params, table
    torch.cuda.empty_cache()
