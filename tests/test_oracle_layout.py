"""Pins of the oracle's flatten / pad / shard / pack / copy-out.

Brute force on every small (T, N): the flat buffer is rebuilt one element at a
time by walking the parameters, and each rank's shard by counting elements.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import layout
from synth import shapes


def _brute_flat(params, world, align=1):
    elems = []
    for p in params:
        for x in np.asarray(p).ravel(order="C"):
            elems.append(x)
    t = len(elems)
    s = 0  # the smallest multiple of align whose N copies hold every element
    while s * world < t or s % align:
        s += 1
    while len(elems) < s * world:
        elems.append(0.0)
    return np.array(elems, dtype=np.float32), s


def _lists_up_to(total_max):
    rng = np.random.default_rng(7)
    yield []
    yield [0]
    yield [1]
    for t in range(1, total_max + 1):
        # a few random splits of t into 1..5 parts (zero-size parts included)
        for _ in range(3):
            k = int(rng.integers(1, 6))
            cuts = sorted(rng.integers(0, t + 1, size=k - 1).tolist())
            parts = [b - a for a, b in zip([0] + cuts, cuts + [t])]
            yield parts


def test_brute_force_small():
    count = 0
    for numels in _lists_up_to(64):
        params = [np.arange(1, n + 1, dtype=np.float32) * (i + 1) * 1000 + np.float32(0.5)
                  for i, n in enumerate(numels)]
        for world in range(1, 10):
            want_flat, want_s = _brute_flat(params, world)
            lay = layout.flat_layout(numels, world)
            assert lay.total == sum(numels)
            assert lay.shard == want_s and lay.padded == want_s * world
            assert 0 <= lay.pad < world or (lay.total == 0 and lay.pad == 0)
            flat = layout.flatten(params, world, dtype=np.float32) if params else np.zeros(0, np.float32)
            assert np.array_equal(flat.view(np.uint32), want_flat.view(np.uint32))
            # offsets: parameter i begins where i-1 ended
            run = 0
            for off, n in zip(lay.offsets, numels):
                assert off == run
                run += n
            if flat.size:
                shards = [layout.shard_of(flat, world, r) for r in range(world)]
                for r, sh in enumerate(shards):
                    assert np.array_equal(sh, want_flat[r * want_s:(r + 1) * want_s])
                assert np.array_equal(np.concatenate(shards), flat)
                outs = layout.copy_out(flat, [(n,) for n in numels])
                for o, p in zip(outs, params):
                    assert np.array_equal(o, p)
            count += 1
    assert count > 500


def test_tiny_shard_is_param():
    shp = shapes.tiny()
    params = [np.full(s, i + 1, dtype=np.float32) for i, (_, s) in enumerate(shp)]
    for r in range(4):
        master, m, v = layout.pack_shard(params, 4, r)
        assert np.array_equal(master, params[r].ravel())
        assert not m.any() and not v.any()


def test_tiny_ragged_layout_and_pad():
    numels = shapes.numels(shapes.tiny_ragged())
    lay = layout.flat_layout(numels, 4)
    assert (lay.total, lay.padded, lay.shard, lay.pad) == (166, 168, 42, 2)
    assert lay.offsets == (0, 15, 22, 165)
    params = [np.arange(n, dtype=np.float32) + 1 for n in numels]
    m3, _, _ = layout.pack_shard(params, 4, 3)
    # last two elements of the last shard are the zero pad, bitwise +0
    assert m3[-2:].view(np.uint32).tolist() == [0, 0]
    assert m3[-3] == 1.0  # the single element of parameter d


@pytest.mark.parametrize("name,world,total,shard,pad", [
    ("gpt2", 8, 124_439_808, 15_554_976, 0),
    ("gpt2", 7, 124_439_808, 17_777_116, 4),
    ("gpt2", 5, 124_439_808, 24_887_962, 2),
    ("llama8b", 8, 8_030_261_248, 1_003_782_656, 0),
    ("70b", 64, 70_553_706_496, 1_102_401_664, 0),
    ("7p5b", 64, 7_500_000_000, 117_187_500, 0),
    ("tiny", 4, 1_048_576, 262_144, 0),
])
def test_config_arithmetic(name, world, total, shard, pad):
    numels = shapes.numels(shapes.WORKLOADS[name][0]())
    lay = layout.flat_layout(numels, world)
    assert (lay.total, lay.shard, lay.pad) == (total, shard, pad)


def test_block_sizes():
    assert sum(shapes.numels(shapes.llama3_8b_block())) == 218_112_000
    assert sum(shapes.numels(shapes.llama_70b_block())) == 855_654_400
    assert len(shapes.gpt2_small()) == 148
    assert len(shapes.llama3_8b()) == 291
    assert len(shapes.llama_70b()) == 723


def test_pack_bf16_source_is_exact_upcast():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    master, _, _ = layout.pack_shard([bits], 1, 0)
    assert master.view(np.uint32).tolist() == [int(b) << 16 for b in bits]


def test_multidim_params_flatten_row_major():
    # A tensor of shape (a, b, c) enters the flat buffer with its last index
    # varying fastest: element [i, j, k] sits at off + (i*b + j)*c + k. Written
    # with explicit index arithmetic, and checked against torch's flatten of a
    # contiguous tensor.
    rng = np.random.default_rng(11)
    shp = [(2, 3), (4,), (1, 2, 5), (3, 1), ()]
    params = [rng.standard_normal(s).astype(np.float32) for s in shp]
    world = 4
    flat = layout.flatten(params, world, dtype=np.float32)
    lay = layout.flat_layout([p.size for p in params], world)
    p0, p2, p3 = params[0], params[2], params[3]
    for i in range(2):
        for j in range(3):
            assert flat[lay.offsets[0] + i * 3 + j] == p0[i, j]
    for j in range(2):
        for k in range(5):
            assert flat[lay.offsets[2] + j * 5 + k] == p2[0, j, k]
    for i in range(3):
        assert flat[lay.offsets[3] + i] == p3[i, 0]
    assert flat[lay.offsets[4]] == params[4]
    want = torch.cat([torch.from_numpy(p).reshape(-1) for p in params]).numpy()
    assert np.array_equal(flat[:lay.total], want)
    assert not flat[lay.total:].any()
    outs = layout.copy_out(flat, shp)
    for o, p in zip(outs, params):
        assert o.shape == p.shape and np.array_equal(o, p)
    master, _, _ = layout.pack_shard(params, world, 1)
    assert np.array_equal(master, want[lay.shard:2 * lay.shard])


def test_copy_out_shapes_and_pad_dropped():
    shp = [(2, 3), (4,), (1, 1, 5)]
    gathered = np.arange(16, dtype=np.float32)  # 15 elements + 1 pad
    outs = layout.copy_out(gathered, shp)
    assert [o.shape for o in outs] == shp
    assert outs[2].ravel().tolist() == list(range(10, 15))


def test_brute_force_small_with_aligned_slices():
    # S rounded up to a multiple of align: found by counting, the padding at
    # the tail, the parameter offsets and real elements those of align = 1
    for numels in list(_lists_up_to(40))[::3]:
        params = [np.arange(1, n + 1, dtype=np.float32) * (i + 1) * 1000 + np.float32(0.5)
                  for i, n in enumerate(numels)]
        for world in range(1, 7):
            base = layout.flat_layout(numels, world)
            for align in (1, 2, 3, 8, 64):
                want_flat, want_s = _brute_flat(params, world, align)
                lay = layout.flat_layout(numels, world, align)
                assert lay.shard == want_s and lay.padded == want_s * world
                assert lay.offsets == base.offsets and lay.total == base.total
                assert base.shard <= lay.shard < base.shard + align
                if not params:
                    continue
                flat = layout.flatten(params, world, dtype=np.float32, align=align)
                assert np.array_equal(flat.view(np.uint32), want_flat.view(np.uint32))
                for r in range(world):
                    master, m, v = layout.pack_shard(params, world, r, align)
                    assert np.array_equal(master, want_flat[r * want_s:(r + 1) * want_s])
                    assert not m.any() and not v.any()
                outs = layout.copy_out(flat, [(n,) for n in numels])
                for o, p in zip(outs, params):
                    assert np.array_equal(o, p)


def test_aligned_slices_by_hand():
    # six elements over three ranks: S = 2 by the pages' rule; with slices
    # rounded up to 4 elements the ranks hold [1 2 3 4], [5 6 0 0], [0 0 0 0]
    flat = layout.flatten([np.array([1, 2, 3, 4, 5, 6], np.float32)], 3, align=4)
    assert [layout.shard_of(flat, 3, r).tolist() for r in range(3)] == [[1, 2, 3, 4], [5, 6, 0, 0], [0, 0, 0, 0]]
    lay = layout.flat_layout([6], 3, 4)
    assert (lay.shard, lay.padded, lay.pad) == (4, 12, 6)
    # a slice that is already a multiple keeps its size
    assert layout.flat_layout([128], 2, 64).shard == 64


def test_errors():
    with pytest.raises(ValueError):
        layout.flat_layout([3], 2, 0)
    with pytest.raises(ValueError):
        layout.flat_layout([3], 0)
    with pytest.raises(ValueError):
        layout.flat_layout([3, -1], 2)
    with pytest.raises(ValueError):
        layout.shard_of(np.zeros(8, np.float32), 4, 4)
    with pytest.raises(ValueError):
        layout.shard_of(np.zeros(7, np.float32), 4, 0)
    with pytest.raises(ValueError):
        layout.copy_out(np.zeros(3, np.float32), [(4,)])


def test_contiguous_assignment_matches_illustration():
    # Latent Atlas FSDP s5.1: six flattened elements over three GPUs -> [p1,p2], [p3,p4], [p5,p6]
    flat = layout.flatten([np.array([1, 2, 3, 4, 5, 6], np.float32)], 3)
    assert [layout.shard_of(flat, 3, r).tolist() for r in range(3)] == [[1, 2], [3, 4], [5, 6]]
    # and for every (n, N) below 20 the shards partition the padded buffer in order
    for n, w in itertools.product(range(1, 20), range(1, 8)):
        fl = layout.flatten([np.arange(n, dtype=np.float32)], w)
        assert np.array_equal(np.concatenate([layout.shard_of(fl, w, r) for r in range(w)]), fl)


def test_flat_window_equals_slices_of_flatten():
    rng = np.random.default_rng(5)
    for _ in range(50):
        numels = rng.integers(0, 30, size=int(rng.integers(1, 8))).tolist()
        params = [rng.standard_normal(n).astype(np.float32) for n in numels]
        world = int(rng.integers(1, 9))
        flat = layout.flatten(params, world, dtype=np.float32)
        for _ in range(10):
            f0 = int(rng.integers(0, flat.size + 1))
            f1 = int(rng.integers(f0, flat.size + 1))
            win = layout.flat_window(lambda i, a, b: params[i][a:b], numels, f0, f1)
            assert np.array_equal(win.view(np.uint32), flat[f0:f1].view(np.uint32))
