"""Pins of the oracle's per-parameter dim-0 sharding (FSDP2 Shard(0))."""
import itertools

import numpy as np
import pytest
import torch

from oracle import dim0
from synth import shapes


def _torch_chunk_shard(p, world, rank):
    # torch.chunk on dim 0, each rank's chunk padded with zero rows to the first chunk's size
    t = torch.from_numpy(np.asarray(p))
    if t.dim() == 0:
        t = t.reshape(1)
    chunks = torch.chunk(t, world, dim=0)
    rows0 = chunks[0].shape[0]
    mine = chunks[rank] if rank < len(chunks) else t[:0]
    pad = torch.zeros((rows0 - mine.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype)
    return torch.cat([mine, pad]).reshape(-1).numpy()


def test_matches_torch_chunk_on_small_shapes():
    rng = np.random.default_rng(0)
    count = 0
    for d0, d1, world in itertools.product(range(0, 12), (1, 3), range(1, 9)):
        shp = (d0, d1) if d1 > 1 else (d0,)
        p = rng.standard_normal(shp).astype(np.float32)
        for r in range(world):
            got = dim0.shard_dim0([p], world, r)
            assert np.array_equal(got, _torch_chunk_shard(p, world, r)), (shp, world, r)
            count += 1
    assert count > 500


def test_multi_parameter_shard_and_roundtrip():
    rng = np.random.default_rng(1)
    for _ in range(40):
        k = int(rng.integers(1, 6))
        shps = []
        for _ in range(k):
            nd = int(rng.integers(0, 4))
            shps.append(tuple(int(x) for x in rng.integers(0, 7, size=nd)))
        params = [rng.standard_normal(s).astype(np.float32) if s else np.float32(rng.standard_normal()) for s in shps]
        for world in (1, 2, 3, 5, 8):
            lay = dim0.dim0_layout(shps, world)
            shards = [dim0.shard_dim0(params, world, r) for r in range(world)]
            # a rank's shard is its torch.chunk pieces concatenated in order
            for r in range(world):
                want = np.concatenate([_torch_chunk_shard(p, world, r) for p in params]) if params else np.zeros(0)
                assert np.array_equal(shards[r], want.astype(np.float32))
                assert shards[r].size == lay.local_total
            back = dim0.copy_out_dim0(np.concatenate(shards), shps, world)
            for b, p in zip(back, params):
                assert np.array_equal(b, np.asarray(p).reshape(b.shape))


def test_gpt2_token_embedding_at_eight_ranks():
    # ceil(50257 / 8) = 6283 rows per rank; the last rank pads 7 rows
    lay = dim0.dim0_layout([(50257, 768)], 8)
    assert lay.chunk == (6283 * 768,)
    assert dim0.valid(50257 * 768, lay.chunk[0], 7) == (50257 - 7 * 6283) * 768 == 6276 * 768
    assert 8 * 6283 - 50257 == 7


def test_tiny_ragged_layout():
    lay = dim0.dim0_layout([s for _, s in shapes.tiny_ragged()], 4)
    assert lay.chunk == (5, 2, 39, 1) and lay.local_offsets == (0, 5, 7, 46) and lay.local_total == 47
    # per-parameter padding: 4 * 47 = 188 elements hold the unit's 166
    assert 4 * lay.local_total - 166 == 22


def test_llama_block_divides_evenly():
    lay = dim0.dim0_layout([s for _, s in shapes.llama3_8b_block()], 8)
    assert 8 * lay.local_total == 218_112_000


def test_errors():
    with pytest.raises(ValueError):
        dim0.dim0_layout([(3,)], 0)
    with pytest.raises(ValueError):
        dim0.copy_out_dim0(np.zeros(3, np.float32), [(4,)], 2)
