"""The update captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

Every entry point is asynchronous on the caller's stream and neither allocates
nor synchronizes, so a whole update can be captured once and replayed without
per-launch host overhead (what a launch-bound shard such as Tiny needs). Each
replay is checked bitwise against the same calls made eagerly on a separate
copy of the state, with fresh contributions copied into the captured input
buffers and eager work and synchronizations between replays. Kernel arguments
are fixed at capture, the AdamW step number included, so both sides use one
step number throughout.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from _gpu import bits32, device_rows, device_state, host, hparams

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32)) if a.dtype == torch.float32 else \
        torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else \
        torch.equal(a, b)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("world,dtype", [(8, "bf16"), (64, "bf16"), (4, "f32")])
def test_graph_replay_of_the_clipped_update(world, dtype):
    n, hp, step, max_norm = 262144 + 7, hparams(), 3, 0.01
    rows = device_rows(8100 + world, world, n, dtype)
    gs = device_state(8200 + world, n)
    es = tuple(t.clone() for t in gs)

    def bufs():
        return dict(g=torch.empty(n, device="cuda"), ss=torch.empty(1, device="cuda", dtype=torch.float64),
                    ws=torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8),
                    coef=torch.empty(1, device="cuda"), slot=torch.empty(n, device="cuda", dtype=torch.bfloat16))

    gb, eb = bufs(), bufs()

    def update(state, b):
        zs.zs_reduce_grads(rows, b["g"], sumsq_out=b["ss"], workspace=b["ws"])
        zs.zs_clip_coefficient(b["ss"], max_norm, b["coef"])
        zs.zs_adamw_step(*state, b["g"], step=step, grad_scale=b["coef"], bf16_out=b["slot"], **hp)

    graph = _capture(lambda: update(gs, gb))
    # the capture's warm-up ran once on the graph side: bring the eager side level
    update(es, eb)
    torch.cuda.synchronize()
    for x, y in zip(gs, es):
        assert _same(x, y)
    for it in range(4):
        for r, fresh in zip(rows, device_rows(8300 + 10 * it, world, n, dtype)):
            r.copy_(fresh)
        update(es, eb)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(gs, es):
            assert _same(x, y), f"replay {it}"
        for k in ("g", "ss", "coef", "slot"):
            assert _same(gb[k], eb[k]), f"replay {it}: {k}"
        assert float(eb["coef"].item()) < 1.0  # the clip is active: max_norm is below the norm


@pytest.mark.parametrize("world", [8, 64])  # the one-wave and the rank-major 8-wave shape
def test_graph_replay_of_the_single_pass(world):
    n, hp, step = 1_000_003, hparams(), 2
    rows = device_rows(8400, world, n, "bf16")
    gs = device_state(8401, n)
    es = tuple(t.clone() for t in gs)
    gslot = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    eslot = torch.empty_like(gslot)
    graph = _capture(lambda: zs.zs_sharded_step(rows, *gs, step=step, bf16_out=gslot, **hp))
    zs.zs_sharded_step(rows, *es, step=step, bf16_out=eslot, **hp)
    for it in range(4):
        for r, fresh in zip(rows, device_rows(8500 + 10 * world + it, world, n, "bf16")):
            r.copy_(fresh)
        zs.zs_sharded_step(rows, *es, step=step, bf16_out=eslot, **hp)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(gs, es):
            assert _same(x, y), f"replay {it}"
        assert _same(gslot, eslot)
    assert np.isfinite(bits32(host(gs[0])).view(np.float32)).all()
