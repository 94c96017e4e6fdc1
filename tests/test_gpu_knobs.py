"""Every launch-shape knob leaves every result unchanged, bit for bit (the fp64
sum of squares to within its rounding, since it is associated per workgroup).

The knobs (ZS_* environment variables, read once per process and only when
ZS_TUNING=1 opts in) pick workgroup
sizes, staging depths, rank-chunk widths, LDS reservations and grid caps. Each
case below runs the same seeded update in a child process under one setting
(a grid cap of a few workgroups forces every kernel through its grid-stride
loop) and compares all outputs with the default setting's, bitwise: the
single pass and the two calls, the accumulation, the cast, the flat and dim-0
copy-outs (the latter with odd-sized chunks, so through the realigning copy),
the single pass into a bf16 slot on a 2-byte boundary, and the pack. The world
sizes take every default launch shape: one-wave (8; 12 with its rows in one
batch), rank-major (16, 64; 33 with a short second walk of 1 rank).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[2])
import fsdp_sharded_optimizer_flatparameter_amd as zs
from synth import gen

out = {}
hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
def h(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()
for world, dt, n in ((8, torch.bfloat16, 300_007), (64, torch.bfloat16, 70_001), (16, torch.float32, 50_003),
                     (33, torch.bfloat16, 90_007), (12, torch.bfloat16, 120_003)):
    g0 = gen.device_generator(900 + world)
    rows = [gen.device_normal(g0, n, 1e-3, dt) for _ in range(world)]
    st = [gen.device_normal(g0, n, 0.02), gen.device_normal(g0, n, 1e-4), gen.device_normal(g0, n, 1e-6).abs_()]
    two = [t.clone() for t in st]
    slot = torch.empty(n, device="cuda", dtype=torch.bfloat16)
    slot2 = torch.empty_like(slot)
    zs.zs_sharded_step(rows, *st, step=3, bf16_out=slot, **hp)
    g = torch.empty(n, device="cuda")
    ss = torch.empty(1, device="cuda", dtype=torch.float64)
    ws = torch.empty(zs.zs_workspace_bytes(n), device="cuda", dtype=torch.uint8)
    zs.zs_reduce_grads(rows, g, sumsq_out=ss, workspace=ws)
    zs.zs_adamw_step(*two, g, step=3, bf16_out=slot2, **hp)
    acc = torch.empty(n, device="cuda")
    ass = torch.empty(1, device="cuda", dtype=torch.float64)
    zs.zs_accumulate_grads(rows, acc, scale=0.5, first=True)
    zs.zs_accumulate_grads(rows, acc, scale=0.5, sumsq_out=ass, workspace=ws)
    cast = torch.empty_like(slot)
    zs.zs_cast_for_gather(st[0], cast)
    shapes = [(n // 3,), (n - n // 3 - 5,), (5,)]
    dst = [torch.empty(s, device="cuda", dtype=torch.bfloat16) for s in shapes]
    zs.zs_copy_out(slot, zs.ParamTable(dst))
    dst0 = [torch.empty(sh, device="cuda", dtype=torch.bfloat16) for sh in shapes]
    t0 = zs.Dim0Table(dst0, 5)
    gathered0 = gen.device_normal(g0, 5 * t0.local_total, 1.0, torch.bfloat16)
    zs.zs_copy_out_dim0(gathered0, t0)
    odd = torch.empty(n + 1, device="cuda", dtype=torch.bfloat16)[1:]  # a slot on a 2-byte boundary
    st_odd = [gen.device_normal(g0, n, 0.02), gen.device_normal(g0, n, 1e-4), gen.device_normal(g0, n, 1e-6).abs_()]
    zs.zs_sharded_step(rows, *st_odd, step=3, bf16_out=odd, **hp)
    master = torch.empty(-(-n // 4), device="cuda")
    srcs = [gen.device_normal(g0, s[0], 0.02) for s in shapes]
    zs.zs_pack_shard(zs.ParamTable(srcs), 4, 3, master)
    torch.cuda.synchronize()
    for k, t in (("fused", st), ("two", two)):
        for i, x in enumerate(t):
            out[f"{world}_{k}{i}"] = h(x)
    for k, t in (("slot", slot), ("slot2", slot2), ("g", g), ("acc", acc), ("cast", cast), ("master", master)):
        out[f"{world}_{k}"] = h(t)
    out[f"{world}_ss"] = ss.cpu().numpy()
    out[f"{world}_ass"] = ass.cpu().numpy()
    out[f"{world}_copied"] = np.concatenate([h(d) for d in dst])
    out[f"{world}_copied_dim0"] = np.concatenate([h(d) for d in dst0])
    out[f"{world}_odd_slot"] = h(odd)
    for i, x in enumerate(st_odd):
        out[f"{world}_odd{i}"] = h(x)
np.savez(sys.argv[1], **out)
"""

SETTINGS = [
    {},
    {"ZS_GRID_CAP": "5"},
    {"ZS_FUSED_BS": "256", "ZS_FUSED_G": "2", "ZS_RANK_CHUNK": "4"},
    {"ZS_FUSED_BS": "64", "ZS_FUSED_G": "4", "ZS_FUSED_LDS": "32768"},
    {"ZS_ACCUM_SHAPE": "1", "ZS_REDUCE_G": "4", "ZS_ADAMW_V": "4", "ZS_ADAMW_LDS": "0"},
]


def _run(tmp_path, env_over, tag):
    env = {k: v for k, v in os.environ.items() if not k.startswith("ZS_")}
    env.update(env_over)
    if env_over:
        env["ZS_TUNING"] = "1"
    path = str(tmp_path / f"{tag}.npz")
    print(f"knobs {env_over}", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD, path, ROOT], env=env, capture_output=True,
                         text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, (env_over, res.stdout[-2000:], res.stderr[-2000:])
    return dict(np.load(path))


def test_no_knob_changes_a_result(tmp_path):
    base = _run(tmp_path, SETTINGS[0], "base")
    for w in (8, 64, 16, 33, 12):  # the single pass is bitwise the two calls under the defaults
        for i in range(3):
            assert np.array_equal(base[f"{w}_fused{i}"], base[f"{w}_two{i}"])
        assert np.array_equal(base[f"{w}_slot"], base[f"{w}_slot2"])
    for k, setting in enumerate(SETTINGS[1:]):
        got = _run(tmp_path, setting, f"s{k}")
        assert got.keys() == base.keys()
        for key in base:
            if key.endswith("ss"):
                # the fp64 sum of squares is associated per workgroup: its last
                # bits follow the grid (it stays deterministic for one setting)
                assert abs(got[key][0] - base[key][0]) <= 1e-12 * base[key][0], (setting, key)
            else:
                assert np.array_equal(got[key], base[key]), (setting, key)
