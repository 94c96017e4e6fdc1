"""The tile plans of the streaming kernels, checked on the host.

The reduce, the single pass and the ZeRO-2 accumulation hand each workgroup
the lane groups of one tile of a plan (zs_launch.hpp): one tile per `span`
groups, or, balanced, full tiles for every round of resident workgroups but
the last and the last round's groups split evenly over all of them. A tile
that overlapped another, left a gap or ran past the array would corrupt or
skip elements, so tests/c/tile_plan.cpp sweeps sizes (every size up to 700
groups, sizes around whole rounds, the 7.5B shard and the 70B chunk, 2^40
groups) against spans and slot counts and checks every tile of every plan.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "fsdp_sharded_optimizer_flatparameter_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_tile_plans_cover_every_group_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "tile_plan")
    cmd = [hipcc, "-O2", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(HERE, "c", "tile_plan.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok "), run.stdout
    assert int(run.stdout.split()[1]) > 50000
