"""bench.py's command-line contract on the host (no GPU needed for these paths)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120,
                          env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
    r = _run("--gpus", "8", "--steps", "3", "--warmup", "1")
    assert r.returncode == 2


def test_multi_rank_launch_is_refused():
    r = _run(env={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("7p5b", "llama8b", "70b", "gpt2", "tiny"):
        assert w in r.stdout
