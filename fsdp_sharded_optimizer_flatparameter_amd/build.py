"""Build libzs.so (the C-ABI library of HIP kernels) in-tree for gfx950.

    python -m fsdp_sharded_optimizer_flatparameter_amd.build [-v]

Each source is compiled by hipcc in parallel; the objects are linked into
fsdp_sharded_optimizer_flatparameter_amd/libzs.so, replaced atomically. The
standalone C-ABI test driver (tests/c/zs_driver) is linked against it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libzs.so")

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: gfx950 only. Packed-fp32 VALU ops are kept out of the generated code, and
# floating-point contraction is off: every operation rounds as written, fused
# multiply-adds appear only where the source calls fmaf/fma.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=off"]

SOURCES = ["abi.cpp", "tuning.cpp", "reduce.hip", "adamw.hip", "fused.hip", "accumulate.hip",
           "segments.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libzs)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
        if verbose:
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libzs.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    build_driver()
    return LIB


DRIVER_SRC = os.path.join(ROOT, "tests", "c", "zs_driver.cpp")
DRIVER = os.path.join(ROOT, "tests", "c", "zs_driver")


def build_driver() -> str:
    """The standalone C-ABI test driver (host code only), linked against the
    in-tree libzs.so through a path relative to the binary."""
    tmp = DRIVER + ".tmp"
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", f"-I{INCLUDE}", DRIVER_SRC, f"-L{PKG}", "-lzs",
           "-Wl,-rpath,$ORIGIN/../../fsdp_sharded_optimizer_flatparameter_amd", "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=os.path.dirname(DRIVER))
    if res.returncode != 0:
        raise RuntimeError(f"driver build failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, DRIVER)
    return DRIVER


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
