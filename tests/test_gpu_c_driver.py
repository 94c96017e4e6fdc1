"""The sharded update driven through the C ABI by a standalone program (no Python
or PyTorch in the process that calls the library), checked against the oracle.

tests/c/zs_driver reads the inputs this test writes, runs zs_reduce_grads (with
the sum of squares), zs_adamw_step, zs_sharded_step, zs_copy_out and
zs_pack_shard on its own device buffers, and writes every output back.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import adamw as oadamw
from oracle import bf16 as obf16
from oracle import layout as olayout
from oracle import reduce as oreduce
from synth import gen
from _gpu import bits32, check_adamw, check_bf16, check_mean, hparams

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "zs_driver")


def _run(tmp_path, world, dtype, numels, step, seed):
    n = sum(numels)
    hp = hparams()
    rows = gen.host_grad_rows(seed, world, n, dtype)
    th = gen.host_normal(seed + 1, n, gen.THETA_SIGMA)
    m = gen.host_normal(seed + 2, n, 1e-4)
    v = np.abs(gen.host_normal(seed + 3, n, 1e-6))
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([world, 1 if dtype == "bf16" else 0], np.int32).tobytes())
        f.write(np.array([n, step], np.int64).tobytes())
        f.write(np.array([hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]],
                         np.float64).tobytes())
        f.write(np.array([len(numels)], np.int32).tobytes())
        f.write(np.array(numels, np.int64).tobytes())
        f.write(np.ascontiguousarray(rows).tobytes())
        for a in (th, m, v):
            f.write(a.astype(np.float32).tobytes())
    print(f"zs_driver world={world} dtype={dtype} n={n} params={len(numels)}", flush=True)
    res = subprocess.run([DRIVER, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    raw = open(dst, "rb").read()
    pos = 0

    def take(dt, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dt, count=count, offset=pos)
        pos += a.nbytes
        return a

    out = dict(g=take(np.float32, n), sumsq=take(np.float64, 1)[0],
               two=tuple(take(np.float32, n) for _ in range(3)), two_bf16=take(np.uint16, n),
               one=tuple(take(np.float32, n) for _ in range(3)), one_bf16=take(np.uint16, n),
               copied=take(np.uint16, n), packed=take(np.float32, n))
    assert pos == len(raw)
    return rows, (th, m, v), hp, out


@pytest.mark.parametrize("world,dtype,numels", [
    (4, "bf16", [3, 5 * 7, 1000, 4096, 11]),       # ragged parameter offsets, n = 5145
    (8, "bf16", [262144, 7, 65536 + 1]),           # several tiles and a ragged tail
    (64, "bf16", [100000, 31]),
    (8, "f32", [70000, 3]),
])
def test_c_driver_matches_oracle(tmp_path, world, dtype, numels):
    step = 3
    rows, state, hp, out = _run(tmp_path, world, dtype, numels, step, seed=7000 + world)
    # reduce: bit-exact in the ascending-rank order, and within the bound of the exact mean
    assert np.array_equal(bits32(out["g"]), bits32(oreduce.mean_seq32(rows)))
    check_mean(out["g"], rows)
    ref = oreduce.sumsq(out["g"])
    assert abs(out["sumsq"] - ref) <= 1e-12 * ref
    # AdamW against the oracle fed the library's own gradient; bf16 of its own theta
    th_or = check_adamw(out["two"], state, out["g"], step, hp)
    check_bf16(out["two_bf16"], out["two"][0], th_or)
    # the single pass returns the same bits as the two calls
    for x, y in zip(out["one"], out["two"]):
        assert np.array_equal(bits32(x), bits32(y))
    assert np.array_equal(out["one_bf16"], out["two_bf16"])
    # copy-out of the slot into the parameters, concatenated, is the slot itself
    parts = olayout.copy_out(out["two_bf16"], [(k,) for k in numels])
    assert np.array_equal(np.concatenate([p.ravel() for p in parts]), out["copied"])
    # the world-1 pack of theta split into the parameters is theta
    want = olayout.pack_shard([state[0][o:o + k] for o, k in zip(np.cumsum([0] + numels[:-1]), numels)],
                              1, 0)[0]
    assert np.array_equal(bits32(out["packed"]), bits32(want))
    # the oracle's own sharded step agrees within tolerance end to end
    g_exact = oreduce.mean_exact(rows)
    th1, _, _ = oadamw.adamw_step(*state, g_exact, step, oadamw.HParams(**hp))
    assert np.max(np.abs(out["two"][0].astype(np.float64) - th1)) <= 1e-5 * np.max(np.abs(th1))
    assert np.array_equal(obf16.to_bf16_bits(out["two"][0]), out["two_bf16"])
