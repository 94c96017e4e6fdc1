"""The sharded update driven through the C ABI by a standalone program (no Python
or PyTorch in the process that calls the library), checked against the oracle.

tests/c/zs_driver reads the inputs this test writes, runs zs_reduce_grads (with
the sum of squares), zs_adamw_step, zs_sharded_step, zs_copy_out,
zs_pack_shard, zs_cast_for_gather, zs_accumulate_grads, zs_accumulate_local,
zs_clip_coefficient and the dim-0 layout, pack and copy-out on its own device
buffers, and writes every output back.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import accumulate as oacc
from oracle import adamw as oadamw
from oracle import bf16 as obf16
from oracle import dim0 as odim0
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
               copied=take(np.uint16, n), packed=take(np.float32, n), cast=take(np.uint16, n),
               acc=take(np.float32, n), acc_ss=take(np.float64, 1)[0], local=take(np.float32, n),
               coef=take(np.float32, 1)[0], norm=take(np.float64, 1)[0])
    L = int(take(np.int64, 1)[0])
    out.update(L=L, last_shard=take(np.float32, L), unshard=take(np.uint16, n))
    assert pos == len(raw)
    return rows, (th, m, v), hp, out


@pytest.mark.parametrize("world,dtype,numels", [
    (4, "bf16", [3, 5 * 7, 1000, 4096, 11]),       # ragged parameter offsets, n = 5145
    (8, "bf16", [262144, 7, 65536 + 1]),           # several tiles and a ragged tail
    (64, "bf16", [100000, 31]),
    (8, "f32", [70000, 3]),
    (32, "f32", [140000, 5]),                      # the rank-major shape with fp32 rows
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
    # the standalone cast of the same theta'
    assert np.array_equal(out["cast"], out["two_bf16"])
    # ZeRO-2 accumulation of two micro-batches (the same rows twice, scale 1/2)
    acc_want = oacc.zero2_accumulate([rows, rows], 0.5)
    assert np.array_equal(bits32(out["acc"]), bits32(acc_want))
    assert abs(out["acc_ss"] - oreduce.sumsq(out["acc"])) <= 1e-12 * oreduce.sumsq(out["acc"])
    # ZeRO-1 local accumulation: one rank's fp32 sum of its two micro-batch gradients
    dec = oreduce.decode_rows(rows)
    local_want = (dec[0].copy() + dec[1 % world]).astype(np.float32)
    assert np.array_equal(bits32(out["local"]), bits32(local_want))
    # clipping coefficient from the accumulated gradient's sum of squares
    want_coef, want_norm = oacc.clip_coefficient([out["acc_ss"]], 1e-3)
    assert abs(out["norm"] - want_norm) <= 1e-15 * want_norm
    assert abs(float(out["coef"]) - float(want_coef)) <= np.spacing(np.float32(want_coef))
    # dim-0 sharding of the parameters taken as 1-D: the last rank's pack, and the
    # unshard of every rank's packed shard (cast to bf16) is bf16 of theta
    pieces = [state[0][o:o + k] for o, k in zip(np.cumsum([0] + numels[:-1]), numels)]
    assert out["L"] == odim0.dim0_layout([(k,) for k in numels], world).local_total
    assert np.array_equal(bits32(out["last_shard"]), bits32(odim0.shard_dim0(pieces, world, world - 1)))
    assert np.array_equal(out["unshard"], obf16.to_bf16_bits(state[0]))
