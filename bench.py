#!/usr/bin/env python3
"""Benchmark of one rank's sharded ZeRO/FSDP update on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 7p5b|llama8b|70b|gpt2|tiny]

A step is the rank's shard update: the mean of N bf16 gradient contributions,
fused AdamW on the fp32 master/m/v shard, and the bf16 copy into the rank's
slot of the all-gather buffer -- one launch of the single-pass kernel
(zs_sharded_step). Inputs are synthetic and resident in HBM before timing.
Reported value: shard elements updated per second (Gelem/s).

Before the W counted warm-up steps the device is settled: the step runs for at
least --settle-ms of wall time (measured on MI355X, the first 20 steps after a
cold start run 3-6% slower than the steady state, whatever W is). The JSON
line reports the settle steps; the timed region is exactly K steps.

The 70B shard (fp32 contributions, 64 x 4.4 GB of rows) does not fit in HBM
whole: it is updated in 8 chunks of 137,800,448 elements (the last one 1,680
shorter: chunk boundaries on 256-element multiples, so that every launch's
fp32 state starts on a 128-byte line), one launch each, with one chunk's
worth of rows (35 GB) serving every chunk; a step is the 8 launches.

Also measured (in "parts"): the same update as two launches (reduce, then AdamW
with the fused cast), each kernel alone, the clipped update (reduce with its sum
of squares, clip coefficient, AdamW with the gradient scale), fp32 gradient
accumulation in the ZeRO-2 and ZeRO-1 orders, the unshard copy-out of one
decoder block (flat and dim-0 sharded), GPT-2's dim-0 copy-out at N=5 (most
pieces off the 16-byte grid), the dim-0 pack of that block, the
pack of the shard, the step replayed from a captured HIP graph, and the same
update composed from PyTorch's own ops (rank adds, fused AdamW, copy-cast) as a
library reference. The single pass and the two calls are also timed in
alternating rounds, which is what their ratio ("fused_step_speedup") is taken
from. With the default 7.5B workload, the second target shard -- Llama-3-8B at
N=8 -- is set up right after the 7.5B step is timed, with both shards held at
once (about 75 GB), and its single pass timed the same way ("llama8b_step",
with its own roofline). The JSON line
carries the roofline of the dominant kernel (HIP-event time on the launch
stream) and the CPU oracle timed on a bounded sample of the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published figure
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "fsdp_sharded_optimizer_flatparameter_amd", "csrc")

METRIC = "shard update Gelem/s and achieved HBM GB/s (% of peak), 1 MI355X"

WORKLOADS = {
    "7p5b": dict(shapes="flat_7p5b", world=64, rank=63, wd=0.1,
                 desc="7.5B flat parameters, N=64 simulated ranks, rank 63's shard"),
    "llama8b": dict(shapes="llama3_8b", world=8, rank=7, wd=0.01,
                    desc="Llama-3-8B parameter list, N=8 simulated ranks, rank 7's shard"),
    "70b": dict(shapes="llama_70b", world=64, rank=63, wd=0.01, rows="f32", chunks=8,
                desc="70B parameter list (Llama-3 70B shapes), N=64 simulated ranks, rank 63's shard, "
                     "fp32 contributions, 8 chunks"),
    "gpt2": dict(shapes="gpt2_small", world=8, rank=7, wd=0.01, rotate=3,
                 desc="GPT-2-small parameter list, N=8 simulated ranks, rank 7's shard "
                      "(3 input sets in rotation)"),
    "tiny": dict(shapes="tiny", world=4, rank=3, wd=0.01,
                 desc="4 x 512x512 parameters, N=4 simulated ranks, rank 3's shard"),
}

# CPU sample: whole shards for the small workloads, a window of this many shard
# elements for the large ones (elements per second do not depend on the size
# beyond the last-level cache)
CPU_WINDOW = 1 << 26
CPU_CHUNK = 1 << 22      # elements per oracle call (bounds its temporaries)
CPU_MAX_WORKERS = 16     # the host share of one GPU


# Sources that define each timed kernel and its launch shape; counter-derived
# traffic is reported only while these, and the device compile flags, are
# unchanged since the counters were taken.
KERNEL_SOURCES = {
    "k_fused": ("csrc/fused.hip", "csrc/zs_device.hpp", "csrc/zs_launch.hpp", "csrc/tuning.cpp"),
}


def source_hash(kernel: str) -> str:
    from fsdp_sharded_optimizer_flatparameter_amd import build as zsbuild

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(os.path.dirname(CSRC), name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    flags = [f for f in (*zsbuild.COMMON, *zsbuild.DEVICE) if not f.startswith("-I")]  # no paths
    h.update(" ".join([zsbuild.ARCH, *flags]).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken from the current kernel sources; None otherwise."""
    path = os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src_hash or vals.get("kernel") != kernel:
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def event_time_ms(fn, iters: int, stream, warmup: int = 2) -> float:
    """Average ms per call of fn over `iters` calls after `warmup` untimed ones,
    HIP events on `stream`."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        fn(-1 - i)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def alternating_ms(fns: dict, iters: int, stream, rounds: int = 5) -> dict:
    """Median ms per call of each fn, timed in `rounds` rounds that take every
    fn in turn (iters calls each), so that a slow drift of the device's speed
    over the run weighs on all of them alike."""
    for fn in fns.values():
        for i in range(2):
            fn(-1 - i)
    times = {k: [] for k in fns}
    for _ in range(rounds):
        for k, fn in fns.items():
            times[k].append(event_time_ms(fn, iters, stream, warmup=0))
    return {k: sorted(t)[len(t) // 2] for k, t in times.items()}


def settle(step, seconds: float, min_steps: int = 0) -> int:
    """Run `step` until `seconds` of wall time have passed and at least
    `min_steps` steps have run (synchronising every few steps); returns the
    number of steps run."""
    import torch

    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds or n < min_steps:
        for _ in range(4):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def timed_steps(step, stream, warmup: int, steps: int):
    """W untimed steps, then exactly K steps between synchronisations, with an
    event between steps for the per-step spread; returns (ms per step, spread)."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        step(i)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / steps
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    spread = dict(median=round(per[len(per) // 2], 5), min=round(per[0], 5),
                  max=round(per[-1], 5)) if per else None
    return ms, spread


def gbs_entry(ms: float, bpe: int, elems: int, **extra) -> dict:
    gbs = bpe * elems / (ms * 1e-3) / 1e9
    return dict(ms=round(ms, 5), elems=elems, bytes_per_elem=bpe, gb_s=round(gbs, 1),
                frac_of_peak=round(gbs / PEAK_HBM_GBS, 4), **extra)


# ---------------------------------------------------------------- CPU oracle leg

def cpu_model() -> str:
    """The host CPU as the machine reports it: lscpu's model name, with the
    family / model / stepping numbers from /proc/cpuinfo (a virtual machine may
    report only a brand string such as "AMD EPYC")."""
    name = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        name = next((ln.split(":", 1)[1].strip() for ln in out.splitlines() if ln.startswith("Model name:")), None)
    except (OSError, subprocess.SubprocessError):
        pass
    ids = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if not ln.strip():
                    break  # the first processor's block
                k, _, v = ln.partition(":")
                ids[k.strip()] = v.strip()
    except OSError:
        pass
    name = name or ids.get("model name", "unknown")
    nums = [f"{k} {ids[k]}" for k in ("cpu family", "model", "stepping") if k in ids]
    return f"{name} ({', '.join(nums)})" if nums else name


def cpu_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, CPU_MAX_WORKERS))


def _cpu_worker(conn):
    """Oracle worker process: receives one contiguous chunk of the sample, then
    times the oracle's fp32-emulation update over it (ascending-rank fp32 sum and
    one division by N, AdamW in fp64 from the fp32 state, bf16 cast) on request."""
    data = None
    while True:
        msg = conn.recv()
        if msg[0] == "data":
            data = msg[1:]
            conn.send(("ready", data[1].size))
        elif msg[0] == "run":
            from oracle import adamw as oadamw
            from oracle import step as ostep

            rows, th, m, v, hp = data
            hpo = oadamw.HParams(**hp)
            t0 = time.perf_counter()
            for c0 in range(0, th.size, CPU_CHUNK):
                c1 = min(th.size, c0 + CPU_CHUNK)
                ostep.sharded_step(rows[:, c0:c1], th[c0:c1], m[c0:c1], v[c0:c1], 1, hpo, exact_mean=False)
            conn.send(("done", th.size, time.perf_counter() - t0))
        else:
            conn.close()
            return


class CpuSample:
    """Oracle processes (started before the GPU is touched), each holding one
    contiguous chunk of a bounded, bit-identical host copy of the step's inputs."""

    def __init__(self):
        import multiprocessing as mp

        ctx = mp.get_context("spawn")
        self.workers = cpu_workers()
        self.conns, self.procs = [], []
        for _ in range(self.workers):
            parent, child = ctx.Pipe()
            p = ctx.Process(target=_cpu_worker, args=(child,), daemon=True)
            p.start()
            child.close()
            self.conns.append(parent)
            self.procs.append(p)
        self.n = 0

    def load(self, rows, theta, m, v, a: int, n: int, hp: dict):
        import numpy as np
        import torch

        self.world, self.n = len(rows), n
        self.row_code = "bf16" if rows[0].dtype == torch.bfloat16 else "f32"
        per = -(-n // self.workers)
        self.chunks = [(c, min(n, c + per)) for c in range(0, n, per)]
        for conn, (c0, c1) in zip(self.conns, self.chunks):
            lo, hi = a + c0, a + c1
            if self.row_code == "bf16":
                r = np.stack([x[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16) for x in rows])
            else:
                r = np.stack([x[lo:hi].cpu().numpy() for x in rows])
            conn.send(("data", r, theta[lo:hi].cpu().numpy(), m[lo:hi].cpu().numpy(),
                       v[lo:hi].cpu().numpy(), dict(hp)))
            del r
        for conn in self.conns[:len(self.chunks)]:
            assert conn.recv()[0] == "ready"

    def measure(self) -> dict:
        live = self.conns[:len(self.chunks)]
        live[0].send(("run",))  # one process alone
        _, n1, t1 = live[0].recv()
        t0 = time.perf_counter()
        for conn in live:
            conn.send(("run",))
        done = sum(conn.recv()[1] for conn in live)
        tw = time.perf_counter() - t0
        w = len(live)
        return {"value": round(done / tw / 1e9, 6), "unit": "Gelem/s", "cores": w, "kind": "oracle",
                "sample": f"{self.n} consecutive shard elements x {self.world} {self.row_code} rows (the GPU's "
                          f"own inputs, copied to the host before the first update); the oracle's "
                          f"fp32-emulation path: ascending-rank fp32 running sum and one division by N, AdamW "
                          f"in fp64 from the fp32 state, bf16 cast; {w} contiguous chunks, one per process, "
                          f"{tw:.2f} s wall",
                "single_process_value": round(n1 / t1 / 1e9, 6),
                "single_process_sample": f"the first chunk ({n1} elements) in one process, {t1:.2f} s",
                "cpu_model": cpu_model()}

    def close(self):
        for conn in self.conns:
            try:
                conn.send(("exit",))
            except (OSError, BrokenPipeError):
                pass
        for p in self.procs:
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()


# ---------------------------------------------------------------- the step

def make_shard(name: str, dev):
    """Inputs of one workload's shard update, resident in HBM, and its step."""
    import torch

    import fsdp_sharded_optimizer_flatparameter_amd as zs
    from synth import gen, shapes

    wl = WORKLOADS[name]
    numels = shapes.numels(getattr(shapes, wl["shapes"])())
    world, rank = wl["world"], wl["rank"]
    _, total, padded, S = zs.zs_flat_layout(numels, world)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wl["wd"])
    row_dtype = torch.float32 if wl.get("rows") == "f32" else torch.bfloat16
    csize = -(-S // wl.get("chunks", 1))
    if wl.get("chunks", 1) > 1:
        # chunk boundaries on 1 KiB of fp32 state (256 elements), so that every
        # launch's theta, m and v start on the 128-byte line grid; the last chunk
        # is the shorter one
        csize = -(-csize // 256) * 256
    ranges = [(a, min(S, a + csize)) for a in range(0, S, csize)]
    g0 = gen.device_generator(1000 + sorted(WORKLOADS).index(name), dev)
    rows = [gen.device_normal(g0, csize, gen.GRAD_SIGMA, row_dtype, dev) for _ in range(world)]
    theta = gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    if len(ranges) == 1:
        gather = torch.empty(padded, device=dev, dtype=torch.bfloat16)
        slot = gather[rank * S:(rank + 1) * S]
    else:  # the 70B gather buffer (141 GB) is not needed to time the rank's slot
        slot = torch.empty(S, device=dev, dtype=torch.bfloat16)
    sh = dict(name=name, wl=wl, numels=numels, world=world, rank=rank, S=S, padded=padded, hp=hp,
              row_dtype=row_dtype, row_bytes=4 if row_dtype == torch.float32 else 2, csize=csize,
              ranges=ranges, g0=g0, rows=rows, theta=theta, m=m, v=v, slot=slot, step_no=[0])

    def rows_for(a, b):
        return rows if b - a == csize else [r[:b - a] for r in rows]

    sh["rows_for"] = rows_for

    # zs_sharded_step per range, with its arguments marshalled once (on the
    # stream current when the plans are made)
    def make_plans():
        return [zs.ShardedStep(rows_for(a, b), theta[a:b], m[a:b], v[a:b], bf16_out=slot[a:b], **hp)
                for a, b in ranges]

    sh["make_plans"] = make_plans
    # A shard whose working set is near the 256 MB Infinity Cache (GPT-2: 0.65 GB)
    # steps round-robin over independent copies of its inputs, so that no step
    # finds the previous step's bytes still cached.
    rotation = [make_plans()]
    for _ in range(1, wl.get("rotate", 1)):
        rk = [gen.device_normal(g0, csize, gen.GRAD_SIGMA, row_dtype, dev) for _ in range(world)]
        tk = gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)
        mk, vk = torch.zeros(S, device=dev), torch.zeros(S, device=dev)
        sk = torch.empty(S, device=dev, dtype=torch.bfloat16)
        rotation.append([zs.ShardedStep(rk, tk, mk, vk, bf16_out=sk, **hp)])
    sh["rotation"] = rotation

    def fused_step(_i):
        sh["step_no"][0] += 1
        for plan in rotation[sh["step_no"][0] % len(rotation)]:
            plan(sh["step_no"][0])

    sh["step"] = fused_step
    sh["fused_bpe"] = sh["row_bytes"] * world + 26  # rows + read theta,m,v + write theta,m,v + bf16
    torch.cuda.synchronize()
    return sh


def measure_parts(sh, dev, stream, iters: int, parts: dict) -> None:
    import torch

    import fsdp_sharded_optimizer_flatparameter_amd as zs
    from synth import gen, shapes

    S, world, hp, ranges, rows = sh["S"], sh["world"], sh["hp"], sh["ranges"], sh["rows"]
    theta, m, v, slot, step_no, rows_for = sh["theta"], sh["m"], sh["v"], sh["slot"], sh["step_no"], sh["rows_for"]
    g0, csize = sh["g0"], sh["csize"]
    n_rows_bytes = sh["row_bytes"] * world
    reduce_bpe, adamw_bpe, cast_bpe = n_rows_bytes + 4, 30, 6
    gbuf = torch.empty(S, device=dev)

    def reduce_call(i):
        for a, b in ranges:
            zs.zs_reduce_grads(rows_for(a, b), gbuf[a:b])

    t_reduce = event_time_ms(reduce_call, iters, stream)

    def adamw_call(i):
        step_no[0] += 1
        for a, b in ranges:
            zs.zs_adamw_step(theta[a:b], m[a:b], v[a:b], gbuf[a:b], step=step_no[0], bf16_out=slot[a:b], **hp)

    t_adamw = event_time_ms(adamw_call, iters, stream)
    t_cast = event_time_ms(lambda i: zs.zs_cast_for_gather(theta, slot), iters, stream)

    # the single pass against the two calls, timed in alternating rounds
    def two_call(i):
        reduce_call(i)
        adamw_call(i)

    alt = alternating_ms({"fused": sh["step"], "two_call": two_call}, max(5, iters // 2), stream)
    parts["two_call_step"] = dict(ms=round(alt["two_call"], 5),
                                  gelem_s=round(S / (alt["two_call"] * 1e-3) / 1e9, 3),
                                  bytes_per_elem=reduce_bpe + adamw_bpe,
                                  fused_step_ms_alternating=round(alt["fused"], 5),
                                  fused_step_speedup=round(alt["two_call"] / alt["fused"], 4),
                                  sum_of_parts_ms=round(t_reduce + t_adamw, 5))
    parts["reduce"] = gbs_entry(t_reduce, reduce_bpe, S)
    parts["adamw_cast"] = gbs_entry(t_adamw, adamw_bpe, S)
    parts["cast"] = gbs_entry(t_cast, cast_bpe, S)

    # the step captured once in a HIP graph and replayed: no host launch work
    # per step (what decides the launch-bound Tiny shard)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for plan in sh["make_plans"]():
            plan(1)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for plan in sh["make_plans"]():  # bound to the capture stream
            plan(1)
    t_graph = event_time_ms(lambda i: graph.replay(), iters, stream)
    parts["graph_replayed_step"] = dict(ms=round(t_graph, 5), gelem_s=round(S / (t_graph * 1e-3) / 1e9, 3))
    del graph

    # the same update composed from PyTorch's own ops, as a library reference:
    # in-place fp32 adds of the N contributions in rank order, one division,
    # PyTorch's fused AdamW, and a copy-cast into the slot
    if len(ranges) == 1:
        p = torch.nn.Parameter(theta.clone())
        p.grad = torch.empty_like(p)
        opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                weight_decay=hp["weight_decay"], fused=True)

        def torch_step(i):
            gg = p.grad
            gg.copy_(rows[0])
            for r in rows[1:]:
                gg.add_(r)
            gg.div_(world)
            opt.step()
            slot.copy_(p.detach())

        t_torch = event_time_ms(torch_step, max(5, iters // 4), stream)
        parts["torch_composed_step"] = dict(ms=round(t_torch, 5), gelem_s=round(S / (t_torch * 1e-3) / 1e9, 3))
        del p, opt

    # global-norm clipping: the reduce also returns the fp64 sum of squares of its
    # output, the clip coefficient combines the shards' partials (here the N
    # simulated ranks' copies of this one), and AdamW takes it as a gradient scale
    ws = torch.empty(zs.zs_workspace_bytes(csize), device=dev, dtype=torch.uint8)
    partials = torch.zeros(world, device=dev, dtype=torch.float64)
    coef = torch.empty(1, device=dev)

    def reduce_sumsq_call(i):
        for j, (a, b) in enumerate(ranges):
            zs.zs_reduce_grads(rows_for(a, b), gbuf[a:b], sumsq_out=partials[j:j + 1], workspace=ws)

    parts["reduce_sumsq"] = gbs_entry(event_time_ms(reduce_sumsq_call, iters, stream), reduce_bpe, S)

    def clipped_call(i):
        step_no[0] += 1
        reduce_sumsq_call(i)
        zs.zs_clip_coefficient(partials, 1.0, coef)
        for a, b in ranges:
            zs.zs_adamw_step(theta[a:b], m[a:b], v[a:b], gbuf[a:b], step=step_no[0],
                             grad_scale=coef, bf16_out=slot[a:b], **hp)

    parts["clipped_step"] = gbs_entry(event_time_ms(clipped_call, iters, stream), reduce_bpe + adamw_bpe, S)

    # fp32 gradient accumulation over micro-batches. ZeRO-2 order: every
    # micro-batch's N contributions are reduced and added into the fp32 shard
    # (gbuf serves as the accumulator). ZeRO-1 order: each rank adds its whole
    # local bf16 gradient into a full-size fp32 buffer; timed on S elements of it.
    def accum_call(i):
        for a, b in ranges:
            zs.zs_accumulate_grads(rows_for(a, b), gbuf[a:b], scale=0.25)

    parts["accumulate_zero2"] = gbs_entry(event_time_ms(accum_call, iters, stream), n_rows_bytes + 8, S)
    local = rows[0][:min(csize, S)]
    lacc = gbuf[:local.numel()]
    parts["accumulate_zero1_local"] = gbs_entry(
        event_time_ms(lambda i: zs.zs_accumulate_local(local, lacc), iters, stream),
        sh["row_bytes"] + 8, local.numel())
    del gbuf, ws, partials, coef, lacc

    # unshard copy-out of one decoder block: Llama-3-8B's (218,112,000 elements), or
    # the 70B model's (855,654,400) for that workload
    big = sh["name"] == "70b"
    blk = shapes.llama_70b_block() if big else shapes.llama3_8b_block()
    blk_name, blk_world = ("70b_block", 64) if big else ("llama8b_block", 8)
    bn = shapes.numels(blk)
    gathered_blk = gen.device_normal(g0, sum(bn), 1.0, torch.bfloat16, dev)
    dst = [torch.empty(s, device=dev, dtype=torch.bfloat16) for _, s in blk]
    table = zs.ParamTable(dst)
    t_co = event_time_ms(lambda i: zs.zs_copy_out(gathered_blk, table), 10, stream)
    parts[f"copy_out_{blk_name}"] = gbs_entry(t_co, 4, sum(bn))
    if big:
        # with reshard_after_forward every one of the 80 blocks is unsharded
        # twice per step (forward and backward): the step's copy-out time
        parts["copy_out_70b_per_step_ms"] = round(t_co * 160, 3)
    # the same block under per-parameter dim-0 sharding (a scatter from the N rank
    # regions of the gather buffer)
    dtable = zs.Dim0Table(dst, blk_world)
    gathered_d0 = gen.device_normal(g0, blk_world * dtable.local_total, 1.0, torch.bfloat16, dev)
    t_cd = event_time_ms(lambda i: zs.zs_copy_out_dim0(gathered_d0, dtable), 10, stream)
    parts[f"copy_out_dim0_{blk_name}_n{blk_world}"] = gbs_entry(t_cd, 4, sum(bn))
    del gathered_blk, gathered_d0, dst, table, dtable
    # GPT-2's list under dim-0 sharding at N=5: odd-sized bias and norm chunks
    # put most pieces off the 16-byte grid (the realigning copy path)
    g2 = shapes.gpt2_small()
    g2n = shapes.numels(g2)
    dst2 = [torch.empty(s, device=dev, dtype=torch.bfloat16) for _, s in g2]
    dtab2 = zs.Dim0Table(dst2, 5)
    gathered_g2 = gen.device_normal(g0, 5 * dtab2.local_total, 1.0, torch.bfloat16, dev)
    t_g2 = event_time_ms(lambda i: zs.zs_copy_out_dim0(gathered_g2, dtab2), 10, stream)
    parts["copy_out_dim0_gpt2_n5_misaligned"] = gbs_entry(t_g2, 4, sum(g2n))
    del dst2, dtab2, gathered_g2
    # dim-0 pack of the last rank's shard of the same block from fp32 parameters
    src32 = [gen.device_normal(g0, shapes.numel(s), gen.THETA_SIGMA, None, dev).reshape(s) for _, s in blk]
    ptab = zs.Dim0Table(src32, blk_world)
    L = ptab.local_total
    pm, pmm, pvv = (torch.empty(L, device=dev) for _ in range(3))
    t_pd = event_time_ms(lambda i: zs.zs_pack_shard_dim0(ptab, blk_world - 1, pm, pmm, pvv), 10, stream)
    parts[f"pack_dim0_{blk_name}_n{blk_world}"] = gbs_entry(t_pd, 16, L)
    del src32, ptab, pm, pmm, pvv

    # pack of this shard from per-parameter fp32 tensors (one-time setup work);
    # a single 7.5e9-element parameter, or the 70B list (282 GB of fp32
    # parameters), is represented by the rank's slice of it
    if sh["name"] in ("7p5b", "70b"):
        src = [gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)]
        ptable, pworld, prank = zs.ParamTable(src), 1, 0
    else:
        src = [gen.device_normal(g0, n, gen.THETA_SIGMA, None, dev) for n in sh["numels"]]
        ptable, pworld, prank = zs.ParamTable(src), world, sh["rank"]
    t_pack = event_time_ms(lambda i: zs.zs_pack_shard(ptable, pworld, prank, theta, m, v), 5, stream)
    parts["pack_shard"] = gbs_entry(t_pack, 16, S)
    del src, ptable
    torch.cuda.synchronize()


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="7p5b", choices=sorted(WORKLOADS))
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time the step runs before the W warm-up steps (device settle)")
    ap.add_argument("--settle-steps", type=int, default=40,
                    help="the least number of steps the settle runs, whatever its wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true", help="time only the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before timing, run one plain 1 GiB device copy (torch copy_) as the known-size "
                         "reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard update; --gpus {args.gpus} is not supported "
              "(the update of each rank is independent -- run one process per GPU).", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 given)", file=sys.stderr)
        return 2

    # the oracle's process pool starts before anything touches the GPU
    cpu = CpuSample() if not args.no_cpu_baseline else None
    try:
        return run(args, cpu)
    finally:
        if cpu is not None:
            cpu.close()


def run(args, cpu) -> int:
    import torch

    import fsdp_sharded_optimizer_flatparameter_amd as zs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    zs.load()  # fails loudly when libzs.so is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    sh = make_shard(args.workload, dev)
    S, world, hp = sh["S"], sh["world"], sh["hp"]

    # bit-identical host copy of the oracle's sample, taken before any update
    if cpu is not None:
        n_cpu = min(sh["csize"], CPU_WINDOW)
        a_cpu = 0 if n_cpu == sh["csize"] else (sh["csize"] - n_cpu) // 2
        cpu.load(sh["rows"], sh["theta"], sh["m"], sh["v"], a_cpu, n_cpu, hp)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # ---- the step: settle, W warm-up steps, then exactly K timed steps
    settle_steps = settle(sh["step"], args.settle_ms * 1e-3, args.settle_steps if args.settle_ms > 0 else 0)
    ms_step, spread = timed_steps(sh["step"], stream, args.warmup, args.steps)
    gelem = S / (ms_step * 1e-3) / 1e9
    fused_bpe = sh["fused_bpe"]
    achieved = fused_bpe * S / (ms_step * 1e-3) / 1e9
    kernel_name = "k_fused"
    src_hash = source_hash(kernel_name)
    traffic = read_traffic(args.workload, kernel_name, src_hash)

    # ---- the second target shard: Llama-3-8B at N=8, its single pass timed the
    # same way (settle, W warm-up steps, K steps), right after the first so that
    # both run on the device in the same state (the 7.5B shard stays allocated:
    # together they hold about 75 GB)
    llama_entry = None
    if args.workload == "7p5b" and not args.no_parts and not args.calibrate_copy:
        ll = make_shard("llama8b", dev)
        settle(ll["step"], args.settle_ms * 1e-3, args.settle_steps if args.settle_ms > 0 else 0)
        ms_ll, spread_ll = timed_steps(ll["step"], stream, args.warmup, args.steps)
        llama_entry = gbs_entry(ms_ll, ll["fused_bpe"], ll["S"], kernel=kernel_name,
                                workload=ll["wl"]["desc"],
                                gelem_s=round(ll["S"] / (ms_ll * 1e-3) / 1e9, 3),
                                step_ms=spread_ll)
        del ll
        torch.cuda.empty_cache()

    parts = {}
    library_copy_gbs = runtime_copy_gbs = None
    if not args.no_parts and not args.calibrate_copy:
        # streaming copies of 2 GiB each way: the library's own (zs_copy_out of a
        # one-parameter unit) and the HIP runtime's copy kernel
        src = torch.ones(1 << 30, device=dev, dtype=torch.bfloat16)
        dst = torch.empty_like(src)
        one = zs.ParamTable([dst])
        t_copy = event_time_ms(lambda i: zs.zs_copy_out(src, one), 10, stream)
        library_copy_gbs = 2 * src.numel() * 2 / (t_copy * 1e-3) / 1e9
        t_copy = event_time_ms(lambda i: dst.copy_(src), 10, stream)
        runtime_copy_gbs = 2 * src.numel() * 2 / (t_copy * 1e-3) / 1e9
        del src, dst, one
        parts["fused_step"] = gbs_entry(ms_step, fused_bpe, S)
        if llama_entry is not None:
            parts["llama8b_step"] = llama_entry
        measure_parts(sh, dev, stream, max(10, args.steps), parts)
        if "torch_composed_step" in parts:
            parts["torch_composed_step"]["fused_step_speedup"] = round(parts["torch_composed_step"]["ms"] / ms_step, 3)

    config = {
        "workload": sh["wl"]["desc"],
        "shard_elems": S,
        "world": world,
        "rank": sh["rank"],
        "contributions": "fp32" if sh["row_bytes"] == 4 else "bf16",
        "launches_per_step": len(sh["ranges"]),
        "step": "mean of N contributions + AdamW (fp32 master/m/v) + bf16 cast, one pass",
        "adamw": hp,
    }
    del sh

    cpu_out = cpu.measure() if cpu is not None else None

    out = {
        "metric": METRIC,
        "value": round(gelem, 4),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 5),
        "step_ms": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_elem": fused_bpe,
            "traffic": traffic,
            "library_copy_gb_s": round(library_copy_gbs, 1) if library_copy_gbs else None,
            "runtime_copy_gb_s": round(runtime_copy_gbs, 1) if runtime_copy_gbs else None,
        },
        "cpu_baseline": cpu_out,
        "parts": parts,
        "source_hash": src_hash,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
