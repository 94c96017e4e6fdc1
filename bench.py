#!/usr/bin/env python3
"""Benchmark of one rank's sharded ZeRO/FSDP update on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 7p5b|llama8b|70b|gpt2|tiny]

A step is the rank's shard update: the mean of N bf16 gradient contributions,
fused AdamW on the fp32 master/m/v shard, and the bf16 copy into the rank's
slot of the all-gather buffer -- one launch of the single-pass kernel
(zs_sharded_step). Inputs are synthetic and resident in HBM before timing.
Reported value: shard elements updated per second (Gelem/s).

The 70B shard (fp32 contributions, 64 x 4.4 GB of rows) does not fit in HBM
whole: it is updated in 8 equal chunks, one launch each, with one chunk's worth
of rows (35 GB) serving every chunk; a step is the 8 launches.

Also measured (in "parts"): the same update as two launches (reduce, then AdamW
with the fused cast), each kernel alone, the clipped update (reduce with its sum
of squares, clip coefficient, AdamW with the gradient scale), fp32 gradient
accumulation in the ZeRO-2 and ZeRO-1 orders, the unshard copy-out of one
decoder block (flat and dim-0 sharded), GPT-2's dim-0 copy-out at N=5 (most
pieces off the 16-byte grid), the dim-0 pack of that block, the
pack of the shard, the step replayed from a captured HIP graph, and the same
update composed from PyTorch's own ops (rank adds, fused AdamW, copy-cast) as a
library reference. The JSON line carries the roofline of
the dominant kernel (HIP-event time on the launch stream) and the CPU oracle
timed on a bounded sample of the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="7p5b", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true", help="time only the step")
    ap.add_argument("--cpu-windows", type=int, default=24, help="2^20-element windows for the oracle timing")
    ap.add_argument("--cpu-threads", type=int, default=16, help="threads for the pooled oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="wall time of the pooled oracle timing")
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

    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flatparameter_amd as zs
    from synth import gen, shapes

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    zs.load()  # fails loudly when libzs.so is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    wl = WORKLOADS[args.workload]
    numels = shapes.numels(getattr(shapes, wl["shapes"])())
    world, rank = wl["world"], wl["rank"]
    _, total, padded, S = zs.zs_flat_layout(numels, world)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wl["wd"])

    # ---- inputs, resident in HBM before any timing
    row_dtype = torch.float32 if wl.get("rows") == "f32" else torch.bfloat16
    row_bytes = 4 if row_dtype == torch.float32 else 2
    csize = -(-S // wl.get("chunks", 1))
    ranges = [(a, min(S, a + csize)) for a in range(0, S, csize)]
    g0 = gen.device_generator(1000 + sorted(WORKLOADS).index(args.workload), dev)
    rows = [gen.device_normal(g0, csize, gen.GRAD_SIGMA, row_dtype, dev) for _ in range(world)]
    theta = gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    if len(ranges) == 1:
        gather = torch.empty(padded, device=dev, dtype=torch.bfloat16)
        slot = gather[rank * S:(rank + 1) * S]
    else:  # the 70B gather buffer (141 GB) is not needed to time the rank's slot
        slot = torch.empty(S, device=dev, dtype=torch.bfloat16)
    gbuf = torch.empty(S, device=dev)
    torch.cuda.synchronize()

    def rows_for(a, b):
        return rows if b - a == csize else [r[:b - a] for r in rows]

    # bit-identical host copies of the oracle's sample (taken before any update)
    win = 1 << 20
    nwin = max(1, min(args.cpu_windows, csize // win)) if not args.no_cpu_baseline else 0
    rng = np.random.default_rng(0)
    starts = sorted(int(x) for x in rng.choice(max(1, csize // win), size=nwin, replace=False)) if nwin else []
    cpu_inputs = []
    for s0 in starts:
        a, b = s0 * win, min(csize, s0 * win + win)
        if row_dtype == torch.bfloat16:
            r_h = np.stack([r[a:b].view(torch.int16).cpu().numpy().view(np.uint16) for r in rows])
        else:
            r_h = np.stack([r[a:b].cpu().numpy() for r in rows])
        cpu_inputs.append((r_h, theta[a:b].cpu().numpy(), m[a:b].cpu().numpy(), v[a:b].cpu().numpy()))

    step_no = [0]

    # zs_sharded_step per range, with its arguments marshalled once (on the
    # stream current when the plans are made)
    def make_plans():
        return [zs.ShardedStep(rows_for(a, b), theta[a:b], m[a:b], v[a:b], bf16_out=slot[a:b], **hp)
                for a, b in ranges]

    plans = make_plans()
    # A shard whose working set is near the 256 MB Infinity Cache (GPT-2: 0.65 GB)
    # steps round-robin over independent copies of its inputs, so that no step
    # finds the previous step's bytes still cached.
    rotation = [plans]
    for k in range(1, wl.get("rotate", 1)):
        rk = [gen.device_normal(g0, csize, gen.GRAD_SIGMA, row_dtype, dev) for _ in range(world)]
        tk = gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)
        mk, vk = torch.zeros(S, device=dev), torch.zeros(S, device=dev)
        sk = torch.empty(S, device=dev, dtype=torch.bfloat16)
        rotation.append([zs.ShardedStep(rk, tk, mk, vk, bf16_out=sk, **hp)])

    def fused_step(_i):
        step_no[0] += 1
        for plan in rotation[step_no[0] % len(rotation)]:
            plan(step_no[0])

    if args.calibrate_copy:
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # ---- the step: warmup, then exactly K timed steps between synchronisations;
    # an event between steps gives the per-step spread
    for i in range(args.warmup):
        fused_step(i)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for i in range(args.steps):
        fused_step(i)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_step = marks[0].elapsed_time(marks[-1]) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    spread = dict(median=round(per_step[len(per_step) // 2], 5), min=round(per_step[0], 5),
                  max=round(per_step[-1], 5)) if per_step else None
    gelem = S / (ms_step * 1e-3) / 1e9

    n_rows_bytes = row_bytes * world
    fused_bpe = n_rows_bytes + 26          # rows + read theta,m,v + write theta,m,v + bf16
    reduce_bpe = n_rows_bytes + 4          # rows + write g
    adamw_bpe = 30                         # read g,theta,m,v + write theta,m,v + bf16
    cast_bpe = 6
    achieved = fused_bpe * S / (ms_step * 1e-3) / 1e9
    kernel_name = "k_fused"
    src_hash = source_hash(kernel_name)
    traffic = read_traffic(args.workload, kernel_name, src_hash)

    parts = {}
    copy_gbs = None
    runtime_copy_gbs = None
    if not args.no_parts and not args.calibrate_copy:
        # practical copy ceilings, 2 GiB each way: the library's own streaming copy
        # (zs_copy_out of a one-parameter unit) and the HIP runtime's copy kernel
        src = torch.ones(1 << 30, device=dev, dtype=torch.bfloat16)
        dst = torch.empty_like(src)
        one = zs.ParamTable([dst])
        t_copy = event_time_ms(lambda i: zs.zs_copy_out(src, one), 10, stream)
        copy_gbs = 2 * src.numel() * 2 / (t_copy * 1e-3) / 1e9
        t_copy = event_time_ms(lambda i: dst.copy_(src), 10, stream)
        runtime_copy_gbs = 2 * src.numel() * 2 / (t_copy * 1e-3) / 1e9
        del src, dst, one
    if not args.no_parts:
        iters = max(10, args.steps)

        def reduce_call(i):
            for a, b in ranges:
                zs.zs_reduce_grads(rows_for(a, b), gbuf[a:b])

        t_reduce = event_time_ms(reduce_call, iters, stream)

        def adamw_call(i):
            step_no[0] += 1
            for a, b in ranges:
                zs.zs_adamw_step(theta[a:b], m[a:b], v[a:b], gbuf[a:b], step=step_no[0],
                                 bf16_out=slot[a:b], **hp)

        t_adamw = event_time_ms(adamw_call, iters, stream)
        t_cast = event_time_ms(lambda i: zs.zs_cast_for_gather(theta, slot), iters, stream)
        parts["two_call_step"] = dict(ms=t_reduce + t_adamw, gelem_s=S / ((t_reduce + t_adamw) * 1e-3) / 1e9,
                                      bytes_per_elem=reduce_bpe + adamw_bpe)
        for name, t, bpe in (("reduce", t_reduce, reduce_bpe), ("adamw_cast", t_adamw, adamw_bpe),
                             ("cast", t_cast, cast_bpe), ("fused_step", ms_step, fused_bpe)):
            gbs = bpe * S / (t * 1e-3) / 1e9
            parts[name] = dict(ms=round(t, 5), bytes_per_elem=bpe, gb_s=round(gbs, 1),
                               frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))

        def put(name, t, bpe, elems=S):
            gbs = bpe * elems / (t * 1e-3) / 1e9
            parts[name] = dict(ms=round(t, 5), elems=elems, bytes_per_elem=bpe, gb_s=round(gbs, 1),
                               frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))

        # the step captured once in a HIP graph and replayed: no host launch work
        # per step (what decides the launch-bound Tiny shard)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for plan in make_plans():
                plan(1)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for plan in make_plans():  # bound to the capture stream
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
            parts["torch_composed_step"] = dict(
                ms=round(t_torch, 5), gelem_s=round(S / (t_torch * 1e-3) / 1e9, 3),
                fused_step_speedup=round(t_torch / ms_step, 3))
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

        t_rs = event_time_ms(reduce_sumsq_call, iters, stream)
        put("reduce_sumsq", t_rs, reduce_bpe)

        def clipped_call(i):
            step_no[0] += 1
            reduce_sumsq_call(i)
            zs.zs_clip_coefficient(partials, 1.0, coef)
            for a, b in ranges:
                zs.zs_adamw_step(theta[a:b], m[a:b], v[a:b], gbuf[a:b], step=step_no[0],
                                 grad_scale=coef, bf16_out=slot[a:b], **hp)

        put("clipped_step", event_time_ms(clipped_call, iters, stream), reduce_bpe + adamw_bpe)

        # fp32 gradient accumulation over micro-batches. ZeRO-2 order: every
        # micro-batch's N contributions are reduced and added into the fp32 shard
        # (gbuf serves as the accumulator). ZeRO-1 order: each rank adds its whole
        # local bf16 gradient into a full-size fp32 buffer; timed on S elements of it.
        def accum_call(i):
            for a, b in ranges:
                zs.zs_accumulate_grads(rows_for(a, b), gbuf[a:b], scale=0.25)

        put("accumulate_zero2", event_time_ms(accum_call, iters, stream), n_rows_bytes + 8)
        local = rows[0][:min(csize, S)]
        lacc = gbuf[:local.numel()]
        put("accumulate_zero1_local", event_time_ms(lambda i: zs.zs_accumulate_local(local, lacc), iters,
                                                    stream), row_bytes + 8, local.numel())
        del gbuf, ws, partials, coef, lacc

        # unshard copy-out of one decoder block: Llama-3-8B's (218,112,000 elements), or
        # the 70B model's (855,654,400) for that workload
        big = args.workload == "70b"
        blk = shapes.llama_70b_block() if big else shapes.llama3_8b_block()
        blk_name, blk_world = ("70b_block", 64) if big else ("llama8b_block", 8)
        bn = shapes.numels(blk)
        gathered_blk = gen.device_normal(g0, sum(bn), 1.0, torch.bfloat16, dev)
        dst = [torch.empty(s, device=dev, dtype=torch.bfloat16) for _, s in blk]
        table = zs.ParamTable(dst)
        t_co = event_time_ms(lambda i: zs.zs_copy_out(gathered_blk, table), 10, stream)
        gbs = 4 * sum(bn) / (t_co * 1e-3) / 1e9
        parts[f"copy_out_{blk_name}"] = dict(ms=round(t_co, 5), elems=sum(bn), bytes_per_elem=4,
                                               gb_s=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        if big:
            # with reshard_after_forward every one of the 80 blocks is unsharded
            # twice per step (forward and backward): the step's copy-out time
            parts["copy_out_70b_per_step_ms"] = round(t_co * 160, 3)
        # the same block under per-parameter dim-0 sharding (a scatter from the N rank
        # regions of the gather buffer)
        dtable = zs.Dim0Table(dst, blk_world)
        gathered_d0 = gen.device_normal(g0, blk_world * dtable.local_total, 1.0, torch.bfloat16, dev)
        t_cd = event_time_ms(lambda i: zs.zs_copy_out_dim0(gathered_d0, dtable), 10, stream)
        gbs = 4 * sum(bn) / (t_cd * 1e-3) / 1e9
        parts[f"copy_out_dim0_{blk_name}_n{blk_world}"] = dict(
            ms=round(t_cd, 5), elems=sum(bn), bytes_per_elem=4, gb_s=round(gbs, 1),
            frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        del gathered_blk, gathered_d0, dst, table, dtable
        # GPT-2's list under dim-0 sharding at N=5: odd-sized bias and norm chunks
        # put most pieces off the 16-byte grid (the realigning copy path)
        g2 = shapes.gpt2_small()
        g2n = shapes.numels(g2)
        dst2 = [torch.empty(s, device=dev, dtype=torch.bfloat16) for _, s in g2]
        dtab2 = zs.Dim0Table(dst2, 5)
        gathered_g2 = gen.device_normal(g0, 5 * dtab2.local_total, 1.0, torch.bfloat16, dev)
        t_g2 = event_time_ms(lambda i: zs.zs_copy_out_dim0(gathered_g2, dtab2), 10, stream)
        gbs = 4 * sum(g2n) / (t_g2 * 1e-3) / 1e9
        parts["copy_out_dim0_gpt2_n5_misaligned"] = dict(
            ms=round(t_g2, 5), elems=sum(g2n), bytes_per_elem=4, gb_s=round(gbs, 1),
            frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        del dst2, dtab2, gathered_g2
        # dim-0 pack of the last rank's shard of the same block from fp32 parameters
        src32 = [gen.device_normal(g0, shapes.numel(s), gen.THETA_SIGMA, None, dev).reshape(s) for _, s in blk]
        ptab = zs.Dim0Table(src32, blk_world)
        L = ptab.local_total
        pm, pmm, pvv = (torch.empty(L, device=dev) for _ in range(3))
        t_pd = event_time_ms(lambda i: zs.zs_pack_shard_dim0(ptab, blk_world - 1, pm, pmm, pvv), 10, stream)
        put(f"pack_dim0_{blk_name}_n{blk_world}", t_pd, 16, L)
        del src32, ptab, pm, pmm, pvv

        # pack of this shard from per-parameter fp32 tensors (one-time setup work);
        # a single 7.5e9-element parameter, or the 70B list (282 GB of fp32
        # parameters), is represented by the rank's slice of it
        if args.workload in ("7p5b", "70b"):
            src = [gen.device_normal(g0, S, gen.THETA_SIGMA, None, dev)]
            ptable, pworld, prank = zs.ParamTable(src), 1, 0
        else:
            src = [gen.device_normal(g0, n, gen.THETA_SIGMA, None, dev) for n in numels]
            ptable, pworld, prank = zs.ParamTable(src), world, rank
        t_pack = event_time_ms(lambda i: zs.zs_pack_shard(ptable, pworld, prank, theta, m, v), 5, stream)
        gbs = 16 * S / (t_pack * 1e-3) / 1e9
        parts["pack_shard"] = dict(ms=round(t_pack, 5), bytes_per_elem=16, gb_s=round(gbs, 1),
                                   frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))
        del src, ptable
        torch.cuda.synchronize()

    # ---- CPU oracle on a bounded sample of the same inputs: one pass on one
    # thread, then repeated passes spread over the host's cores (NumPy releases
    # the GIL inside its array loops, so a thread pool runs them in parallel)
    cpu = None
    if cpu_inputs:
        from concurrent.futures import ThreadPoolExecutor

        from oracle import adamw as oadamw
        from oracle import step as ostep

        hpo = oadamw.HParams(**hp)

        def one(win_in):
            r_h, th_h, m_h, v_h = win_in
            ostep.sharded_step(r_h, th_h, m_h, v_h, 1, hpo)
            return th_h.size

        w0 = time.perf_counter()
        done1 = sum(one(x) for x in cpu_inputs)
        wall1 = time.perf_counter() - w0
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        c0, w0 = time.process_time(), time.perf_counter()
        done, passes = 0, 0
        with ThreadPoolExecutor(max_workers=threads) as ex:
            while passes < 1 or time.perf_counter() - w0 < args.cpu_seconds:
                done += sum(ex.map(one, cpu_inputs))
                passes += 1
        wall = time.perf_counter() - w0
        cpu_s = time.process_time() - c0
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
        except OSError:
            pass
        cpu = {"value": round(done / wall / 1e9, 6), "unit": "Gelem/s",
               "cores": max(1, round(cpu_s / wall)), "kind": "oracle",
               "sample": f"{len(cpu_inputs)} windows of {win} shard elements x {world} "
                         f"{'fp32' if row_bytes == 4 else 'bf16'} rows "
                         f"(the GPU's own inputs), fp64 NumPy oracle: exact mean, AdamW, bf16 cast; "
                         f"{passes} passes over a pool of {threads} threads, {wall:.1f} s wall, "
                         f"{cpu_s:.1f} s of CPU time",
               "single_thread_value": round(done1 / wall1 / 1e9, 6),
               "cpu_model": model}

    out = {
        "metric": METRIC,
        "value": round(gelem, 4),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl["desc"],
            "shard_elems": S,
            "world": world,
            "rank": rank,
            "contributions": "fp32" if row_bytes == 4 else "bf16",
            "launches_per_step": len(ranges),
            "step": "mean of N contributions + AdamW (fp32 master/m/v) + bf16 cast, one pass",
            "adamw": hp,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_elem": fused_bpe,
            "traffic": traffic,
            "copy_ceiling_gb_s": round(copy_gbs, 1) if copy_gbs else None,
            "frac_of_copy_ceiling": round(achieved / copy_gbs, 4) if copy_gbs else None,
            "runtime_copy_gb_s": round(runtime_copy_gbs, 1) if runtime_copy_gbs else None,
        },
        "cpu_baseline": cpu,
        "parts": parts,
        "source_hash": src_hash,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
