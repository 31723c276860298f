"""Benchmark of the FSDP data-parallel hot path on one MI355X.

One step = for every FSDP unit of the model, in order: all-gather +
unflatten its bf16 shards into R full-unit receivers, then the fused
reduce-scatter-average of the R bf16 gradient replicas + AdamW on the fp32
master/m/v shards + bf16 recast.  Default schedule "auto": after the
warm-up the overlap sequence (each unit's fused step enqueued together with
the next unit's gather, FSDP's prefetch: one launch per unit for units this
size, into two alternating receive buffers) and the serial one are timed
in alternating rounds on the same buffers, and the faster runs the timed
steps; the line reports the choice and both times.  Default workload: the 12-layer model of TransformerBlocks
(hidden 512, ffn 2048), one FSDP2 per-parameter unit per block, R = 8
virtual ranks in one GPU's memory (37,761,024 parameters).  Inputs are
synthetic, seeded and resident in HBM before timing starts.

Prints one JSON line: params/s of the whole step (the mean over the timed
steps, with the median and min of blocks of them), achieved algorithmic HBM
GB/s, the roofline of the step's dominant kernel from HIP events around its
launches, a plain copy of the same bytes in one launch for comparison, and
the CPU oracle timed on a bounded sample on the host.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="model12_r8")
    ap.add_argument("--schedule", choices=("auto", "serial", "prefetch", "graph", "overlap",
                                           "graph-overlap"),
                    default=None,
                    help="default auto: after the warm-up, time the overlap and the serial "
                         "sequence in alternating rounds on the same buffers and keep the "
                         "faster for the timed steps (both give the same bits); "
                         "serial: per unit gather then fused step on one stream; prefetch: "
                         "gathers on their own stream run ahead of the fused steps, into a "
                         "double receive buffer; graph: the serial sequence replayed as one "
                         "HIP graph per step; overlap: each unit's fused step shares its "
                         "launch with the next unit's gather (double receive buffer); "
                         "graph-overlap: the overlap sequence replayed as one HIP graph")
    ap.add_argument("--cycle-gib", type=float, default=4.0,
                    help="give the workload enough independent copies of its buffers that "
                         "one cycle of steps touches at least this many GiB (the 256 MB "
                         "last-level cache keeps part of a smaller cycle between steps)")
    ap.add_argument("--gathers-per-step", type=int, choices=(1, 2), default=1,
                    help="1: parameters kept from forward to backward "
                         "(reshard_after_forward=False); 2: freed after forward and "
                         "gathered again in backward (reshard_after_forward=True)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the sustained-bandwidth part of the step line (the "
                         "872M-parameter group's fused step and gather, ~40 GB of HBM)")
    ap.add_argument("--sustained-workload", default="group4096_flat_r8",
                    help="the FSDP1 (flat) workload of the sustained-bandwidth part")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--mode", choices=("step", "reshard", "accum", "ddp"), default="step",
                    help="step: the training step (default, the headline); reshard: restore "
                         "the model's sharded state at another world size; accum: a step "
                         "with --micro micro-batches accumulated in fp32; ddp: the DDP "
                         "comparator (all-reduce + AdamW on every rank's full replica)")
    ap.add_argument("--micro", type=int, default=4, help="micro-batches for --mode accum")
    ap.add_argument("--to-ranks", type=int, default=4, help="new world size for --mode reshard")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --calibrate-copy` into profiles/traffic_<workload>.json "
                         "and exit (no GPU needed)")
    args = ap.parse_args()
    if args.schedule is None:
        args.schedule = "auto"
    return args


def kernel_src_hash():
    """Hash of the sources that decide what the kernels do and how they are
    launched, comments and blank space left out (editing a comment does not
    change a kernel)."""
    import re
    h = hashlib.sha256()
    for f in ("kernels.hip", "kernels.hpp", "plan.cpp", "abi.cpp"):
        with open(os.path.join(ROOT, "fully_sharded_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


# Kernels whose traffic the counter runs summarise: key -> (kernel-name
# fragments that select their dispatches in a rocprofv3 counter CSV, what
# the kernel is).
TRAFFIC_KERNELS = {
    "fused": (("::k_fused<", "::k_fused_one<", "::k_fused_pair<"),
              "k_fused / k_fused_one / k_fused_pair (fused reduce-scatter-average + AdamW + "
              "bf16 recast, alone)"),
    "fused_gather": (("::k_fused_two_gather<", "::k_fused_gather<"),
                     "k_fused_two_gather / k_fused_gather (one unit's fused step, then the "
                     "next unit's gather, in one launch)"),
    "allreduce": (("::k_allreduce<",), "k_allreduce (DDP all-reduce-average to R receivers)"),
    "adamw": (("::k_adamw<", "::k_adamw_two<"),
              "k_adamw / k_adamw_two (AdamW + recast on an fp32 gradient)"),
    "gather": (("::k_copy<2, 16, 8, 8>",),
               "k_copy (bf16 gather + unflatten to 8 receivers, 16-byte lanes)"),
    "accumulate": (("::k_accumulate<",), "k_accumulate (fp32 gradient accumulation)"),
    "copy_pairs": (("::k_copy_pairs<4>",), "k_copy_pairs<4> (batched re-shard copy, fp32 arrays)"),
}


def traffic_path(workload, key, mode="step"):
    tag = workload if mode == "step" else f"{workload}_{mode}"
    name = f"traffic_{tag}.json" if key == "fused" else f"traffic_{tag}_{key}.json"
    return os.path.join(ROOT, "profiles", name)


def load_traffic(workload, key="fused", mode="step"):
    """Counter-measured HBM bytes per launch of a kernel, if taken on the
    current kernel sources, else None."""
    path = traffic_path(workload, key, mode)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_src_sha") != kernel_src_hash():
        return None
    return tr.get("bytes_per_launch", tr.get("fused_bytes_per_launch"))


def rows(n_rows, n, dtype, device):
    """n_rows tensors of n elements carved from one buffer, with the
    package's placement rule (fully_sharded_amd.buffers)."""
    from fully_sharded_amd.buffers import rows as carve
    return carve(n_rows, n, dtype, device)


# Timed dispatches of the --calibrate-copy leg: the last plain copies of a
# run (nothing after it launches a kernel).
CALIB_TIMED = 10


def summarise_counters(fetch_csv, write_csv, workload, mode="step"):
    """HBM bytes per launch of each kernel in TRAFFIC_KERNELS that the runs
    dispatched, from the FETCH_SIZE and WRITE_SIZE counters (KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB
    plain copy of --calibrate-copy (1 GiB read, 1 GiB written): the median
    of the run's last CALIB_TIMED copy dispatches, by dispatch id (set-up
    copies earlier in the run can be larger)."""
    import csv
    import statistics

    def load(path, counter, frags):
        sel, copy = [], []
        with open(path) as f:
            for i, r in enumerate(csv.DictReader(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                if any(fr in name for fr in frags):
                    sel.append(float(r["Counter_Value"]))
                elif "copy" in name.lower() and "fsdp" not in name:
                    order = int(r["Dispatch_Id"]) if r.get("Dispatch_Id") else i
                    copy.append((order, float(r["Counter_Value"])))
        if not copy:
            raise SystemExit(f"{path}: no calibration-copy dispatches for {counter}")
        calib = [v for _, v in sorted(copy)[-CALIB_TIMED:]]
        if max(calib) > 1.02 * min(calib):
            raise SystemExit(f"{path}: the last {len(calib)} copy dispatches differ "
                             f"({min(calib)} to {max(calib)} KiB): not the calibration copy")
        return (sum(sel) / len(sel) if sel else None), statistics.median(calib), len(sel)

    gib_kib = float(1 << 20)
    for key, (frags, desc) in TRAFFIC_KERNELS.items():
        fetch, fetch_copy, nf = load(fetch_csv, "FETCH_SIZE", frags)
        write, write_copy, nw = load(write_csv, "WRITE_SIZE", frags)
        if fetch is None or write is None:
            continue
        fs = gib_kib / fetch_copy
        ws = gib_kib / write_copy
        out = {
            "workload": workload,
            "mode": mode,
            "kernel": desc,
            "kernel_src_sha": kernel_src_hash(),
            "dispatches": {"FETCH_SIZE": nf, "WRITE_SIZE": nw},
            "fetch_kib_per_launch": fetch,
            "write_kib_per_launch": write,
            "calibration_copy_kib": {"FETCH_SIZE": fetch_copy, "WRITE_SIZE": write_copy,
                                     "true_kib_each_way": gib_kib},
            "fetch_scale": fs,
            "write_scale": ws,
            "bytes_per_launch": (fetch * fs + write * ws) * 1024.0,
        }
        with open(traffic_path(workload, key, mode), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        print(json.dumps(out))


def launches_per_step(args, units):
    """Kernel launches of one step (the graph schedule adds its one-lane
    scalar kernel)."""
    n = len(units)
    if args.schedule in ("overlap", "graph-overlap"):
        # a unit's step shares its launch with the next gather when it has
        # at most 65,536 work items; with two gathers per step the forward
        # gathers come first and the backward runs from the last unit
        paired = units[:-1] if args.gathers_per_step == 1 else units[1:]
        big = sum(1 for u in paired if len(u.plan.work_items(0)) > 65536)
        return ((args.gathers_per_step - 1) * n + 1 + (n - 1) + big + 1
                + (1 if args.schedule == "graph-overlap" else 0))
    return (args.gathers_per_step + 1) * n + (1 if args.schedule == "graph" else 0)


def setup_units(wl, dev):
    """Plans and device buffers of every unit, inputs drawn on the GPU:
    sharded fp32 master (m = v = 0), bf16 parameter, R gradient replicas."""
    import torch

    import fully_sharded_amd as F
    from fully_sharded_amd.step import Unit
    from workloads import gen
    from workloads.configs import shapes_of

    R = wl["R"]
    gdt = torch.bfloat16 if wl["grad_dtype"] == "bf16" else torch.float32
    pdt = torch.bfloat16 if wl["param_dtype"] == "bf16" else torch.float32
    plans = {}
    units = []
    for u, unit in enumerate(wl["units"]):
        shapes = tuple(shapes_of(unit))
        if shapes not in plans:
            plans[shapes] = F.Plan(list(shapes), R, wl["layout"])
            plans[shapes].prepare()
        pl = plans[shapes]
        full = gen.device_master(wl, u, list(shapes), dev)
        master, m, v, param, grads = F.unit_buffers(pl, pdt, gdt, dev)
        m.zero_()
        v.zero_()
        F.fsdp_shard_pack(pl, full, master)
        F.fsdp_shard_pack(pl, full, param)
        del full
        for r in range(R):
            grads[r].copy_(gen.device_grad(wl, 1, u, r, pl.T, dev))
        units.append(Unit(pl, master, m, v, param, grads))
    torch.cuda.synchronize()
    return plans, units


def main():
    args = parse()
    if args.counters:
        summarise_counters(args.counters[0], args.counters[1], args.workload, args.mode)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the R ranks are virtual ranks in one GPU's "
              f"memory and the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fully_sharded_amd as F
    from fully_sharded_amd.step import StepRunner, Unit, choose_schedule
    from workloads import gen
    from workloads.configs import ADAMW, WORKLOADS, shapes_of

    wl = WORKLOADS[args.workload]
    R = wl["R"]
    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    gdt = torch.bfloat16 if wl["grad_dtype"] == "bf16" else torch.float32
    pdt = torch.bfloat16 if wl["param_dtype"] == "bf16" else torch.float32

    # ---------------------------------------------------------------- set-up
    t_setup = time.perf_counter()
    plans, units = setup_units(wl, dev)
    if args.mode != "step":
        return run_mode(args, wl, plans, units)
    # A small workload would partly stay in the 256 MB last-level cache
    # (MALL) when re-run: give it independent copies of its buffers, cycled
    # step by step, so that one round touches at least --cycle-gib GiB.
    ws = sum(u.plan.T * (2 * R + 28) for u in units)
    cycle = int(args.cycle_gib * (1 << 30))
    n_copies = 1 if ws >= cycle else min(32, -(-cycle // ws))
    copies = [units] + [setup_units(wl, dev)[1] for _ in range(n_copies - 1)]
    T_max = max(p.T for p in plans.values())
    n_recv = 2 if args.schedule in ("prefetch", "overlap", "graph-overlap", "auto") else 1
    runners = []
    for cu in copies:
        recv = [rows(R, T_max, pdt, dev) for _ in range(n_recv)]
        runners.append(StepRunner(cu, ADAMW, recv, schedule=args.schedule,
                                  gathers_per_step=args.gathers_per_step))
    runner = runners[0]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    P = sum(u.plan.T for u in units)

    step_no = [0]

    def step():
        step_no[0] += 1
        runners[step_no[0] % len(runners)].step(step_no[0])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # "auto": both sequences timed on these buffers (ordinary training
    # steps, outside the timed region), the faster one kept
    schedule_choice = None
    if args.schedule == "auto":
        schedule_choice = choose_schedule(runners, step)
        args.schedule = schedule_choice["chosen"]
        schedule_choice["requested"] = "auto"

    # ----------------------------------------- timed region: the clean steps
    # K steps between two HIP events; events between blocks of them (a
    # marker each, no synchronisation) also give the median and the min of
    # the per-block step times
    bounds = step_blocks(args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(1, len(bounds)):
        for _ in range(bounds[i] - bounds[i - 1]):
            step()
        evs[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    block_ms = [evs[i - 1].elapsed_time(evs[i]) / (bounds[i] - bounds[i - 1])
                for i in range(1, len(bounds))]

    # ------------- per-kernel durations: HIP events around back-to-back runs
    # of one kernel over all units (an event between every launch would add
    # its own few microseconds to each), on the stream the kernels run on
    reps = max(5, args.steps // 4)
    hs = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * len(units))

    def fused_pass():
        step_no[0] += 1
        for _, fused in runners[step_no[0] % len(runners)].calls:
            fused(step_no[0], hs)

    gp = [0]

    def gather_pass():
        gp[0] += 1
        for gather, _ in runners[gp[0] % len(runners)].calls:
            gather(hs)

    fused_avg_ms = timed(fused_pass)
    gather_avg_ms = timed(gather_pass)
    pair_avg_ms = None
    if hasattr(runner, "pairs") and len(units) > 1:
        pp = [0]

        def pair_pass():
            pp[0] += 1
            step_no[0] += 1
            for pair in runners[pp[0] % len(runners)].pairs:
                pair(step_no[0], hs)
        pair_avg_ms = timed(pair_pass) * len(units) / (len(units) - 1)

    # the other steps of the path, each timed alone the same way: the
    # reduce-scatter-average and AdamW + recast unfused (a4, a5 + a6), and
    # the init-time pack of the fp32 master and of the cast parameter (a2)
    extra = {}
    for ri, r in enumerate(runners):
        r_units = copies[ri]
        outs = [torch.empty(u.plan.R * u.plan.S, dtype=torch.float32, device=dev)
                for u in r_units]
        fulls = [torch.empty(u.plan.T, dtype=torch.float32, device=dev).uniform_(-0.05, 0.05)
                 for u in r_units]
        extra[ri] = dict(
            rs=[F.bind_reduce_scatter_avg(u.plan, u.grads, o) for u, o in zip(r_units, outs)],
            adamw=[F.bind_adamw_shard_step(u.plan, ADAMW, o, u.master, u.m, u.v, u.param,
                                           grads_are_replicas=False)
                   for u, o in zip(r_units, outs)],
            pack=[F.bind_shard_pack(u.plan, f, u.master) for u, f in zip(r_units, fulls)],
            cast=[F.bind_shard_pack(u.plan, f, u.param) for u, f in zip(r_units, fulls)],
            keep=(outs, fulls))
    xp = [0]

    def pass_of(name, with_step=False):
        def run():
            xp[0] += 1
            step_no[0] += 1
            for call in extra[xp[0] % len(runners)][name]:
                if with_step:
                    call(step_no[0], hs)
                else:
                    call(hs)
        return run

    rs_avg_ms = timed(pass_of("rs"))
    adamw_avg_ms = timed(pass_of("adamw", with_step=True))
    pack_avg_ms = timed(pass_of("pack"))
    cast_avg_ms = timed(pass_of("cast"))
    del extra

    # algorithmic bytes (valid parameters only, padding excluded)
    ges = 2 if gdt == torch.bfloat16 else 4
    pes = 2 if pdt == torch.bfloat16 else 4
    fused_bytes_unit = [u.plan.T * (ges * R + 24 + pes) for u in units]
    gather_bytes_unit = [u.plan.T * (pes + pes * R) for u in units]
    step_bytes = sum(fused_bytes_unit) + args.gathers_per_step * sum(gather_bytes_unit)
    fused_bytes = float(np.mean(fused_bytes_unit))
    fused_gbps = fused_bytes / (fused_avg_ms * 1e-3) / 1e9
    gather_gbps = float(np.mean(gather_bytes_unit)) / (gather_avg_ms * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    kernels = {
        "fused_rs_adamw": {"avg_ms": fused_avg_ms, "bytes": fused_bytes, "gbps": fused_gbps},
        "gather_unflatten": {"avg_ms": gather_avg_ms,
                             "bytes": float(np.mean(gather_bytes_unit)), "gbps": gather_gbps},
        "timed_launches_each": reps * len(units),
    }
    Tm = float(np.mean([u.plan.T for u in units]))
    for key, ms, per_param in (("reduce_scatter_avg", rs_avg_ms, ges * R + 4),
                               ("adamw_recast", adamw_avg_ms, 4 + 24 + pes),
                               ("shard_pack_f32", pack_avg_ms, 8),
                               ("shard_pack_cast", cast_avg_ms, 4 + pes)):
        kernels[key] = {"avg_ms": ms, "bytes": Tm * per_param,
                        "gbps": Tm * per_param / (ms * 1e-3) / 1e9}
    # the roofline: the fused reduce-scatter + AdamW + recast kernel alone,
    # the step the 70% bar is set for; beside it the launch that dominates
    # the step's time as scheduled (in the overlap schedule with short steps
    # the launch holding one unit's fused step and the next unit's gather)
    roofline = roof_entry("fused", fused_bytes, fused_avg_ms, args.workload)
    roofline["target_frac"] = 0.70
    roofline["target_met"] = roofline["frac"] >= 0.70
    dominant = None
    if pair_avg_ms is not None:
        pair_bytes = float(np.mean([fused_bytes_unit[i] + gather_bytes_unit[i + 1]
                                    for i in range(len(units) - 1)]))
        # a step of more than 65,536 work items keeps its gather in a
        # second launch
        one_launch = all(len(u.plan.work_items(0)) <= 65536 for u in units[:-1])
        kernels["fused_then_gather"] = {
            "avg_ms": pair_avg_ms, "bytes": pair_bytes,
            "gbps": pair_bytes / (pair_avg_ms * 1e-3) / 1e9,
            "launches": 1 if one_launch else 2}
        if one_launch and args.schedule in ("overlap", "graph-overlap"):
            dominant = roof_entry("fused_gather", pair_bytes, pair_avg_ms, args.workload)
    plain = plain_copy(fused_bytes, args.cycle_gib, dev, hs, reps)
    # every kernel line against a plain copy of its own bytes in one launch:
    # a short launch loses its ramp and drain whatever it computes
    copies_by_size = {plain["bytes_per_launch"]: plain}
    for key, k in kernels.items():
        if isinstance(k, dict):
            size = plain_copy_bytes(k["bytes"])
            if size not in copies_by_size:
                copies_by_size[size] = plain_copy(k["bytes"], args.cycle_gib, dev, hs, reps)
            pc = copies_by_size[size]
            k["plain_copy_gbps"] = pc["achieved"]
            k["of_plain_copy"] = k["gbps"] / pc["achieved"]
    roofline["of_plain_copy"] = kernels["fused_rs_adamw"]["of_plain_copy"]
    if dominant is not None:
        dominant["of_plain_copy"] = kernels["fused_then_gather"]["of_plain_copy"]

    copy_info = calibration_copy(dev) if args.calibrate_copy else None

    # --------------- sustained bandwidth: the 872M-parameter unit group
    sustained = None
    group_sample = None
    if not args.no_sustained:
        sustained, group_sample = sustained_group(args.sustained_workload, dev, hs,
                                                  not args.no_cpu_baseline)

    # ------------------------------------------ CPU baseline: the oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(units, R, wl, args.cpu_seconds, group_sample)

    line = {
        "metric": "shard-step params/s and achieved HBM GB/s (% of peak), 12-layer R=8",
        "value": P / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_blocks": {"blocks": len(block_ms), "median": float(np.median(block_ms)),
                               "min": min(block_ms)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "units": len(units),
            "R": R,
            "layout": wl["layout"],
            "params": P,
            "param_dtype": wl["param_dtype"],
            "grad_dtype": wl["grad_dtype"],
            "state_dtype": "f32",
            "schedule": args.schedule,
            "schedule_choice": schedule_choice,
            "gathers_per_step": args.gathers_per_step,
            "launches_per_step": launches_per_step(args, units),
            "host_calls_per_step": 2 if args.schedule in ("graph", "graph-overlap")
            else len(units) * args.gathers_per_step + 1 if args.schedule == "overlap"
            else (args.gathers_per_step + 1) * len(units),
            "buffer_copies": len(runners),
            "step": "per unit: gather+unflatten to R receivers, fused RS-avg+AdamW+recast "
                    "(overlap: unit u's fused step shares its launch with unit u+1's gather)",
        },
        "hbm_gbps": step_gbps,
        "hbm_frac": step_gbps / PEAK_HBM_GBPS,
        "step_bytes": step_bytes,
        "kernels": kernels,
        "memory_ledger_per_rank": runner.memory_ledger(pes),
        "roofline": roofline,
        "roofline_dominant_launch": dominant,
        "plain_copy": plain,
        "sustained": sustained,
        "plan_layout": time_plan_layout(wl),
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
        "setup_s": setup_s,
    }
    if copy_info:
        line["copy_calibration"] = copy_info
    print(json.dumps(line), flush=True)


# What the path computes in: the reduce-scatter sums in fp32, AdamW is
# evaluated in IEEE double from the fp32 state (parameters and gradients are
# stored as bf16, the state as fp32).
DTYPE = "f32 reduce + f64 AdamW"


def calibration_copy(dev):
    """A plain 1 GiB device copy (torch's copy kernel), 3 untimed then
    CALIB_TIMED timed launches: the run's reference for the FETCH_SIZE and
    WRITE_SIZE counters (1 GiB read and 1 GiB written per launch)."""
    import torch
    stream = torch.cuda.current_stream()
    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        b.copy_(a)
    c0.record(stream)
    for _ in range(CALIB_TIMED):
        b.copy_(a)
    c1.record(stream)
    torch.cuda.synchronize()
    ms = c0.elapsed_time(c1) / CALIB_TIMED
    del a, b
    return dict(bytes=2 * n * 4, ms=ms, gbps=2 * n * 4 / (ms * 1e-3) / 1e9)


def roof_entry(key, bytes_per_launch, ms, workload, mode="step"):
    """The roofline object of one kernel: algorithmic bytes per launch over
    its average launch time (HIP events around back-to-back launches),
    against MI355X's HBM peak, with the counter-measured bytes when the
    profiles hold them for the current kernel sources."""
    gbps = bytes_per_launch / (ms * 1e-3) / 1e9
    return {"kernel": TRAFFIC_KERNELS[key][1], "bytes_per_launch": bytes_per_launch,
            "avg_ms": ms, "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
            "traffic": load_traffic(workload, key, mode)}


def sustained_group(name, dev, hs, want_sample, launches=8):
    """The sustained-bandwidth workload beside the headline: one 872M-parameter
    group of four hidden-4096 blocks as one FSDP1 FlatParameter at R = 8.
    Its fused step and its gather, each timed with HIP events around
    `launches` back-to-back launches on the stream they run on (after one
    warm-up launch each), with a plain copy of 4 GiB for comparison.  With
    want_sample, also returns host copies of a few 1 Mi-element chunks of its
    inputs for the oracle's chunk-wise leg.  Frees its buffers on return."""
    import numpy as np
    import torch

    import fully_sharded_amd as F
    from workloads.configs import ADAMW, WORKLOADS

    wl = WORKLOADS[name]
    if wl["layout"] != "flat" or len(wl["units"]) != 1:
        raise SystemExit(f"--sustained-workload {name}: needs one FSDP1 (flat) unit")
    R = wl["R"]
    pdt = torch.bfloat16 if wl["param_dtype"] == "bf16" else torch.float32
    _, units = setup_units(wl, dev)
    u = units[0]
    T = u.plan.T
    recv = rows(R, T, pdt, dev)
    fused = F.bind_adamw_shard_step(u.plan, ADAMW, u.grads, u.master, u.m, u.v, u.param)
    gather = F.bind_gather_unflatten(u.plan, u.param, recv)
    t = [0]

    def fstep():
        t[0] += 1
        fused(t[0], hs)
    fstep()
    gather(hs)
    fused_ms = _timed(fstep, launches)
    gather_ms = _timed(lambda: gather(hs), launches)
    ges = 2 if wl["grad_dtype"] == "bf16" else 4
    pes = 2 if wl["param_dtype"] == "bf16" else 4
    fb = float(T * (ges * R + 24 + pes))
    gb = float(T * (pes + pes * R))
    out = {"workload": name, "params": T, "R": R, "layout": wl["layout"],
           "launches_timed": launches}
    for key, b, ms in (("fused_rs_adamw", fb, fused_ms), ("gather_unflatten", gb, gather_ms)):
        gbps = b / (ms * 1e-3) / 1e9
        out[key] = {"avg_ms": ms, "bytes": b, "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
    out["step_ms"] = fused_ms + gather_ms
    out["step_gbps"] = (fb + gb) / (out["step_ms"] * 1e-3) / 1e9
    out["fused_rs_adamw"]["target_met"] = out["fused_rs_adamw"]["frac"] >= 0.70
    sample = None
    if want_sample:
        # chunks of 1 Mi elements at 16 places of the shard space; the
        # FlatParameter's shard element j of rank r is flat element r*S + j
        S = u.plan.S
        n = min(1 << 20, S)
        sample = {"workload": name, "R": R, "grad_dtype": wl["grad_dtype"],
                  "param_dtype": wl["param_dtype"], "chunks": []}
        for c in range(16):
            r = (5 * c) % R
            j0 = int(((c * 0.618) % 1.0) * (S - n))
            lo = r * S + j0
            hi = min(lo + n, T)
            if hi <= lo:
                continue
            sample["chunks"].append({
                "grads": [_host(g[lo:hi]) for g in u.grads],
                "master": _host(u.master[lo:hi]), "m": _host(u.m[lo:hi]),
                "v": _host(u.v[lo:hi])})
    del fused, gather, recv, units, u
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    plain = plain_copy(min(fb, 4 << 30), 4.0, dev, hs, 4)
    out["plain_copy"] = plain
    out["fused_rs_adamw"]["of_plain_copy"] = out["fused_rs_adamw"]["gbps"] / plain["achieved"]
    return out, sample


def step_blocks(steps, n_blocks=10):
    """Boundaries 0 = b_0 < b_1 < ... < b_n = steps of at most n_blocks
    near-equal blocks of timed steps."""
    n = max(1, min(n_blocks, steps))
    return [round(i * steps / n) for i in range(n + 1)]


def time_plan_layout(wl, budget_s=0.5):
    """Host time of fsdp_plan_layout for the workload's distinct unit shape
    lists (the plans the step uses; device upload excluded), averaged over
    repeats within about budget_s."""
    import fully_sharded_amd as F
    from workloads.configs import shapes_of
    shape_sets = list(dict.fromkeys(tuple(shapes_of(u)) for u in wl["units"]))
    reps, t0 = 0, time.perf_counter()
    while True:
        for sh in shape_sets:
            F.fsdp_plan_layout(list(sh), wl["R"], wl["layout"])
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 1000:
            break
    return {"ms": (time.perf_counter() - t0) / reps * 1e3, "plans": len(shape_sets),
            "repeats": reps, "where": "host, one thread"}


def plain_copy_bytes(bytes_per_launch):
    """Bytes one launch of the comparison copy moves for a kernel moving
    bytes_per_launch: the same, in whole fp32 elements (4 read + 4 written
    each), at least 8 KiB and at most 4 GiB."""
    return 8 * max(1024, int(min(bytes_per_launch, 4 << 30)) // 8)


def plain_copy(bytes_per_launch, cycle_gib, dev, hs, reps):
    """The simplest stream pattern at the dominant launch's size, for
    comparison: a plain fp32 copy (one read and one write stream, 16-byte
    nontemporal lanes, no occupancy cap) moving the same number of bytes in
    one launch of the library's copy kernel (fsdp_shard_pack of one [n]
    parameter at R = 1), over enough buffer pairs that the 256 MB last-level
    cache serves none of it.  Launches are capped at 4 GiB moved, beyond
    which the rate no longer grows."""
    import torch

    import fully_sharded_amd as F
    n = plain_copy_bytes(bytes_per_launch) // 8
    plan = F.Plan([(n,)], 1, "flat")
    plan.prepare()
    n_pairs = max(2, min(32, -(-int(cycle_gib * (1 << 30)) // (8 * n))))
    bufs = [(torch.ones(n, dtype=torch.float32, device=dev),
             torch.empty(n, dtype=torch.float32, device=dev)) for _ in range(n_pairs)]
    calls = [F.bind_shard_pack(plan, a, b) for a, b in bufs]
    for c in calls:
        c(hs)
    k = [0]

    def one():
        calls[k[0] % n_pairs](hs)
        k[0] += 1
    ms = _timed(one, max(reps, 2 * n_pairs))
    del bufs, calls
    torch.cuda.empty_cache()
    return {"kernel": "k_copy (fsdp_shard_pack: one fp32 parameter, R = 1)",
            "bytes_per_launch": 8 * n, "avg_ms": ms, "achieved": 8 * n / (ms * 1e-3) / 1e9,
            "frac": 8 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, "buffer_pairs": n_pairs}


# ------------------------------------------------------------ other modes
def _timed(fn, reps):
    """ms per call of fn over reps back-to-back calls, HIP events on the
    current stream (the stream every call below launches on)."""
    import torch
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _host(t):
    import numpy as np
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _cpu_loop(work, budget_s):
    """Run work() (returns params processed) until ~budget_s of CPU time."""
    done = 0
    secs = 0.0
    calls = 0
    while secs < budget_s and calls < 1000:
        t0 = time.perf_counter()
        done += work()
        secs += time.perf_counter() - t0
        calls += 1
    return done, secs, calls


def _line(args, wl, metric, value, ms, cfg, kernels, roofline, cpu, extra=None):
    """Print a widened mode's JSON line; every kernel in it, and the
    roofline's, is also compared with a plain copy of its bytes."""
    import torch
    hs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    reps = max(5, args.steps // 4)
    plain = plain_copy(roofline["bytes_per_launch"], args.cycle_gib, "cuda", hs, reps)
    for k in kernels.values():
        pc = (plain if plain_copy_bytes(k["bytes"]) == plain["bytes_per_launch"]
              else plain_copy(k["bytes"], args.cycle_gib, "cuda", hs, reps))
        k["plain_copy_gbps"] = pc["achieved"]
        k["of_plain_copy"] = k["gbps"] / pc["achieved"]
    if args.calibrate_copy:
        extra = dict(extra or {}, copy_calibration=calibration_copy("cuda"))
    d = {
        "metric": metric, "value": value, "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": dict({"workload": args.workload, "units": len(wl["units"]), "R": wl["R"],
                        "layout": wl["layout"], "mode": args.mode}, **cfg),
        "kernels": kernels, "roofline": roofline, "plain_copy": plain, "cpu_baseline": cpu,
    }
    if extra:
        d.update(extra)
    print(json.dumps(d), flush=True)


def run_mode(args, wl, plans, units):
    import ctypes

    import numpy as np
    import torch

    import fully_sharded_amd as F
    from oracle import fsdp_oracle as O
    from workloads.configs import ADAMW

    R = wl["R"]
    dev = "cuda"
    stream = torch.cuda.current_stream()
    hs = ctypes.c_void_p(stream.cuda_stream)
    P = sum(u.plan.T for u in units)
    budget = 0.0 if args.no_cpu_baseline else args.cpu_seconds

    if args.mode == "reshard":
        # restore the whole model's sharded state (bf16 parameter, fp32
        # master, m, v) at world size --to-ranks, same layout
        R2 = args.to_ranks
        dst_plans = {k: F.Plan(list(k), R2, wl["layout"]) for k in plans}
        rsh = {k: F.Resharder(plans[k], dst_plans[k]) for k in plans}
        jobs = []
        for u in units:
            k = tuple(u.plan.shapes)
            S2 = dst_plans[k].S
            p2 = torch.empty(R2 * S2, dtype=u.param.dtype, device=dev)
            st2 = rows(3, R2 * S2, torch.float32, dev)
            jobs.append([(rsh[k], u.param, p2)] + [(rsh[k], a, b) for a, b in
                                                    zip((u.master, u.m, u.v), st2)])
        # one launch per resharder and dtype: the bf16 parameters of every
        # unit, then the fp32 master, m and v of every unit
        batches = []
        for k, rs in rsh.items():
            pairs = [pr for job in jobs for pr in job if pr[0] is rs]
            for want in (units[0].param.dtype, torch.float32):
                sel = [pr for pr in pairs if pr[1].dtype == want]
                for i in range(0, len(sel), 64):
                    batches.append((rs, [pr[1] for pr in sel[i:i + 64]],
                                    [pr[2] for pr in sel[i:i + 64]]))

        def restore():
            for rs, srcs, dsts in batches:
                F.fsdp_reshard_batch(rs, srcs, dsts, hs)

        for _ in range(args.warmup):
            restore()
        ms = _timed(restore, args.steps)
        # the dominant launch: the largest fp32 batch (master, m, v of every
        # unit), T*4 bytes read and T*4 written per array
        big = max((b for b in batches if b[1][0].dtype == torch.float32),
                  key=lambda b: len(b[1]))
        # timed alternating with a second copy of its buffers, so the 256 MB
        # last-level cache cannot serve what the previous launch touched
        big2 = (big[0], [a.clone() for a in big[1]], [torch.empty_like(b) for b in big[2]])
        ms_launch = _timed(lambda: [F.fsdp_reshard_batch(b[0], b[1], b[2], hs)
                                    for b in (big, big2)], max(5, args.steps)) / 2
        bytes_launch = float(big[0].src_plan.T * 8 * len(big[1]))
        u0 = units[0]
        po = O.plan_layout(list(u0.plan.shapes), R, wl["layout"])
        po2 = O.plan_layout(list(u0.plan.shapes), R2, wl["layout"])
        hosts = [_host(x).reshape(R, po.S) for x in (u0.param, u0.master, u0.m, u0.v)]
        def cpu_work():
            for h in hosts:
                O.reshard(po, po2, h)
            return po.T
        done, secs, calls = _cpu_loop(cpu_work, budget) if budget else (0, 0, 0)
        cpu = None if not budget else {
            "value": done / secs, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} restores of unit 0 (parameter, master, m, v; "
                      f"R={R} -> {R2}), {done} params in {secs:.2f} s, one thread"}
        _line(args, wl, f"reshard (restore at R={R2}) params/s and HBM GB/s, {R}->{R2}",
              P / (ms * 1e-3), ms, {"to_ranks": R2, "params": P,
                                     "bytes_per_param": 28, "launches": len(batches)},
              {"reshard_fp32_batch": {"avg_ms": ms_launch, "bytes": bytes_launch,
                                      "arrays": len(big[1]),
                                "gbps": bytes_launch / (ms_launch * 1e-3) / 1e9}},
              roof_entry("copy_pairs", bytes_launch, ms_launch, args.workload, "reshard"), cpu,
              {"hbm_gbps": P * 28 / (ms * 1e-3) / 1e9})
        return

    if args.mode == "accum":
        K = args.micro
        if K < 1:
            raise SystemExit("--micro must be >= 1")
        T_max = max(p.T for p in plans.values())
        recv = rows(R, T_max, units[0].param.dtype, dev)
        accs = [rows(R, u.plan.T, torch.float32, dev) for u in units]
        calls = [(F.bind_grad_accumulate(u.plan, u.grads, a),
                  F.bind_gather_unflatten(u.plan, u.param, recv),
                  F.bind_adamw_shard_step(u.plan, ADAMW, a, u.master, u.m, u.v, u.param))
                 for u, a in zip(units, accs)]
        step_no = [0]

        def step():
            step_no[0] += 1
            for acc, gather, fused in calls:
                for k in range(K):
                    acc(k == 0, hs)
                gather(hs)
                fused(step_no[0], hs)

        for _ in range(args.warmup):
            step()
        ms = _timed(step, args.steps)
        # the accumulate launches of whole passes (K per unit: the first
        # copies, 6 bytes per element and rank; the others add, 10), per launch
        ms_acc = _timed(lambda: [c[0](k == 0, hs) for c in calls for k in range(K)],
                        max(5, args.steps)) / (len(calls) * K)
        Tm = float(np.mean([u.plan.T for u in units]))
        acc_bytes = Tm * R * (6 + 10 * (K - 1)) / K
        step_bytes = P * (R * 6 + (K - 1) * R * 10 + (2 + 2 * R) + (4 * R + 26))
        u0 = units[0]
        po = O.plan_layout(list(u0.plan.shapes), R, wl["layout"])
        hg = [_host(g) for g in u0.grads]
        st = [_host(x).reshape(R, po.S) for x in (u0.master, u0.m, u0.v)]

        def cpu_work():
            accs_h = [O.grad_accumulate([hg[r]] * K) for r in range(R)]
            O.shard_step(po, accs_h, st[0], st[1], st[2], 1, ADAMW, wl["param_dtype"])
            return po.T
        done, secs, ncalls = _cpu_loop(cpu_work, budget) if budget else (0, 0, 0)
        cpu = None if not budget else {
            "value": done / secs, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{ncalls} accumulated steps of unit 0 (K={K}, R={R}), {done} params in "
                      f"{secs:.2f} s, one thread"}
        _line(args, wl, f"accumulated-step params/s and HBM GB/s, K={K} micro-batches",
              P / (ms * 1e-3), ms, {"micro_batches": K, "params": P},
              {"accumulate": {"avg_ms": ms_acc, "bytes": acc_bytes,
                              "gbps": acc_bytes / (ms_acc * 1e-3) / 1e9}},
              roof_entry("accumulate", acc_bytes, ms_acc, args.workload, "accum"), cpu,
              {"hbm_gbps": step_bytes / (ms * 1e-3) / 1e9, "step_bytes": step_bytes})
        return

    if args.mode == "ddp":
        # every rank holds the full model: R full replicas of parameter,
        # master, m and v; the gradient all-reduce-average gives every rank
        # the whole averaged gradient; every rank runs AdamW on all of it.
        from fully_sharded_amd.step import StepRunner
        from workloads import gen
        jobs = []
        for i, u in enumerate(units):
            T = u.plan.T
            rep = F.Plan([(R * T,)], 1, "flat")      # R replicas as one flat array
            avg = torch.empty(R * T, dtype=torch.float32, device=dev)
            full = gen.device_master(wl, i, list(u.plan.shapes), dev)
            master, m, v = rows(3, R * T, torch.float32, dev)
            master.view(R, T).copy_(full.expand(R, T))
            m.zero_()
            v.zero_()
            param = torch.empty(R * T, dtype=u.param.dtype, device=dev)
            param.view(R, T).copy_(full.expand(R, T))
            outs = list(avg.view(R, T).unbind(0))
            jobs.append((u, rep, avg, outs, (rep, master, m, v, param)))
        step_no = [0]

        def step():
            step_no[0] += 1
            for u, rep, avg, outs, (rp, master, m, v, param) in jobs:
                F.fsdp_allreduce_avg(u.plan, u.grads, outs, hs)
                F.fsdp_adamw_shard_step(rp, ADAMW, step_no[0], avg, master, m, v, param,
                                        grads_are_replicas=False, stream=hs)

        for _ in range(args.warmup):
            step()
        ms = _timed(step, args.steps)
        ms_ar = _timed(lambda: [F.fsdp_allreduce_avg(j[0].plan, j[0].grads, j[3], hs)
                                for j in jobs], max(5, args.steps)) / len(jobs)
        tt = [10 ** 6]

        def adamw_pass():
            tt[0] += 1
            for u, rep, avg, outs, (rp, master, m, v, param) in jobs:
                F.fsdp_adamw_shard_step(rp, ADAMW, tt[0], avg, master, m, v, param,
                                        grads_are_replicas=False, stream=hs)
        ms_adamw = _timed(adamw_pass, max(5, args.steps)) / len(jobs)
        Tm = float(np.mean([u.plan.T for u in units]))
        ar_bytes = Tm * (2 * R + 4 * R)
        pes = 2 if units[0].param.dtype == torch.bfloat16 else 4
        adamw_bytes = Tm * R * (4 + 24 + pes)
        step_bytes = P * (6 * R + 30 * R)
        # the FSDP step on the same model, same run, for the comparison
        recv = rows(R, max(p.T for p in plans.values()), units[0].param.dtype, dev)
        runner = StepRunner(units, ADAMW, [recv])
        fs = [0]

        def fstep():
            fs[0] += 1
            runner.step(fs[0])
        for _ in range(args.warmup):
            fstep()
        ms_fsdp = _timed(fstep, args.steps)
        S_tot = sum(u.plan.S for u in units)
        n_units = len(units)
        # HBM bytes per step from the counter runs of this mode (FETCH_SIZE +
        # WRITE_SIZE per launch, scaled by a plain copy), where the profiles
        # hold them for the current kernels
        tr = {k: load_traffic(args.workload, k, "ddp")
              for k in ("allreduce", "adamw", "fused", "gather")}
        measured = {
            "ddp": (n_units * (tr["allreduce"] + tr["adamw"])
                    if tr["allreduce"] and tr["adamw"] else None),
            "fsdp": (n_units * (tr["fused"] + tr["gather"])
                     if tr["fused"] and tr["gather"] else None),
            "source": "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch of bench.py --mode ddp "
                      "(profiles/traffic_<workload>_ddp_*.json), times the units per step",
        }
        if measured["ddp"] and measured["fsdp"]:
            measured["ddp_over_fsdp"] = measured["ddp"] / measured["fsdp"]
        ledger = {
            "state_bytes_per_rank": {"ddp": 16 * P, "fsdp": 16 * S_tot},
            "comm_elems_per_rank_per_step": {
                "ddp_allreduce": 2.0 * (R - 1) / R * P,
                "fsdp_reshard_after_forward": sum(u.plan.comm_ledger(True)["total"]
                                                  for u in units),
                "fsdp_keep_after_forward": sum(u.plan.comm_ledger(False)["total"]
                                               for u in units)},
            "hbm_bytes_per_step": {"ddp": step_bytes,
                                   "fsdp": P * (4 * R + 28)},
            "hbm_bytes_per_step_measured": measured,
        }
        u0 = units[0]
        hg = [_host(g) for g in u0.grads]
        T0 = u0.plan.T
        z = np.zeros(T0, np.float32)
        m0 = _host(jobs[0][4][1])[:T0].copy()

        def cpu_work():
            avg = O.allreduce_avg(hg)
            for r in range(R):
                O.adamw_step(m0, z, z, avg[r], 1, **ADAMW)
            return T0
        done, secs, ncalls = _cpu_loop(cpu_work, budget) if budget else (0, 0, 0)
        cpu = None if not budget else {
            "value": done / secs, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{ncalls} DDP steps of unit 0 (all-reduce + AdamW on {R} replicas), "
                      f"{done} params in {secs:.2f} s, one thread"}
        _line(args, wl, "DDP-comparator step params/s (all-reduce + AdamW on every replica)",
              P / (ms * 1e-3), ms, {"params": P},
              {"allreduce_avg": {"avg_ms": ms_ar, "bytes": ar_bytes,
                                 "gbps": ar_bytes / (ms_ar * 1e-3) / 1e9},
               "adamw_replicas": {"avg_ms": ms_adamw, "bytes": adamw_bytes,
                                  "gbps": adamw_bytes / (ms_adamw * 1e-3) / 1e9}},
              roof_entry("allreduce", ar_bytes, ms_ar, args.workload, "ddp"), cpu,
              {"hbm_gbps": step_bytes / (ms * 1e-3) / 1e9, "step_bytes": step_bytes,
               "fsdp_ms_per_step_same_run": ms_fsdp, "ddp_over_fsdp_time": ms / ms_fsdp,
               "ledger": ledger})
        return
    raise SystemExit(f"unknown mode {args.mode}")


def cpu_workers():
    """Host processes for the oracle's all-cores leg: the cores this process
    may run on, at most 16 (one GPU's share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    import platform
    name = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return name


def oracle_unit_worker(job):
    """One oracle process of the all-cores leg: one unit's training steps, as
    the one-core leg runs them (R gathers, then the shard step), repeated
    until budget_s of compute; returns (params, seconds, steps, the first
    step's results or None)."""
    shapes, R, layout, grads, master, param, pdt, budget_s, want_first = job
    import numpy as np

    from oracle import fsdp_oracle as O
    from workloads.configs import ADAMW
    po = O.plan_layout(shapes, R, layout)
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    first = None
    done, secs, t = 0, 0.0, 0
    while secs < budget_s and t < 1000:
        t += 1
        t0 = time.perf_counter()
        for _ in range(R):
            O.gather_unflatten(po, param)
        master, m, v, param = O.shard_step(po, grads, master, m, v, t, ADAMW, pdt)
        secs += time.perf_counter() - t0
        done += po.T
        if want_first and first is None:
            first = (master, m, v, param)
    return done, secs, t, first


def oracle_chunk_worker(job):
    """One oracle process of the group leg: the step's element-wise work
    (rank-order mean, AdamW, recast) on one chunk, repeated until budget_s."""
    chunk, pdt, budget_s = job
    from oracle import fsdp_oracle as O
    from workloads.configs import ADAMW
    done, secs, t = 0, 0.0, 0
    while secs < budget_s and t < 1000:
        t += 1
        t0 = time.perf_counter()
        g = O.rank_order_mean(chunk["grads"])
        p2, _, _ = O.adamw_step(chunk["master"], chunk["m"], chunk["v"], g, t, ADAMW["lr"],
                                ADAMW["beta1"], ADAMW["beta2"], ADAMW["eps"],
                                ADAMW["weight_decay"])
        if pdt == "bf16":
            O.bf16_rne(p2)
        secs += time.perf_counter() - t0
        done += chunk["master"].size
    return done, secs, t


def cpu_baseline(state, R, wl, budget_s, group_sample=None):
    """The oracle, as it stands, on the same inputs (copied back to the host),
    timed on the host in three legs:
      one core:   per unit, R gathers (one per receiving rank) then the shard
                  step, units in order, step after step, in this process
                  (NumPy's element-wise loops run on one thread);
      all cores:  the same per-unit steps, one spawned process per unit (at
                  most one per usable core, 16 at most), all at once; the
                  first step of unit 0 is checked bit for bit against the
                  one-core leg's; rate = parameters stepped / the longest
                  process's compute time;
      group:      chunks of the sustained workload's inputs (when that part
                  ran), one process per chunk: the step's element-wise work.
    `value` and `cores` are the all-cores leg's.  The worker processes start
    fresh interpreters (they never touch the GPU)."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np

    from oracle import fsdp_oracle as O
    from workloads.configs import ADAMW

    if max(u.plan.T for u in state) * R > (1 << 26):
        return None   # the oracle copies whole units to the host: too large here
    plans = {}
    units = []
    for s in state:
        pl = s.plan
        key = tuple(pl.shapes)
        if key not in plans:
            plans[key] = O.plan_layout(list(pl.shapes), R, wl["layout"])
        po = plans[key]
        units.append(dict(po=po, shapes=list(pl.shapes), grads=[_host(g) for g in s.grads],
                          master=_host(s.master).reshape(R, po.S).copy(),
                          m=np.zeros((R, po.S), np.float32), v=np.zeros((R, po.S), np.float32),
                          param=_host(s.param).reshape(R, po.S).copy()))
    init = [(u["master"].copy(), u["param"].copy()) for u in units]
    pdt = wl["param_dtype"]
    share = {"one": 0.4, "all": 0.35, "group": 0.25} if group_sample else \
        {"one": 0.55, "all": 0.45, "group": 0.0}

    # ---- one core
    done = 0
    secs = 0.0
    unit_steps = 0
    t = 0
    first = None
    while secs < share["one"] * budget_s and t < 1000:
        t += 1
        for u in units:
            po = u["po"]
            t0 = time.perf_counter()
            for _ in range(R):
                O.gather_unflatten(po, u["param"])
            u["master"], u["m"], u["v"], u["param"] = O.shard_step(
                po, u["grads"], u["master"], u["m"], u["v"], t, ADAMW, pdt)
            secs += time.perf_counter() - t0
            if first is None:
                first = (u["master"], u["m"], u["v"], u["param"])
            done += po.T
            unit_steps += 1
            if secs >= share["one"] * budget_s:
                break
    one = {"value": done / secs, "unit": "params/s", "cores": 1,
           "sample": f"{unit_steps} unit-steps over {t} step(s) of the {len(state)}-unit "
                     f"model (per unit: {R} gathers + reduce-scatter-average + AdamW + "
                     f"recast), {done} params in {secs:.2f} s, one process"}

    # ---- all cores: one process per unit
    nproc = min(cpu_workers(), len(units))
    ctx = multiprocessing.get_context("spawn")
    jobs = [(u["shapes"], R, wl["layout"], u["grads"], m0, p0, pdt, share["all"] * budget_s,
             i == 0) for i, (u, (m0, p0)) in enumerate(zip(units[:nproc], init))]
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=nproc, mp_context=ctx) as pool:
        res = list(pool.map(oracle_unit_worker, jobs))
        wall = time.perf_counter() - t0
        got = res[0][3]
        for a, b, name in zip(got, first, ("master", "m", "v", "param")):
            if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
                raise SystemExit(f"oracle all-cores leg differs from the one-core leg ({name})")
        done = sum(r[0] for r in res)
        secs = max(r[1] for r in res)
        allc = {"value": done / secs, "unit": "params/s", "cores": nproc,
                "sample": f"{nproc} processes, one unit of the {len(state)}-unit model each, "
                          f"running its steps as the one-core leg does "
                          f"({sum(r[2] for r in res)} unit-steps; unit 0's first step "
                          f"bit-identical to the one-core leg's), {done} params, longest "
                          f"process {secs:.2f} s of compute ({wall:.2f} s wall with start-up)"}

        # ---- the sustained workload, chunk by chunk
        grp = None
        if group_sample and group_sample["chunks"]:
            ch = group_sample["chunks"]
            gjobs = [(c, group_sample["param_dtype"], share["group"] * budget_s) for c in ch]
            with ProcessPoolExecutor(max_workers=min(cpu_workers(), len(ch)),
                                     mp_context=ctx) as gpool:
                gres = list(gpool.map(oracle_chunk_worker, gjobs))
            gdone = sum(r[0] for r in gres)
            gsecs = max(r[1] for r in gres)
            grp = {"value": gdone / gsecs, "unit": "params/s",
                   "cores": min(cpu_workers(), len(ch)),
                   "sample": f"{len(ch)} chunks of up to 1 Mi elements of the "
                             f"{group_sample['workload']} shard space (R={group_sample['R']}"
                             f"), one process each: reduce-scatter-average + AdamW + "
                             f"recast, {sum(r[2] for r in gres)} chunk passes, {gdone} params, "
                             f"longest process {gsecs:.2f} s"}
    return {
        "value": allc["value"],
        "unit": "params/s",
        "cores": nproc,
        "kind": "oracle",
        "sample": allc["sample"],
        "cpu_model": cpu_model(),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "legs": {"one_core": one, "all_cores": allc, "sustained_workload_chunks": grp},
    }


if __name__ == "__main__":
    main()
