"""Throughput of the halo-sharded conv + GroupNorm layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = halo pack + halo unpack + per-shard conv (all shards, one grouped
launch) + GroupNorm (partials, combine, apply) over the whole sharded volume,
inputs already resident in HBM.  Prints one JSON line.  The forward step is
timed as a replayed HIP graph of those launches (--graph on, the default);
per-kernel average durations come from the same number of eager steps, each
library call bracketed with HIP events on the stream it runs on, and the
longest one is reported in `roofline` against its algorithmic bytes (or
flops) per launch.  The CPU baseline is the
fp64 oracle timed on a bounded slab of the same workload on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sharded conv+GroupNorm voxels/s on 1 MI355X; % MFMA peak (conv), % HBM BW (halo/norm)"
METRIC_DGRAD = "sharded conv input-gradient (halo exchange of dy + conv) voxels/s on 1 MI355X"
METRIC_STRIDED = "sharded stride-2 conv (halo exchange + strided 'same' conv) input voxels/s on 1 MI355X"
METRIC_TRANSPOSED = "sharded stride-2 transposed conv (halo exchange + upsampling conv) output voxels/s on 1 MI355X"
METRIC_POOL = "sharded 2x downsampling (halo exchange + 'valid' average pooling, k=2 s=2) input voxels/s on 1 MI355X"
METRIC_BWD = ("sharded conv+GroupNorm backward (GroupNorm backward, halo exchange of dy, input gradient, "
              "weight gradient) voxels/s on 1 MI355X")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
FP32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--pass", dest="pass_", choices=("forward", "dgrad", "backward", "pool", "strided", "transposed"),
                    default="forward",
                    help="the layer's forward step, the input gradient of its conv, its whole backward step, "
                         "a 2x average-pool downsampling or a stride-2 conv of its input shards, or a stride-2 "
                         "transposed conv from half its resolution up to it")
    ap.add_argument("--exchange", choices=("pack+unpack", "fused"), default="pack+unpack",
                    help="halo exchange as two copies through a message buffer, or one fused copy")
    ap.add_argument("--graph", choices=("on", "off"), default="on",
                    help="time the step as a replayed HIP graph (per-stage times come from an eager run of "
                         "the same steps); the input-gradient pass always runs eagerly")
    ap.add_argument("--cold", choices=("on", "off"), default="on",
                    help="forward and input-gradient passes: after the timed steps, time each stage again over "
                         "the same number of steps with a 1 GiB buffer written between steps (caches flushed); "
                         "reports median and min per stage")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--nested", choices=("on", "off"), default="on",
                    help="with no --workload: also time every other workload's forward step and nest its "
                         "figures in the headline line")
    ap.add_argument("--cpu-rows", type=int, default=None, help="rows of the oracle's CPU sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling the HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files into a traffic record")
    ap.add_argument("--record-stage", default="conv", choices=("conv", "strided", "transposed", "pool"),
                    help="the stage whose kernels --record-traffic counts")
    ap.add_argument("--record-out", default=None, help="where --record-traffic writes its JSON")
    return ap.parse_args()


COPY_BYTES = 1 << 30                 # bytes read (and written) by --calibrate-copy
STAGE_KERNELS = {                    # kernel-name fragments of each library stage
    "halo_pack": ("halo_copy",), "halo_unpack": ("halo_copy",), "halo_exchange": ("halo_copy",),
    "conv": ("conv_rows", "conv_taps", "conv_gemm", "conv_direct"),
    "gn_partials": ("gn_max", "gn_stats"), "gn_apply": ("gn_apply",),
    "wgrad": ("wgrad_tr", "wgrad_grp", "wgrad_direct"), "gn_backward": ("gn_max", "gnb_"), "pool": ("pool_kernel", "pool_fixed"),
    "strided": ("conv_sx_mfma", "conv_strided"), "transposed": ("conv_sx_mfma", "conv_transposed"),
}


STAGE_SOURCES = {                    # library sources that define each stage's kernels and launches
    "halo_pack": ("halo.hip", "plan.cpp", "internal.h"), "halo_unpack": ("halo.hip", "plan.cpp", "internal.h"),
    "halo_exchange": ("halo.hip", "plan.cpp", "internal.h"),
    "conv": ("conv.hip", "internal.h"),
    "gn_partials": ("groupnorm.hip", "internal.h"), "gn_apply": ("groupnorm.hip", "internal.h"),
    "wgrad": ("wgrad.hip", "internal.h"), "gn_backward": ("groupnorm.hip", "internal.h"),
    "pool": ("pool.hip", "internal.h"), "strided": ("strided.hip", "internal.h"),
    "transposed": ("strided.hip", "internal.h"),
}


def source_digest(stage: str) -> str:
    """Digest of the sources of one stage: a traffic record is valid only for
    the kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "halo_sharded_conv_amd", "csrc")
    for f in STAGE_SOURCES[stage]:
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _counter_means(path, fragments, pick_max=False):
    """Mean counter value per dispatch of the kernels whose names contain a
    fragment (or the largest single dispatch value with pick_max)."""
    import csv
    vals = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if fragments and not any(f in r["Kernel_Name"] for f in fragments):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no matching dispatches in {path}")
    per = {}
    for (_, name), v in vals.items():
        per.setdefault(name, []).append(v)
    if pick_max:
        return {name: (max(v), len(v)) for name, v in per.items()}
    return {name: (sum(v) / len(v), len(v)) for name, v in per.items()}


def record_traffic(args):
    """HBM bytes per conv launch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    COPY_BYTES."""
    import synth
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.record_traffic
    wl = synth.workload(args.workload or synth.BENCH_WORKLOAD)
    stage = args.record_stage
    f = _counter_means(fetch_csv, STAGE_KERNELS[stage])["FETCH_SIZE"]
    w = _counter_means(write_csv, STAGE_KERNELS[stage])["WRITE_SIZE"]
    # the copy is the elementwise dispatch that reads; the fill before it only writes
    cf = _counter_means(cfetch_csv, ("elementwise",), pick_max=True)["FETCH_SIZE"]
    cw = _counter_means(cwrite_csv, ("elementwise",), pick_max=True)["WRITE_SIZE"]
    f_scale = COPY_BYTES / (cf[0] * 1024.0)
    w_scale = COPY_BYTES / (cw[0] * 1024.0)
    rec = {
        "workload": wl.name, "stage": stage, "source_digest": source_digest(stage),
        "fetch_kib_per_dispatch": f[0], "write_kib_per_dispatch": w[0], "dispatches": [f[1], w[1]],
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": cf[0], "copy_write_kib": cw[0],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "traffic_bytes": f[0] * 1024.0 * f_scale + w[0] * 1024.0 * w_scale,
    }
    out = args.record_out or traffic_path(wl, stage)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def calibrate_copy():
    """A plain 1 GiB device copy b = a * 1 through an elementwise kernel
    (16 bytes per lane, whole 128-byte lines: the access shape of the
    library's kernels).  torch's copy_ is avoided: it runs a runtime blit
    kernel whose read counter scales differently."""
    import torch
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def traffic_path(wl, stage):
    """Where the traffic record of one stage on one workload lives (the conv's
    carries no stage suffix)."""
    suffix = "" if stage == "conv" else f"_{stage}"
    return os.path.join(ROOT, "profiles", f"traffic_{wl.name}{suffix}.json")


def load_traffic(wl, stage):
    """Measured HBM bytes per launch of `stage`, or None when no record exists
    or the kernels changed since it was taken."""
    p = traffic_path(wl, stage)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("stage") != stage or stage not in STAGE_SOURCES or rec.get("source_digest") != source_digest(stage):
        return None
    return rec["traffic_bytes"]


def algorithmic(wl, layer):
    """Algorithmic HBM bytes and flops per launch of each stage."""
    import numpy as np
    esize = 4 if wl.dtype == "f32" else 2
    vox = wl.voxels
    x_bytes = vox * wl.cin * esize
    y_bytes = vox * wl.cout * 4
    plan = layer.in_plan
    payload = plan.msg_bytes
    # zeros written into the margins on the global faces (the conv's padding)
    zero_bytes = 0
    for i in range(plan.num_halo_boxes, plan.num_halo_boxes + plan.num_zero_boxes):
        zero_bytes += plan.batch * int(np.prod(plan.halo_box(i)["ext"])) * wl.cin * esize
    return {
        "halo_pack": {"bytes": 2 * payload},                 # read boxes, write message
        "halo_unpack": {"bytes": 2 * payload + zero_bytes},  # read message, write margins and zero faces
        "halo_exchange": {"bytes": 2 * payload + zero_bytes},   # read boxes, write margins and zero faces
        "conv": {"bytes": x_bytes + y_bytes, "flops": wl.conv_flops},
        "gn_partials": {"bytes": y_bytes},
        "gn_apply": {"bytes": 2 * y_bytes},
        # max |dz|, then (y, dz) for the sums, then (y, dz) -> dy in the conv's operand type
        "gn_backward": {"bytes": 5 * y_bytes + vox * wl.cout * esize},
        # x and dy (operand type) read, dw written
        "wgrad": {"bytes": x_bytes + vox * wl.cout * esize + wl.cout * wl.cin * wl.taps * 4,
                  "flops": wl.conv_flops},
    }


def cpu_baseline(wl, rows, w_fwd=None, backward=False):
    """The oracle (fp64 numpy) on the first `rows` rows of the outermost axis:
    conv + GroupNorm, or (w_fwd given: wl is the input-gradient layer) the
    input gradient of the forward conv, or (backward) the layer's backward
    step: GroupNorm backward, input gradient and weight gradient."""
    if backward:
        return cpu_baseline_backward(wl, rows)
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    sub_shape = (rows,) + tuple(wl.spatial[1:])
    sub = synth.small_variant(wl, sub_shape, [(s,) for s in sub_shape], name_suffix="cpu_sample")
    x = synth.make_input(sub)
    t0 = time.perf_counter()
    if w_fwd is None:
        w = oracle.widen(synth.make_weight(wl), wl.dtype)
        t0 = time.perf_counter()
        y = oracle.conv_same(oracle.widen(x, wl.dtype), w)
        z = oracle.group_norm(y, wl.groups, wl.eps)
    else:
        w = oracle.widen(w_fwd, wl.dtype)
        t0 = time.perf_counter()
        z = oracle.conv_same_dgrad(oracle.widen(x, wl.dtype), w)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": sub.voxels / dt, "unit": "voxels/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} rows of the outermost axis ({sub.voxels} voxels, "
                      + ("conv + GroupNorm" if w_fwd is None else "input gradient of the conv")
                      + f" in fp64 numpy, {dt:.1f} s)", "seconds": round(dt, 2), "checksum": float(np.abs(z).sum())}


def cpu_baseline_backward(wl, rows):
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth
    sub_shape = (rows,) + tuple(wl.spatial[1:])
    sub = synth.small_variant(wl, sub_shape, [(s,) for s in sub_shape], name_suffix="cpu_sample")
    x = oracle.widen(synth.make_input(sub), wl.dtype)
    w = oracle.widen(synth.make_weight(wl), wl.dtype)
    y = oracle.conv_same(x, w)
    dz = synth.make_upstream_grad(sub, seed=31)
    t0 = time.perf_counter()
    dy, dg, db = oracle.group_norm_backward(y, dz, wl.groups, wl.eps)
    # the conv backward takes dy in the operand type
    dyc = oracle.widen(synth.f32_to_bf16_bits(dy.astype(np.float32)), wl.dtype) if wl.dtype == "bf16" else dy
    dx = oracle.conv_same_dgrad(dyc, w)
    dw = oracle.conv_same_wgrad(x, dyc, wl.ksize)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": sub.voxels / dt, "unit": "voxels/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} rows of the outermost axis ({sub.voxels} voxels, GroupNorm backward + input "
                      f"gradient + weight gradient in fp64 numpy, {dt:.1f} s)", "seconds": round(dt, 2),
            "checksum": float(np.abs(dy).sum() + np.abs(dx).sum() + np.abs(dw).sum())}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from halo_sharded_conv_amd.layer import ShardedConvGN

    name = args.workload or synth.BENCH_WORKLOAD
    wl_fwd = synth.workload(name)
    if args.pass_ == "backward":
        return bench_backward(args, wl_fwd)
    if args.pass_ == "pool":
        return bench_pool(args, wl_fwd)
    if args.pass_ == "strided":
        return bench_strided(args, wl_fwd)
    if args.pass_ == "transposed":
        return bench_transposed(args, wl_fwd)
    out = bench_layer(args, wl_fwd, cold=args.cold == "on", cpu=not args.no_cpu_baseline)
    if args.pass_ == "forward" and args.workload is None and args.nested == "on":
        # the other workloads of the layer, same step and timing, one entry each
        nested = {wl_fwd.name: summary(out)}
        for other in synth.WORKLOADS:
            if other != wl_fwd.name:
                nested[other] = summary(bench_layer(args, synth.workload(other), cold=False, cpu=False))
        out["workloads"] = nested
    print(json.dumps(out), flush=True)


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON record)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def summary(rec):
    """The per-workload figures nested in the headline line."""
    keep = ("value", "ms_per_step", "gpu_ms_per_step", "eager_ms_per_step", "roofline", "kernels")
    out = {k: rec[k] for k in keep if k in rec}
    out["config"] = {k: rec["config"][k] for k in ("shape", "cout", "kernel", "shards", "groups")}
    return out


def bench_layer(args, wl_fwd, cold, cpu):
    """One forward (or input-gradient) step of a workload: build its layer,
    time its stages eagerly and the step as a replayed graph; returns the
    record."""
    import gc

    import torch

    import synth
    from halo_sharded_conv_amd.layer import ShardedConvGN
    progress(f"{wl_fwd.name} ({args.pass_}): generating the input")
    if args.pass_ == "dgrad":
        # input gradient of the layer's conv: dy (Cout channels) -> dx (Cin)
        from halo_sharded_conv_amd.layer import dgrad_config
        wl = dgrad_config(wl_fwd)
        layer = ShardedConvGN(wl)
        layer.set_weight_dgrad(synth.make_weight(wl_fwd))
    else:
        wl = wl_fwd
        layer = ShardedConvGN(wl)
        layer.set_weight(synth.make_weight(wl))
    layer.load_input(synth.make_input(wl))
    stream = torch.cuda.current_stream()
    progress(f"{wl_fwd.name}: timing {args.warmup} + {args.steps} steps")

    if args.exchange == "fused":
        halo = [("halo_exchange", lambda: layer.exchange_fused())]
    else:
        halo = [("halo_pack", lambda: layer.exchange_pack()), ("halo_unpack", lambda: layer.exchange_unpack())]
    stages = halo + [("conv", layer.conv)]
    if args.pass_ == "forward":
        stages += [("gn_partials", layer.norm_partials), ("gn_apply", layer.norm_combine_apply)]

    per_kernel_ms, ms_per_step, gpu_ms = time_stages(args, stages, stream)
    eager_ms = ms_per_step
    if args.pass_ == "forward" and args.graph == "on":
        ms_per_step, gpu_ms = time_graph(args, stages)
    cold_rec = time_stages_cold(args, stages, stream) if cold and args.steps > 0 else None

    rec = report(args, wl, layer, per_kernel_ms, ms_per_step, gpu_ms,
                 METRIC if args.pass_ == "forward" else METRIC_DGRAD,
                 None if args.pass_ == "forward" else synth.make_weight(wl_fwd),
                 eager_ms=eager_ms if args.pass_ == "forward" and args.graph == "on" else None, cold=cold_rec,
                 cpu=cpu)
    del layer, stages, halo
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def time_stages(args, stages, stream):
    """Warm-up, then K timed steps; HIP events around every stage on its stream."""
    import numpy as np
    import torch
    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()
    ev = {k: [] for k, _ in stages}
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        for k, fn in stages:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[k].append((a, b))
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end) / args.steps
    per_kernel_ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    return per_kernel_ms, wall * 1e3 / args.steps, gpu_ms


FLUSH_BYTES = 1 << 30                # written between cold steps: 4x the 256 MB Infinity Cache


def time_stages_cold(args, stages, stream):
    """K more eager steps, each after a 1 GiB write that evicts L2 and the
    Infinity Cache, so no stage starts with its operands cache-resident; HIP
    events around every stage and around the step, median and min over the
    steps.  The flush itself is outside every event pair."""
    import numpy as np
    import torch
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    ev = {k: [] for k, _ in stages}
    steps = []
    for i in range(args.steps):
        flush.fill_(float(i))
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for k, fn in stages:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[k].append((a, b))
        s1 = torch.cuda.Event(enable_timing=True)
        s1.record(stream)
        steps.append((s0, s1))
    torch.cuda.synchronize()
    del flush
    out = {k: {"median_ms": round(float(np.median([a.elapsed_time(b) for a, b in v])), 5),
               "min_ms": round(float(np.min([a.elapsed_time(b) for a, b in v])), 5)} for k, v in ev.items()}
    t = [a.elapsed_time(b) for a, b in steps]
    out["step"] = {"median_ms": round(float(np.median(t)), 5), "min_ms": round(float(np.min(t)), 5)}
    return out


def bench_backward(args, wl_fwd):
    """The layer's backward step: GroupNorm backward (dz -> dy at the conv
    output, written in the conv's operand type straight into the halo-padded
    shards of the input-gradient conv), halo exchange of dy, input gradient
    (conv with the transposed, flipped weights) and weight gradient.  The
    forward step runs once before timing (it leaves y, the statistics and the
    exchanged x)."""
    import torch

    import halo_sharded_conv_amd as hsc
    import synth
    from halo_sharded_conv_amd.layer import ShardedConvGN, dgrad_config

    wl = wl_fwd
    fwd = ShardedConvGN(wl)
    w = synth.make_weight(wl)
    fwd.set_weight(w)
    fwd.load_input(synth.make_input(wl))
    fwd.step()
    fwd.alloc_backward()
    fwd.load_upstream_grad(synth.make_upstream_grad(wl, seed=31))
    bwd = ShardedConvGN(dgrad_config(wl))
    bwd.set_weight_dgrad(w)
    dw = torch.empty(wl.cout * wl.cin * wl.taps, dtype=torch.float32, device="cuda")
    wws = torch.empty(hsc.st_conv_wgrad_workspace_bytes(fwd.in_plan, wl.cout, wl.ksize), dtype=torch.uint8,
                      device="cuda")
    torch.cuda.synchronize()
    if args.exchange == "fused":
        halo = [("halo_exchange", lambda: bwd.exchange_fused())]
    else:
        halo = [("halo_pack", lambda: bwd.exchange_pack()), ("halo_unpack", lambda: bwd.exchange_unpack())]
    stages = [("gn_backward", lambda: fwd.norm_backward(dy_bufs=bwd.x_bufs, dy_plan=bwd.in_plan))] + halo + [
        ("conv", bwd.conv),
        ("wgrad", lambda: hsc.st_conv_wgrad(fwd.in_plan, fwd.x_bufs, bwd.in_plan, bwd.x_bufs, wl.ksize, dw, wws))]
    per_kernel_ms, ms_per_step, gpu_ms = time_stages(args, stages, torch.cuda.current_stream())
    eager_ms = ms_per_step
    if args.graph == "on":
        ms_per_step, gpu_ms = time_graph(args, stages)
    print(json.dumps(report(args, wl, fwd, per_kernel_ms, ms_per_step, gpu_ms, METRIC_BWD, None, dgrad_layer=bwd,
                            eager_ms=eager_ms if args.graph == "on" else None)), flush=True)


def time_graph(args, stages):
    """The step captured once in a HIP graph, W replays untimed, then K
    replays bracketed by synchronisations (host clock) and events."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn in stages:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in stages:
            fn()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / args.steps, start.elapsed_time(end) / args.steps


def shape_change_roofline(wl, key, ms, flops, alg_bytes, kernels, traffic):
    """Roofline of the strided / transposed conv kernel.  bf16 shapes with
    Cin % 16 == 0, Cout % 16 == 0 and the weights of a 32-channel block within
    160 KiB run on the matrix cores: HBM-bound below
    MI355X's ridge (~315 flop/byte; the 32- and 64-channel layers, 60-100),
    MFMA-bound above it (256 channels).  The rest run on fp32 FMA: the ALU
    roofline against the 157.3 TFLOP/s fp32 vector peak."""
    tf = flops / (ms * 1e-3) / 1e12
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    mfma = (wl.dtype == "bf16" and wl.cin % 16 == 0 and wl.cout % 16 == 0
            and wl.taps * wl.cin * 32 * 2 <= 160 * 1024)
    kernels[key].update({"TFLOP/s": round(tf, 2),
                         ("mfma_frac" if mfma else "fp32_frac"):
                             round(tf / (MFMA_BF16_PEAK_TFLOPS if mfma else FP32_PEAK_TFLOPS), 4),
                         "path": "bf16 MFMA" if mfma else "fp32 FMA"})
    peak_tf = MFMA_BF16_PEAK_TFLOPS if mfma else FP32_PEAK_TFLOPS
    kernels[key]["attainable_frac"] = round(tf / min(peak_tf, flops / alg_bytes * HBM_PEAK_GBS / 1e3), 4)
    if mfma and flops / alg_bytes >= MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        # above the ridge (256-channel layers): the matrix cores bound it
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "kernel": key, "traffic": traffic}
    if mfma:
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": key, "traffic": traffic}
    return {"bound": "alu", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / FP32_PEAK_TFLOPS, 4), "kernel": key, "traffic": traffic}


def bench_strided(args, wl):
    """Downsampling conv of the layer's input shards: halo exchange and a
    stride-2 'same' conv with the layer's weights into the fp32 output plan
    the library derives."""
    import numpy as np
    import torch

    import halo_sharded_conv_amd as hsc
    import synth
    from halo_sharded_conv_amd.layer import ShardedConvGN

    s = 2
    layer = ShardedConvGN(wl)
    layer.load_input(synth.make_input(wl))
    w = synth.make_weight(wl)                                   # raw [Cout][Cin][k..] in the operand type
    wt = torch.from_numpy(np.ascontiguousarray(w.view(np.int16) if w.dtype == np.uint16 else w).reshape(-1)).cuda()
    q = hsc.st_plan_strided(layer.in_plan, wl.ksize, s, wl.cout)
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(q.num_shards)]
    ws = torch.empty(hsc.st_conv_strided_workspace_bytes(layer.in_plan, wl.cout, wl.ksize), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    stages = [("halo_pack", lambda: layer.exchange_pack()), ("halo_unpack", lambda: layer.exchange_unpack()),
              ("strided", lambda: hsc.st_conv_strided_sharded(layer.in_plan, layer.x_bufs, wt, None, wl.ksize, s,
                                                              q, outs, ws))]
    per_kernel_ms, ms_per_step, gpu_ms = time_stages(args, stages, torch.cuda.current_stream())
    eager_ms = ms_per_step
    if args.graph == "on":
        ms_per_step, gpu_ms = time_graph(args, stages)
    esize = 4 if wl.dtype == "f32" else 2
    out_vox = wl.batch * int(np.prod([sum(a) for a in q.shards]))
    flops = 2 * out_vox * wl.cin * wl.cout * wl.taps
    alg = {"halo_pack": 2 * layer.in_plan.msg_bytes, "halo_unpack": 2 * layer.in_plan.msg_bytes,
           "strided": wl.voxels * wl.cin * esize + out_vox * wl.cout * 4}
    kernels = {}
    for key, ms in per_kernel_ms.items():
        gbs = alg[key] / (ms * 1e-3) / 1e9
        kernels[key] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof = shape_change_roofline(wl, "strided", per_kernel_ms["strided"], flops, alg["strided"], kernels,
                                 load_traffic(wl, "strided"))
    out = {"metric": METRIC_STRIDED, "value": wl.voxels / (ms_per_step * 1e-3), "unit": "voxels/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32" if roof["bound"] == "alu" else "bf16", "data": "synthetic",
           "config": {"workload": wl.name, "shape": [wl.batch, wl.cin, *wl.spatial], "cout": wl.cout,
                      "kernel": wl.ksize, "stride": s, "operands": wl.dtype, "shards": [list(a) for a in wl.shards],
                      "out_shards": [list(a) for a in q.shards], "pass": "strided",
                      "launch": "hip graph replay" if args.graph == "on" else "eager"},
           "roofline": roof, "kernels": kernels}
    if args.graph == "on":
        out["eager_ms_per_step"] = round(eager_ms, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_strided(args, wl, w, s)
    print(json.dumps(out), flush=True)


def bench_transposed(args, wl_out):
    """Upsampling conv of a decoder stage: an input at half the layer's
    resolution (every shard's extents halved, Cin channels, the layer's
    operand type, halo ksize/2), halo exchange, and a stride-2 transposed conv
    into the fp32 output plan the library derives, which has the layer's
    volume and sharding shapes."""
    import dataclasses

    import numpy as np
    import torch

    import halo_sharded_conv_amd as hsc
    import synth
    from halo_sharded_conv_amd.layer import ShardedConvGN

    s = 2
    if any(e % s for a in wl_out.shards for e in a):
        raise SystemExit(f"{wl_out.name}: shard sizes are not multiples of the stride")
    wl = dataclasses.replace(wl_out, name=wl_out.name + "_half", spatial=tuple(n // s for n in wl_out.spatial),
                             shards=tuple(tuple(e // s for e in a) for a in wl_out.shards))
    layer = ShardedConvGN(wl)
    layer.load_input(synth.make_input(wl))
    w = synth.make_weight(wl)                                   # [Cout][Cin][k..] bits
    # the transposed conv's weight [in = Cin][out = Cout]: the same bits with
    # the two channel axes swapped
    wtr = np.ascontiguousarray(np.swapaxes(w, 0, 1))
    wt = torch.from_numpy(np.ascontiguousarray(wtr.view(np.int16) if wtr.dtype == np.uint16 else wtr).reshape(-1)).cuda()
    q = hsc.st_plan_transposed(layer.in_plan, wl.ksize, s, wl.cout)
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(q.num_shards)]
    ws = torch.empty(hsc.st_conv_transposed_workspace_bytes(layer.in_plan, wl.cout, wl.ksize), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    stages = [("halo_pack", lambda: layer.exchange_pack()), ("halo_unpack", lambda: layer.exchange_unpack()),
              ("transposed", lambda: hsc.st_conv_transposed_sharded(layer.in_plan, layer.x_bufs, wt, None, wl.ksize,
                                                                    s, q, outs, ws))]
    per_kernel_ms, ms_per_step, gpu_ms = time_stages(args, stages, torch.cuda.current_stream())
    eager_ms = ms_per_step
    if args.graph == "on":
        ms_per_step, gpu_ms = time_graph(args, stages)
    esize = 4 if wl.dtype == "f32" else 2
    out_vox = wl.batch * int(np.prod([sum(a) for a in q.shards]))
    # taps that reach an output, summed over the s^d phases of one input cell
    p = wl.ksize // 2
    per_axis = sum(len(range((r + p) % s, wl.ksize, s)) for r in range(s))
    flops = 2 * wl.voxels * per_axis ** wl.ndim * wl.cin * wl.cout
    alg = {"halo_pack": 2 * layer.in_plan.msg_bytes, "halo_unpack": 2 * layer.in_plan.msg_bytes,
           "transposed": wl.voxels * wl.cin * esize + out_vox * wl.cout * 4}
    kernels = {}
    for key, ms in per_kernel_ms.items():
        gbs = alg[key] / (ms * 1e-3) / 1e9
        kernels[key] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof = shape_change_roofline(wl, "transposed", per_kernel_ms["transposed"], flops, alg["transposed"], kernels,
                                 load_traffic(wl_out, "transposed"))
    out = {"metric": METRIC_TRANSPOSED, "value": out_vox / (ms_per_step * 1e-3), "unit": "voxels/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32" if roof["bound"] == "alu" else "bf16", "data": "synthetic",
           "config": {"workload": wl_out.name, "input_shape": [wl.batch, wl.cin, *wl.spatial], "cout": wl.cout,
                      "kernel": wl.ksize, "stride": s, "operands": wl.dtype,
                      "in_shards": [list(a) for a in wl.shards], "out_shards": [list(a) for a in q.shards],
                      "pass": "transposed", "launch": "hip graph replay" if args.graph == "on" else "eager"},
           "roofline": roof, "kernels": kernels}
    if args.graph == "on":
        out["eager_ms_per_step"] = round(eager_ms, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_transposed(args, wl, wtr, s)
    print(json.dumps(out), flush=True)


def bench_pool(args, wl):
    """Downsampling of the layer's input shards: halo exchange (halo 1 = k - 1)
    and 'valid' 2x2(x2) average pooling into the output plan the library
    derives, in the input's type."""
    import numpy as np
    import torch

    import halo_sharded_conv_amd as hsc
    import synth

    k = s = 2
    d = wl.ndim
    tdt = torch.float32 if wl.dtype == "f32" else torch.int16
    p = hsc.st_plan_shards(d, wl.batch, wl.cin, wl.spatial, wl.shards, [k - 1] * d, wl.dtype)
    q = hsc.st_plan_pooled(p, k, s)
    bufs = [torch.zeros(p.shard_info(i)["elems"], dtype=tdt, device="cuda") for i in range(p.num_shards)]
    x = synth.make_input(wl)
    xs = x.view(np.int16) if x.dtype == np.uint16 else x
    for i in range(p.num_shards):
        inf = p.shard_info(i)
        v = bufs[i].view(p.padded_shape(i))
        v[tuple([slice(None)] + [slice(1, 1 + e) for e in inf["extent"]] + [slice(None)])].copy_(
            torch.from_numpy(np.ascontiguousarray(xs[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])])))
    msg = torch.zeros(max(16, p.msg_bytes), dtype=torch.uint8, device="cuda")
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=tdt, device="cuda") for i in range(q.num_shards)]
    torch.cuda.synchronize()
    stages = [("halo_pack", lambda: hsc.st_halo_pack(p, bufs, msg)),
              ("halo_unpack", lambda: hsc.st_halo_unpack(p, msg, bufs, True)),
              ("pool", lambda: hsc.st_pool_sharded(p, bufs, k, s, "avg", q, outs))]
    per_kernel_ms, ms_per_step, gpu_ms = time_stages(args, stages, torch.cuda.current_stream())
    eager_ms = ms_per_step
    if args.graph == "on":
        ms_per_step, gpu_ms = time_graph(args, stages)
    esize = 4 if wl.dtype == "f32" else 2
    out_vox = wl.batch * int(np.prod([sum(a) for a in q.shards]))
    alg = {"halo_pack": 2 * p.msg_bytes, "halo_unpack": 2 * p.msg_bytes,
           "pool": wl.voxels * wl.cin * esize + out_vox * wl.cin * esize}
    kernels = {}
    for key, ms in per_kernel_ms.items():
        gbs = alg[key] / (ms * 1e-3) / 1e9
        kernels[key] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof = {"bound": "hbm", "achieved": kernels["pool"]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kernels["pool"]["GB/s"] / HBM_PEAK_GBS, 4), "kernel": "pool",
            "traffic": load_traffic(wl, "pool")}
    out = {"metric": METRIC_POOL, "value": wl.voxels / (ms_per_step * 1e-3), "unit": "voxels/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "gpu_ms_per_step": round(gpu_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if wl.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": wl.name, "shape": [wl.batch, wl.cin, *wl.spatial], "pool": "avg k2 s2",
                      "shards": [list(a) for a in wl.shards], "out_shards": [list(a) for a in q.shards],
                      "pass": "pool", "launch": "hip graph replay" if args.graph == "on" else "eager"},
           "roofline": roof, "kernels": kernels}
    if args.graph == "on":
        out["eager_ms_per_step"] = round(eager_ms, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_pool(args, wl, k, s)
    print(json.dumps(out), flush=True)



def _threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def cpu_baseline_strided(args, wl, w, s):
    """The oracle's stride-s conv on the first rows of the input."""
    import numpy as np

    import oracle
    import synth
    rows = args.cpu_rows or max(s, min(wl.spatial[0], int(1.0e6 // (wl.voxels // wl.spatial[0]) + 1)) // s * s)
    sub_shape = (rows,) + tuple(wl.spatial[1:])
    sub = synth.small_variant(wl, sub_shape, [(n,) for n in sub_shape], name_suffix="cpu_sample")
    xsub = oracle.widen(synth.make_input(sub), wl.dtype)
    wsub = oracle.widen(w, wl.dtype)
    t0 = time.perf_counter()
    y = oracle.conv_strided(xsub, wsub, s)
    dt = time.perf_counter() - t0
    return {"value": sub.voxels / dt, "unit": "voxels/s", "cores": _threads(), "kind": "oracle",
            "sample": f"first {rows} rows of the outermost axis ({sub.voxels} input voxels, "
                      f"stride-{s} conv in fp64 numpy, {dt:.2f} s)", "seconds": round(dt, 3),
            "checksum": float(np.abs(y).sum())}


def cpu_baseline_transposed(args, wl, wtr, s):
    """The oracle's stride-s transposed conv on the first rows of the input."""
    import numpy as np

    import oracle
    import synth
    rows = args.cpu_rows or max(1, min(wl.spatial[0], int(0.5e6 // (wl.voxels // wl.spatial[0]) + 1)))
    sub_shape = (rows,) + tuple(wl.spatial[1:])
    sub = synth.small_variant(wl, sub_shape, [(n,) for n in sub_shape], name_suffix="cpu_sample")
    ysub = oracle.widen(synth.make_input(sub), wl.dtype)
    wtr64 = oracle.widen(wtr, wl.dtype)
    t0 = time.perf_counter()
    x = oracle.conv_transposed(ysub, wtr64, s)
    dt = time.perf_counter() - t0
    return {"value": x.shape[0] * int(np.prod(x.shape[1:-1])) / dt, "unit": "voxels/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"first {rows} rows of the input's outermost axis ({sub.voxels} input, "
                      f"{sub.voxels * s ** wl.ndim} output voxels, transposed conv in fp64 numpy, {dt:.2f} s)",
            "seconds": round(dt, 3), "checksum": float(np.abs(x).sum())}


def cpu_baseline_pool(args, wl, k, s):
    """The oracle's 'valid' average pooling on the first rows of the input."""
    import numpy as np

    import oracle
    import synth
    rows = args.cpu_rows or max(2, min(wl.spatial[0], int(2.0e6 // (wl.voxels // wl.spatial[0]) + 1)) // 2 * 2)
    sub_shape = (rows,) + tuple(wl.spatial[1:])
    sub = synth.small_variant(wl, sub_shape, [(n,) for n in sub_shape], name_suffix="cpu_sample")
    xsub = oracle.widen(synth.make_input(sub), wl.dtype)
    t0 = time.perf_counter()
    y = oracle.pool_valid(xsub, k, s, "avg")
    dt = time.perf_counter() - t0
    return {"value": sub.voxels / dt, "unit": "voxels/s", "cores": _threads(), "kind": "oracle",
            "sample": f"first {rows} rows of the outermost axis ({sub.voxels} voxels, 'valid' "
                      f"average pooling in fp64 numpy, {dt:.2f} s)", "seconds": round(dt, 3),
            "checksum": float(np.abs(y).sum())}

def report(args, wl, layer, per_kernel_ms, ms_per_step, gpu_ms, metric, w_fwd, dgrad_layer=None, eager_ms=None,
           cold=None, cpu=True):
    """One JSON line: throughput, per-stage rates and the longest stage against its roofline."""
    alg = algorithmic(wl, layer)
    if dgrad_layer is not None:
        # the exchange and the conv run on the input-gradient layer
        d_alg = algorithmic(dgrad_layer.cfg, dgrad_layer)
        for k in ("halo_pack", "halo_unpack", "halo_exchange", "conv"):
            alg[k] = d_alg[k]
    kernels = {}
    for k, ms in per_kernel_ms.items():
        rec = {"ms": round(ms, 5)}
        if alg[k].get("bytes"):
            rec["GB/s"] = round(alg[k]["bytes"] / (ms * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(rec["GB/s"] / HBM_PEAK_GBS, 4)
        if alg[k].get("flops"):
            peak = FP32_PEAK_TFLOPS if wl.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
            rec["TFLOP/s"] = round(alg[k]["flops"] / (ms * 1e-3) / 1e12, 2)
            rec["mfma_frac"] = round(rec["TFLOP/s"] / peak, 4)
            if alg[k].get("bytes"):
                # attainable roofline: min(compute peak, arithmetic intensity x HBM peak)
                attain = min(peak, alg[k]["flops"] / alg[k]["bytes"] * HBM_PEAK_GBS / 1e3)
                rec["attainable_frac"] = round(rec["TFLOP/s"] / attain, 4)
        kernels[k] = rec

    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    if alg[dom].get("flops"):
        ai = alg[dom]["flops"] / alg[dom]["bytes"]
        peak_t = FP32_PEAK_TFLOPS if wl.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        ridge = peak_t * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai < ridge:
            roof = {"bound": "hbm", "achieved": kernels[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        else:
            # fp32 layers run on the vector ALUs (fp32 FMA), bf16 layers on the matrix cores
            roof = {"bound": "alu" if wl.dtype == "f32" else "mfma", "achieved": kernels[dom]["TFLOP/s"],
                    "peak": peak_t, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kernels[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(wl, dom)

    out = {
        "metric": metric,
        "value": wl.voxels / (ms_per_step * 1e-3),
        "unit": "voxels/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "shape": [wl.batch, wl.cin, *wl.spatial], "cout": wl.cout,
                   "kernel": wl.ksize, "shards": [list(s) for s in wl.shards], "halo": wl.halo, "exchange": args.exchange, "pass": args.pass_,
                   "groups": wl.groups, "accumulate": "f32", "outputs": "f32",
                   "launch": "hip graph replay" if eager_ms is not None else "eager"},
        "roofline": roof,
        "kernels": kernels,
    }
    if eager_ms is not None:
        out["eager_ms_per_step"] = round(eager_ms, 4)
    if cold is not None:
        out["cold_eager"] = cold
    if cpu and not args.no_cpu_baseline:
        progress(f"{wl.name}: oracle CPU baseline on {cpu_rows(args, wl)} rows")
        out["cpu_baseline"] = cpu_baseline(wl, cpu_rows(args, wl), w_fwd, backward=args.pass_ == "backward")
    return out


def cpu_rows(args, wl):
    """Rows of the outermost axis in the oracle's CPU sample: about 300 GFLOP
    of fp64 conv (~10-30 s on the host), at least one row."""
    if args.cpu_rows:
        return args.cpu_rows
    per_row = wl.conv_flops // wl.spatial[0]
    return max(1, min(wl.spatial[0], int(300e9 // per_row)))


if __name__ == "__main__":
    main()
