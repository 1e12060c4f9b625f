#!/usr/bin/env python3
"""Throughput of the Hyena-SE / Hyena-MR forward on one MI355X.

One step = one pass of the whole forward path over one batch of synthetic
input: a Hyena-SE layer (l_h = 7) and then a Hyena-MR layer (l_h = 128), each
y = q (.) (h * (k (.) v)) at B = 1, L = 8192, D = 4096, 16 channels per
filter group, bf16 I/O with fp32 accumulation, with independent seeded inputs
per layer (the two layers of a striped block at the 8K pretraining context).
``--workload`` selects another shape for exploration (se, mr, mr_b4,
long_stripe); the default line is the stripe.

Reported (one JSON line):
  value        whole-step throughput, G(token*channel)/s = 2 * B*L*D / step time
               (both layers count), inputs resident in HBM;
  roofline     the dominant kernel, the layer whose launches took longer in
               this run (MR and SE now take about the same time, so either
               can be reported; `kernel` names it): algorithmic bytes per
               launch (q, k, v read once, y written once: 8 B per
               token*channel) / its mean launch time from HIP events on the
               launch stream (one event per kernel boundary in every step of
               an evented pass of max(K, 20) steps right after the timed
               region; the timed region itself carries events in every 5th
               step, reported beside), against the 8 TB/s HBM3E peak; `traffic` is the
               measured HBM bytes per launch from the committed rocprofv3
               counter summary, or null if the kernel code changed since;
  layers       the same figures for each layer's kernel;
  chunk_direction  each layer with one filter per channel: the direct kernel
               (8 taps or fewer) or the chunk-direction GEMM kernel, each
               with its backward;
  long_filter  a filter as long as the sequence (the FFT path), with the
               filter spectra computed per call and kept across calls, and
               its backward (dq, dk, dv, dh);
  backward     dq, dk, dv and dh of each layer;
  stream_reference  a hand-written read-3/write-1 streaming kernel with the
               forward's access pattern (256- and 512-byte row segments; the
               attainable rate on the box), torch's addcmul and a copy over the
               same bytes; each layer's `frac_of_attainable` divides by the best;
  cpu_baseline the fp64 oracle on the host cores over the full step's inputs;
  naive_conv1d the same step written with torch's depthwise F.conv1d (bf16),
               with and without the layout permutes;
  extra_shapes the MR layer at B=4, L=32768, and the 2^20-row stripe (SE then
               MR; step time and per-layer launches), unless --skip-extra-shapes;
  halo_shard   (with --halo) the second half of the MR layer through the
               history-prefix entry point, beside the plain forward.
Input sets rotate over ``--sets`` copies per layer so that no launch finds its
operands in the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Hyena-SE/MR fwd: G(token·channel)/s and % of HBM-bandwidth roofline, D=4096"
UNIT = "G(token·channel)/s"
HBM_PEAK_GBS = 8000.0
EVENT_EVERY = 5          # per-kernel events in every 5th timed step (coprime with the input sets)
MIN_EVENT_STEPS = 20     # the evented pass after the timed region has at least this many steps
KERNEL_SRC = os.path.join(ROOT, "gated_convolution_sequence_amd", "csrc", "hyena_conv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOAD_LAYERS = {
    "stripe_8k": ["se", "mr"],
    "se": ["se"],
    "mr": ["mr"],
    "mr_b4": ["mr_b4"],
    "long_stripe": ["long_se", "long_mr"],
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stripe_8k", choices=sorted(WORKLOAD_LAYERS))
    ap.add_argument("--sets", type=int, default=4, help="input copies per layer (cache rotation)")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-naive", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--skip-chunk-direction", action="store_true")
    ap.add_argument("--skip-long-filter", action="store_true")
    ap.add_argument("--halo", action="store_true",
                    help="also time one shard of the MR layer through hyena_conv_fwd_halo (the second half "
                         "of the sequence with its l_h - 1 prefix rows); off by default because its "
                         "launches share the MR layer's kernel instance")
    ap.add_argument("--skip-extra-shapes", action="store_true",
                    help="leave out the batched MR layer (B=4, L=32768) and the 2^20-row stripe; their "
                         "launches share kernel instances with the default step's layers, so a "
                         "profiler's per-kernel statistics of the step need this flag")
    ap.add_argument("--skip-stream-reference", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="rough CPU budget of the oracle baseline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="instead of the step, run a plain device copy of this many MiB "
                         "(reference point for the HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                    "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output of this bench and of "
                         "--calibrate-copy-mib into profiles/traffic.json")
    return ap.parse_args()


def _counter_means(d):
    """{kernel name: mean Counter_Value} over the dispatches in a rocprofv3 --pmc output dir."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                k = r["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib=1024):
    """HBM bytes per launch of each layer's kernel, scaled by a plain copy's counters.

    FETCH_SIZE / WRITE_SIZE are in KiB per dispatch.  The copy of ``copy_mib``
    MiB reads and writes exactly that many bytes; the ratio of that figure to
    its counter readings scales the kernel's readings to bytes.
    """
    import re
    copy_bytes = copy_mib << 20

    def copy_reading(d):
        m = _counter_means(d)
        k = [n for n in m if "copyBuffer" in n or "copy" in n.lower()]
        return max(m[n] for n in k) * 1024.0

    f_scale = copy_bytes / copy_reading(copy_fetch_dir)
    w_scale = copy_bytes / copy_reading(copy_write_dir)
    fetch, write = _counter_means(fetch_dir), _counter_means(write_dir)
    layers = {}
    for name, kib in fetch.items():
        m = re.search(r"hyena_fwd_kernel<false, (\d+), (\d+), (\d+)(?:, false, false(?:, \d+)?)?>", name)
        if not m:
            continue
        kh = int(m.group(1))
        layer = {1: "se", 4: "mr"}.get(kh)
        if layer is None:
            continue
        fb = kib * 1024.0 * f_scale
        wb = write.get(name, float("nan")) * 1024.0 * w_scale
        layers[layer] = {"kernel": m.group(0), "fetch_bytes": round(fb),
                         "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb),
                         "fetch_counter_KiB": round(kib, 1),
                         "write_counter_KiB": round(write.get(name, float("nan")), 1)}
    out = {"kernel_source_sha256": source_digest(),
           "scale": {"fetch": round(f_scale, 4), "write": round(w_scale, 4),
                     "copy_bytes": copy_bytes},
           "layers": layers,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -o run -- "
               "python3 bench.py --steps 8 --warmup 2 --skip-cpu-baseline --skip-naive --skip-extra-shapes "
               "--skip-stream-reference",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -o run -- "
               "python3 bench.py --steps 8 --warmup 2 --skip-cpu-baseline --skip-naive --skip-extra-shapes "
               "--skip-stream-reference",
               "rocprofv3 --pmc FETCH_SIZE ... -- python3 bench.py --calibrate-copy-mib %d" % copy_mib,
               "rocprofv3 --pmc WRITE_SIZE ... -- python3 bench.py --calibrate-copy-mib %d" % copy_mib]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def calibrate_copy(mib: int, reps: int = 10):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE give the counter scale."""
    import torch
    n = mib << 20
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def source_digest() -> str:
    """SHA-256 of the kernel source's code: comments, blank lines and trailing
    spaces removed, so that a comment edit keeps the counters current while any
    change to the code itself makes them stale."""
    import re
    with open(KERNEL_SRC, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.split("\n") if line.strip())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()


def measured_traffic(layer: str):
    """HBM bytes per launch from the committed counter summary, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != source_digest():
        return None
    entry = t.get("layers", {}).get(layer)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this operator is benchmarked on a single MI355X; "
              "--gpus %d is not supported (a longer sequence splits into row shards, each run "
              "with hyena_conv_fwd_halo on its own GPU)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return

    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import WORKLOADS, make_inputs

    if not os.path.exists(hc.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    layer_names = WORKLOAD_LAYERS[args.workload]
    layers = [WORKLOADS[n] for n in layer_names]

    # ---- inputs: set 0 from the seeds, further sets are copies -------------
    t_gen = time.time()
    sets = []
    for w in layers:
        q, k, v, h = make_inputs(w, dev)
        n_sets = args.sets if w.elems * 8 * args.sets <= (64 << 30) else 1
        per = [(q, k, v, h, torch.empty_like(q))]
        for _ in range(n_sets - 1):
            per.append((q.clone(), k.clone(), v.clone(), h, torch.empty_like(q)))
        sets.append(per)
    torch.cuda.synchronize()
    print("inputs ready in %.1fs" % (time.time() - t_gen), file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(i, events=None):
        # events[0] before the first layer, events[li + 1] after layer li:
        # one timestamp per kernel boundary
        if events is not None:
            hip_ev.record(events[0], stream)
        for li, w in enumerate(layers):
            q, k, v, h, y = sets[li][i % len(sets[li])]
            hc.conv_fwd(q, k, v, h, w.group_size, out=y, stream=stream)
            if events is not None:
                hip_ev.record(events[li + 1], stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ------------------------------------
    # Every EVENT_EVERY-th step records one HIP event per kernel boundary on
    # the launch stream (the per-kernel durations of the roofline).  The
    # events skip the system-scope fence: a default event writes back and
    # invalidates the caches, which costs about 2 us per record here and
    # lengthens the kernels it brackets.
    K = args.steps
    sampled = list(range(0, K, EVENT_EVERY))
    hip_ev = HipEvents()
    ev = {i: [hip_ev.create() for _ in range(len(layers) + 1)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, ev.get(i))
    t_issued = time.perf_counter()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    host_issue_us = (t_issued - t0) * 1e6 / K
    ms_per_step = wall * 1e3 / K

    elems_step = sum(w.elems for w in layers)
    value = elems_step / (wall / K) / 1e9
    timed_ms = [[hip_ev.elapsed_ms(ev[i][li], ev[i][li + 1]) for i in sampled] for li in range(len(layers))]

    # ---- evented pass: the same steps with one event per kernel boundary in
    # every step (at least MIN_EVENT_STEPS), after the timed region so that
    # its wall clock carries no event records beyond the sampled ones
    n_ev = max(K, MIN_EVENT_STEPS)
    ev2 = [[hip_ev.create() for _ in range(len(layers) + 1)] for _ in range(n_ev)]
    for i in range(n_ev):
        step(K + i, ev2[i])
    torch.cuda.synchronize()

    layer_stats = {}
    for li, w in enumerate(layers):
        ms = [hip_ev.elapsed_ms(e[li], e[li + 1]) for e in ev2]
        mean_ms = sum(ms) / len(ms)
        alg_bytes = w.elems * (4 * (2 if w.dtype == "bf16" else 4))
        achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
        span, wgs = hc.plan(w.B, w.L, w.D, w.group_size, w.l_h,
                            hc.DTYPE_BF16 if w.dtype == "bf16" else hc.DTYPE_F32)
        layer_stats[w.name] = {
            "B": w.B, "L": w.L, "D": w.D, "l_h": w.l_h, "kernel_KH": (w.l_h - 1 + 31) // 32,
            "mean_us": round(mean_ms * 1e3, 2), "median_us": round(statistics.median(ms) * 1e3, 2),
            "p10_us": round(sorted(ms)[len(ms) // 10] * 1e3, 2),
            "p90_us": round(sorted(ms)[(9 * len(ms)) // 10] * 1e3, 2),
            "G_tok_ch_per_s": round(w.elems / (mean_ms * 1e-3) / 1e9, 2),
            "alg_bytes": alg_bytes, "achieved_GBs": round(achieved, 1),
            "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
            "span_chunks": span, "workgroups": wgs, "event_samples": len(ms),
            "timed_region_mean_us": round(sum(timed_ms[li]) / len(timed_ms[li]) * 1e3, 2),
            "timed_region_event_samples": len(timed_ms[li]),
        }
    dom = max(layer_stats, key=lambda n: layer_stats[n]["mean_us"])
    d = layer_stats[dom]
    traffic = measured_traffic(dom)
    roofline = {"bound": "hbm", "achieved": d["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["achieved_GBs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "hyena_fwd_kernel<bf16, KH=%d> (%s layer)" % (d["kernel_KH"], dom),
                "alg_bytes_per_launch": d["alg_bytes"], "mean_launch_us": d["mean_us"],
                "event_samples": d["event_samples"]}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": UNIT, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if layers[0].dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q,k,v; Gaussian SE taps, decaying MR taps)",
        "config": {"workload": "%s: %s" % (args.workload, " then ".join(
            "%s(B=%d,L=%d,D=%d,group_size=%d,l_h=%d)" % (w.name, w.B, w.L, w.D, w.group_size, w.l_h)
            for w in layers)), "l_b": 64, "input_sets_rotated": len(sets[0])},
        "roofline": roofline,
        "layers": layer_stats,
        "host_issue_us_per_step": round(host_issue_us, 2),
    }

    # ---- one filter per channel (chunk-direction kernel), same layers -------
    if not args.skip_chunk_direction:
        out["chunk_direction"] = chunk_direction_rates(layers, sets, stream, max(MIN_EVENT_STEPS, K))

    # ---- a long filter (FFT convolution path), at the first layer's shape --
    if not args.skip_long_filter:
        out["long_filter"] = long_filter_rates(layers[0], stream, max(MIN_EVENT_STEPS, K))

    # ---- backward of each layer (outside the forward step's timed region)
    if not args.skip_backward:
        out["backward"] = backward_rates(layers, sets, stream, max(MIN_EVENT_STEPS, K))

    if args.halo:
        out["halo_shard"] = halo_shard_rate(layers[-1], sets[-1], stream, max(20, K // 4))

    # ---- attainable streaming rate on this GPU (same bytes, no convolution)
    if not args.skip_stream_reference:
        ref = stream_reference(layers[-1], sets[-1], stream, max(MIN_EVENT_STEPS, K))
        out["stream_reference"] = ref
        att = ref.get("attainable_GBs")
        if att:
            for st in layer_stats.values():
                st["frac_of_attainable"] = round(st["achieved_GBs"] / att, 4)
            roofline["frac_of_attainable"] = round(d["achieved_GBs"] / att, 4)


    # ---- naive baseline: torch depthwise conv1d ---------------------------
    if not args.skip_naive:
        out["naive_conv1d"] = naive_conv1d(layers, sets, stream, max(5, K // 10))

    # ---- CPU baseline: the oracle on the host -----------------------------
    if not args.skip_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, sets, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    # ---- the other workload shapes: batched MR and the 2^20-row stripe -----
    if not args.skip_extra_shapes and args.workload == "stripe_8k":
        sets.clear()  # the step's inputs are no longer needed
        torch.cuda.empty_cache()
        out["extra_shapes"] = {
            "mr_b4": batched_mr_rate(stream, max(MIN_EVENT_STEPS, K)),
            "long_stripe": long_stripe_rate(stream, max(MIN_EVENT_STEPS, K)),
        }
    print(json.dumps(out), flush=True)


def backward_rates(layers, sets, stream, reps):
    """Time hyena_conv_bwd (dq, dk, dv, dh) per layer on rotated inputs.

    Minimal traffic of the backward is 14 B per token*channel in bf16 (q, k,
    v, dy read once; dq, dk, dv written once).  The library's bf16 backward
    is one pass over the rows that moves those bytes (q, k, v, dy -> dq, dk,
    dv, partial dh), plus a small reduction of the partial dh; each span of
    16 chunks also reads the 32*KH rows of k, v before it and of q, dy after
    it, and reads k, v again as the dk, dv gates (mostly L2 hits).  fp32
    runs dq, dk/dv and dh as separate passes: 14 element-widths (56 B).
    """
    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import normal_activation
    res = {}
    for li, w in enumerate(layers):
        per = sets[li]
        dys = [normal_activation((w.B, w.L, w.D), w.torch_dtype, per[0][0].device, w.seed + 9 + i)
               for i in range(len(per))]
        code = hc.DTYPE_BF16 if w.dtype == "bf16" else hc.DTYPE_F32
        dq, dk, dv = (torch.empty_like(per[0][0]) for _ in range(3))
        dh = torch.empty((w.G, w.l_h), dtype=torch.float32, device=per[0][0].device)
        ws_n = hc.bwd_workspace_bytes(w.B, w.L, w.D, w.group_size, w.l_h, code)
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=per[0][0].device)
        fn = hc.lib().hyena_conv_bwd

        def call(i):
            q, k, v, h, _ = per[i % len(per)]
            st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), h.data_ptr(), dys[i % len(per)].data_ptr(),
                    w.B, w.L, w.D, w.group_size, w.l_h, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    dh.data_ptr(), ws.data_ptr(), ws_n, code, stream.cuda_stream)
            if st != 0:
                raise hc.HyenaError(st, "hyena_conv_bwd")
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        eb = 2 if w.dtype == "bf16" else 4
        moved = (7 if w.dtype == "bf16" else 14) * eb * w.elems  # element accesses x width
        res[w.name] = {"us": round(us, 2), "G_tok_ch_per_s": round(w.elems / (us * 1e-6) / 1e9, 2),
                       "min_bytes": 7 * eb * w.elems, "moved_bytes": moved,
                       "GBs_vs_min_bytes": round(7 * eb * w.elems / (us * 1e-6) / 1e9, 1),
                       "GBs_moved": round(moved / (us * 1e-6) / 1e9, 1),
                       "kernels": 2 if w.dtype == "bf16" else 4, "workspace_bytes": ws_n}
        del dys
    return res


class HipEvents:
    """HIP timing events without the system-scope fence (hipEventDisableSystemFence),
    created in the HIP runtime this process already loaded (the one torch and the
    library use, so torch's stream handles are valid).  Only timestamps are
    read, after a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)
        self.events = []

    def create(self):
        e = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags: %d" % rc)
        self.events.append(e)
        return e

    def record(self, e, stream):
        rc = self.lib.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord: %d" % rc)

    def elapsed_ms(self, a, b):
        f = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime: %d" % rc)
        return f.value


def halo_shard_rate(w, per, stream, reps):
    """One shard of a layer as one of two GPUs would run it: rows [L/2, L)
    through hyena_conv_fwd_halo with the l_h - 1 rows before L/2 as the
    prefix, next to the plain forward of an L/2-row sequence (no prefix).
    Mean launch times from fence-free HIP events; the input sets rotate."""
    import torch
    import gated_convolution_sequence_amd as hc
    s, P = w.L // 2, w.l_h - 1
    shards = []
    for (q, k, v, h, _) in per:
        sl = lambda a: a[:, s:].contiguous()
        pre = lambda a: a[:, s - P:s].contiguous()
        shards.append((sl(q), sl(k), sl(v), h, pre(k), pre(v), torch.empty_like(sl(q))))
    ev = HipEvents()

    def timed(with_prefix):
        for i in range(3):
            q, k, v, h, kp, vp, y = shards[i % len(shards)]
            hc.conv_fwd(q, k, v, h, w.group_size, out=y, stream=stream,
                        k_prev=kp if with_prefix else None, v_prev=vp if with_prefix else None)
        torch.cuda.synchronize()
        marks = [(ev.create(), ev.create()) for _ in range(reps)]
        for i, (e0, e1) in enumerate(marks):
            q, k, v, h, kp, vp, y = shards[i % len(shards)]
            ev.record(e0, stream)
            hc.conv_fwd(q, k, v, h, w.group_size, out=y, stream=stream,
                        k_prev=kp if with_prefix else None, v_prev=vp if with_prefix else None)
            ev.record(e1, stream)
        torch.cuda.synchronize()
        return sum(ev.elapsed_ms(e0, e1) for e0, e1 in marks) / reps
    t_halo, t_plain = timed(True), timed(False)
    alg = 8 * w.B * (w.L - s) * w.D
    res = {"layer": w.name, "B": w.B, "rows": w.L - s, "prefix_rows": P, "D": w.D, "l_h": w.l_h,
           "halo_us": round(t_halo * 1e3, 2), "plain_us": round(t_plain * 1e3, 2),
           "halo_hbm_frac": round(alg / (t_halo * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "plain_hbm_frac": round(alg / (t_plain * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "launches": reps}
    del shards
    torch.cuda.empty_cache()
    return res


def _evented_launches(call, reps, stream):
    """Per-launch durations (ms) of ``reps`` calls, each between two fence-free
    HIP events on the launch stream, after three untimed calls."""
    import torch
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    ev = HipEvents()
    marks = [(ev.create(), ev.create()) for _ in range(reps)]
    for i, (e0, e1) in enumerate(marks):
        ev.record(e0, stream)
        call(i)
        ev.record(e1, stream)
    torch.cuda.synchronize()
    return [ev.elapsed_ms(e0, e1) for e0, e1 in marks]


def _launch_stats(w, ms):
    mean_ms = sum(ms) / len(ms)
    alg = 8 * w.elems
    import gated_convolution_sequence_amd as hc
    span, wgs = hc.plan(w.B, w.L, w.D, w.group_size, w.l_h, hc.DTYPE_BF16)
    return {"B": w.B, "L": w.L, "D": w.D, "group_size": w.group_size, "l_h": w.l_h,
            "mean_us": round(mean_ms * 1e3, 1), "median_us": round(statistics.median(ms) * 1e3, 1),
            "p10_us": round(sorted(ms)[len(ms) // 10] * 1e3, 1),
            "p90_us": round(sorted(ms)[(9 * len(ms)) // 10] * 1e3, 1),
            "G_tok_ch_per_s": round(w.elems / (mean_ms * 1e-3) / 1e9, 2),
            "alg_bytes": alg, "achieved_GBs": round(alg / (mean_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "span_chunks": span, "workgroups": wgs, "event_samples": len(ms)}


def batched_mr_rate(stream, reps):
    """The MR layer at B=4, L=32768, D=4096 (4 GiB of q, k, v and y per input
    set; two sets alternate): per-launch durations from fence-free HIP events
    around each launch, and the fraction of the HBM peak at 8 B per
    token*channel."""
    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["mr_b4"]
    q, k, v, h = make_inputs(w, torch.device("cuda:0"))
    sets = [(q, k, v, torch.empty_like(q)), (q.clone(), k.clone(), v.clone(), torch.empty_like(q))]

    def call(i):
        a, b, c, y = sets[i % 2]
        hc.conv_fwd(a, b, c, h, w.group_size, out=y, stream=stream)
    res = _launch_stats(w, _evented_launches(call, reps, stream))
    del sets, q, k, v, h
    torch.cuda.empty_cache()
    return res


def long_stripe_rate(stream, steps):
    """The 2^20-row stripe (an SE layer, then an MR layer, B=1, D=4096; one
    input set per layer, 32 GiB each, so nothing stays in a cache between
    launches): the wall-clock time of ``steps`` steps between two device
    synchronisations, and each layer's per-launch durations from fence-free
    HIP events in every step."""
    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import WORKLOADS, make_inputs
    ws = [WORKLOADS["long_se"], WORKLOADS["long_mr"]]
    dev = torch.device("cuda:0")
    data = []
    for w in ws:
        q, k, v, h = make_inputs(w, dev)
        data.append((q, k, v, h, torch.empty_like(q)))
    torch.cuda.synchronize()

    def step(events=None):
        if events is not None:
            hip_ev.record(events[0], stream)
        for li, w in enumerate(ws):
            q, k, v, h, y = data[li]
            hc.conv_fwd(q, k, v, h, w.group_size, out=y, stream=stream)
            if events is not None:
                hip_ev.record(events[li + 1], stream)
    hip_ev = HipEvents()
    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    evs = [[hip_ev.create() for _ in range(len(ws) + 1)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    res = {"workload": "long_se(B=1,L=1048576,D=4096,group_size=16,l_h=7) then "
                       "long_mr(B=1,L=1048576,D=4096,group_size=16,l_h=128)",
           "steps": steps, "ms_per_step": round(wall * 1e3, 3),
           "value": round(sum(w.elems for w in ws) / wall / 1e9, 2), "unit": UNIT,
           "hbm_frac_step": round(sum(8 * w.elems for w in ws) / wall / 1e9 / HBM_PEAK_GBS, 4), "layers": {}}
    for li, w in enumerate(ws):
        res["layers"][w.name] = _launch_stats(w, [hip_ev.elapsed_ms(e[li], e[li + 1]) for e in evs])
    del data
    torch.cuda.empty_cache()
    return res


def chunk_direction_rates(layers, sets, stream, reps):
    """Each layer with group_size 1: every channel its own filter (its group's
    taps repeated, so the result is the grouped layer's), which runs the
    direct kernel (8 taps or fewer) or the chunk-direction kernel.  Timed back
    to back on the rotated inputs."""
    import torch
    import gated_convolution_sequence_amd as hc
    res = {}
    for li, w in enumerate(layers):
        per = sets[li]
        h1 = torch.repeat_interleave(per[0][3], w.group_size, dim=0).contiguous()

        def call(i):
            q, k, v, _, y = per[i % len(per)]
            hc.conv_fwd(q, k, v, h1, 1, out=y, stream=stream)
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        alg = w.elems * (8 if w.dtype == "bf16" else 16)
        span, wgs = hc.plan(w.B, w.L, w.D, 1, w.l_h, hc.DTYPE_BF16 if w.dtype == "bf16" else hc.DTYPE_F32)
        res[w.name + "_gs1"] = {"group_size": 1, "us": round(us, 2),
                                "G_tok_ch_per_s": round(w.elems / (us * 1e-6) / 1e9, 2),
                                "achieved_GBs": round(alg / (us * 1e-6) / 1e9, 1),
                                "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "span_chunks": span, "workgroups": wgs,
                                "kernel": ("hyena_fwd_direct_kernel" if w.l_h <= 8 else "hyena_fwd_cd_kernel")}
        res[w.name + "_gs1"]["backward"] = _gs1_backward_rate(w, per, h1, stream, reps)
    return res


def _gs1_backward_rate(w, per, h1, stream, reps):
    """dq, dk, dv, dh with one filter per channel.  Up to 8 taps (the direct
    kernels): one walk backwards in time over q, k, v, dy and the per-group
    reduction.  Longer filters: the chunk-direction kernel for dq, the same
    walked backwards with two gates for dk and dv, the lag products of dh on
    the matrix cores (bf16) and the reduction."""
    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import normal_activation
    code = hc.DTYPE_BF16 if w.dtype == "bf16" else hc.DTYPE_F32
    dys = [normal_activation((w.B, w.L, w.D), w.torch_dtype, per[0][0].device, w.seed + 19 + i)
           for i in range(len(per))]
    dq, dk, dv = (torch.empty_like(per[0][0]) for _ in range(3))
    dh = torch.empty((w.D, w.l_h), dtype=torch.float32, device=per[0][0].device)
    ws_n = hc.bwd_workspace_bytes(w.B, w.L, w.D, 1, w.l_h, code)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=per[0][0].device)
    fn = hc.lib().hyena_conv_bwd

    def call(i):
        q, k, v, _, _ = per[i % len(per)]
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), h1.data_ptr(), dys[i % len(per)].data_ptr(),
                w.B, w.L, w.D, 1, w.l_h, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dh.data_ptr(),
                ws.data_ptr(), ws_n, code, stream.cuda_stream)
        if st != 0:
            raise hc.HyenaError(st, "hyena_conv_bwd")
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    eb = 2 if w.dtype == "bf16" else 4
    # direct: q, k, v, dy read once, dq, dk, dv written once, 7 element
    # accesses per token*channel (plus the l_h - 1 rows each span reads on
    # either side); longer filters: dq pass 4 (k, v, dy; dq), dk/dv pass 6
    # (dy, q, k, v; dk, dv), lag pass 4 (dy, q, k, v): 14
    direct = w.l_h <= 8
    moved = (7 if direct else 14) * eb * w.elems
    del dys
    return {"us": round(us, 2), "G_tok_ch_per_s": round(w.elems / (us * 1e-6) / 1e9, 2),
            "moved_bytes": moved, "GBs_moved": round(moved / (us * 1e-6) / 1e9, 1),
            "kernels": 2 if direct else 4, "workspace_bytes": ws_n}


def long_filter_rates(w, stream, reps):
    """hyena_conv_fwd_long at the layer's B, L, D and group size with a filter
    as long as the sequence (l_h = L, an LI-length filter), seeded inputs.

    Bytes the three transform kernels move per token*channel (N = 2L, bf16
    I/O, fp32 complex work area of one value per channel pair and point):
    rows 4 (k, v) + 8, columns 8 + 8, output 8 + 4 (q, y): 40 B, plus the
    filter pass.  The operator's own minimum is 8 B (q, k, v read, y written).
    """
    import torch
    import gated_convolution_sequence_amd as hc
    from workloads import make_inputs
    lw = w.with_(l_h=w.L, filt="se", seed=w.seed + 50)
    q, k, v, h = make_inputs(lw, stream.device)
    y = torch.empty_like(q)
    code = hc.DTYPE_BF16 if lw.dtype == "bf16" else hc.DTYPE_F32
    ws_n = hc.long_workspace_bytes(lw.B, lw.L, lw.D, lw.group_size, lw.l_h, code)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    for _ in range(2):
        hc.conv_fwd_long(q, k, v, h, lw.group_size, out=y, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    def timed(reuse):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            hc.conv_fwd_long(q, k, v, h, lw.group_size, out=y, workspace=ws, stream=stream, reuse_spectra=reuse)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps
    us = timed(False)
    us_kept = timed(True)
    # the backward (hyena_conv_bwd_long: dq, dk, dv and dh) on the same inputs
    g = torch.Generator(device=q.device).manual_seed(lw.seed + 51)
    dy = torch.randn(q.shape, generator=g, device=q.device).to(q.dtype)
    ws_b = torch.empty(hc.bwd_long_workspace_bytes(lw.B, lw.L, lw.D, lw.group_size, lw.l_h, code),
                       dtype=torch.uint8, device=q.device)
    for _ in range(2):
        hc.conv_bwd_long(q, k, v, h, dy, lw.group_size, workspace=ws_b, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        hc.conv_bwd_long(q, k, v, h, dy, lw.group_size, workspace=ws_b, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us_bwd = e0.elapsed_time(e1) * 1e3 / reps
    # the same with the filter spectra the previous calls left in the workspace
    e0.record(stream)
    for _ in range(reps):
        hc.conv_bwd_long(q, k, v, h, dy, lw.group_size, workspace=ws_b, stream=stream, reuse_spectra=True)
    e1.record(stream)
    torch.cuda.synchronize()
    us_bwd_kept = e0.elapsed_time(e1) * 1e3 / reps
    ws_bwd = ws_b.numel()
    del dy, ws_b
    moved = 40 * lw.elems
    # the filter pass reads h directly up to 512 filters, else transposes it first
    n_filter = 2 if lw.D // lw.group_size <= 512 else 3
    res = {"B": lw.B, "L": lw.L, "D": lw.D, "group_size": lw.group_size, "l_h": lw.l_h,
           "us": round(us, 1), "G_tok_ch_per_s": round(lw.elems / (us * 1e-6) / 1e9, 2),
           "moved_bytes_model": moved, "GBs_moved": round(moved / (us * 1e-6) / 1e9, 1),
           "frac_of_peak_moved": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "workspace_bytes": ws_n, "kernels": 3 + n_filter, "calls_averaged": reps,
           "us_spectra_kept": round(us_kept, 1), "kernels_spectra_kept": 3,
           "G_tok_ch_per_s_spectra_kept": round(lw.elems / (us_kept * 1e-6) / 1e9, 2),
           "backward": {"us": round(us_bwd, 1), "G_tok_ch_per_s": round(lw.elems / (us_bwd * 1e-6) / 1e9, 2),
                        "workspace_bytes": ws_bwd, "kernels": 8 + n_filter,
                        "us_spectra_kept": round(us_bwd_kept, 1), "kernels_spectra_kept": 8,
                        "frac_of_peak_min_bytes": round(14 * lw.elems / (us_bwd * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
    del q, k, v, h, y, ws
    return res


def _stream_ref_lib():
    import ctypes
    from gated_convolution_sequence_amd import _build
    if not os.path.exists(_build.STREAM_REF_LIB):
        _build.build_stream_ref()
    lib = ctypes.CDLL(_build.STREAM_REF_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.hyena_stream_read3_write1.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.hyena_stream_read3_write1.restype = ctypes.c_int
    lib.hyena_stream_configs.restype = ctypes.c_int
    lib.hyena_stream_config.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    return lib


def stream_reference(w, per, stream, reps):
    """What plain streaming kernels reach on the same tensors and rotation.

    ``hip_read3_write1_*``: the hand-written kernel in csrc/stream_ref.hip,
    y = q*k*v (three bf16 reads, one write: the operator's 8 bytes per
    token*channel) with 16-byte non-temporal buffer loads and the grouped
    forward kernels' access patterns (row segments of 256 or 512 bytes per
    workgroup, 8-chunk spans) and the fastest patterns a sweep found (shorter
    spans, wider segments).  Per-launch durations from fence-free HIP events
    around each launch, as for the operator's layers; ``attainable_GBs`` is
    the best of them.  torch's addcmul (same bytes) and a device copy (one
    read, one write) are timed around ``reps`` back-to-back launches.
    """
    import ctypes
    import torch
    res = {}
    lib = _stream_ref_lib()
    eb = 2 if w.dtype == "bf16" else 4
    best = 0.0
    if w.dtype == "bf16":
        cfg = (ctypes.c_int * 6)()
        for ci in range(lib.hyena_stream_configs()):
            lib.hyena_stream_config(ci, cfg)
            waves, seg, span, pf, order = list(cfg)[:5]

            def call(i, ci=ci):
                q, k, v, _, y = per[i % len(per)]
                st = lib.hyena_stream_read3_write1(ci, q.data_ptr(), k.data_ptr(), v.data_ptr(), y.data_ptr(),
                                                   w.B, w.L, w.D, stream.cuda_stream)
                if st != 0:
                    raise RuntimeError("hyena_stream_read3_write1: %d" % st)
            ms = _evented_launches(call, reps, stream)
            mean_ms = sum(ms) / len(ms)
            gbs = w.elems * eb * 4 / (mean_ms * 1e-3) / 1e9
            best = max(best, gbs)
            res["hip_read3_write1_seg%d_w%d_span%d_pf%d%s" % (seg, waves, span, pf, "_spans_fastest" if order else "")] = {
                "mean_us": round(mean_ms * 1e3, 2), "median_us": round(statistics.median(ms) * 1e3, 2),
                "GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "event_samples": len(ms)}
        res["attainable_GBs"] = round(best, 1)
        res["attainable_frac_of_peak"] = round(best / HBM_PEAK_GBS, 4)
    for name, fn, nbytes in (
            ("addcmul_read3_write1", lambda s: torch.addcmul(s[0], s[1], s[2], out=s[4]), 4),
            ("copy_read1_write1", lambda s: s[4].copy_(s[0]), 2)):
        for i in range(3):
            fn(per[i % len(per)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(per[i % len(per)])
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        moved = w.elems * eb * nbytes
        res[name] = {"us": round(us, 2), "GBs": round(moved / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def naive_conv1d(layers, sets, stream, reps):
    """The step as a user would write it with torch ops (MIOpen depthwise conv)."""
    import torch
    import torch.nn.functional as F

    def layer_fn(w, q, k, v, h, permute):
        weight = torch.repeat_interleave(h, w.group_size, dim=0).flip(-1)[:, None, :].contiguous()
        if permute:
            x = (k * v).transpose(1, 2)  # [B, D, L]
            z = F.conv1d(x, weight, padding=w.l_h - 1, groups=w.D)[..., :w.L]
            return q * z.transpose(1, 2)
        return F.conv1d(k, weight, padding=w.l_h - 1, groups=w.D)[..., :w.L]

    res = {}
    try:
        for permute in (True, False):
            for i in range(2):
                for li, w in enumerate(layers):
                    q, k, v, h, _ = sets[li][i % len(sets[li])]
                    kk = k if permute else k.view(w.B, w.D, w.L)
                    layer_fn(w, q, kk, v, h, permute)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(reps):
                for li, w in enumerate(layers):
                    q, k, v, h, _ = sets[li][i % len(sets[li])]
                    kk = k if permute else k.view(w.B, w.D, w.L)
                    layer_fn(w, q, kk, v, h, permute)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / reps
            key = "with_permutes_and_gating" if permute else "conv1d_only"
            res[key] = {"ms_per_step": round(dt * 1e3, 4),
                        "value": round(sum(w.elems for w in layers) / dt / 1e9, 2), "unit": UNIT}
    except Exception as e:  # report, do not hide, a failing baseline
        res["error"] = repr(e)
    return res


def cpu_baseline(layers, sets, budget_s):
    """fp64 oracle over the step's inputs on the host cores (bounded sample)."""
    import torch

    import oracle

    per_layer = []
    t_total, elems_total = 0.0, 0
    sample_desc = []
    for li, w in enumerate(layers):
        q, k, v, h, _ = sets[li][0]
        # bounded sample: whole sequences of the first `ch` channels
        rate_probe_ch = min(w.D, 64)
        cols = lambda a, c: a[:, :, :c].to("cpu", dtype=torch.float64).numpy()
        hq = h[: rate_probe_ch // w.group_size].to("cpu", dtype=torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.conv_fwd_ref(cols(q, rate_probe_ch), cols(k, rate_probe_ch), cols(v, rate_probe_ch),
                            hq, w.group_size)
        probe = time.perf_counter() - t0
        per_elem = probe / (w.B * w.L * rate_probe_ch)
        share = budget_s / len(layers)
        ch = int(min(w.D, max(rate_probe_ch, share / (per_elem * w.B * w.L))))
        ch = max(w.group_size, (ch // w.group_size) * w.group_size)
        hq = h[: ch // w.group_size].to("cpu", dtype=torch.float64).numpy()
        qa, ka, va = cols(q, ch), cols(k, ch), cols(v, ch)
        t0 = time.perf_counter()
        oracle.conv_fwd_ref(qa, ka, va, hq, w.group_size)
        dt = time.perf_counter() - t0
        n = w.B * w.L * ch
        per_layer.append({"layer": w.name, "channels": ch, "seconds": round(dt, 3),
                          "G_tok_ch_per_s": round(n / dt / 1e9, 5)})
        sample_desc.append("%s: all %d rows x first %d of %d channels" % (w.name, w.B * w.L, ch, w.D))
        # the step's time at this rate: every layer's full size
        t_total += dt * (w.elems / n)
        elems_total += w.elems
    threads = oracle.num_threads()
    # one thread: the same channels as above (the same row width, so the
    # same cache behaviour), the first R rows only, R >= 2 l_h (rows before
    # l_h have shorter sums), sized from the rate above for about 3 s per
    # layer; scaled to the full step the same way
    t_step_1, desc_1, secs_1 = 0.0, [], 0.0
    oracle.set_num_threads(1)
    try:
        for li, w in enumerate(layers):
            q, k, v, h, _ = sets[li][0]
            ch = per_layer[li]["channels"]
            per_elem_1 = per_layer[li]["seconds"] * threads / (w.B * w.L * ch)
            R = int(min(w.L, max(2 * w.l_h, 3.0 / max(per_elem_1 * w.B * ch, 1e-12))))
            rows = lambda a: a[:, :R, :ch].to("cpu", dtype=torch.float64).numpy()
            hq = h[: ch // w.group_size].to("cpu", dtype=torch.float64).numpy()
            qa, ka, va = rows(q), rows(k), rows(v)
            t0 = time.perf_counter()
            oracle.conv_fwd_ref(qa, ka, va, hq, w.group_size)
            dt1 = time.perf_counter() - t0
            secs_1 += dt1
            t_step_1 += dt1 * (w.elems / (w.B * R * ch))
            desc_1.append("%s: first %d of %d rows x first %d channels" % (w.name, R, w.L, ch))
    finally:
        oracle.set_num_threads(threads)
    try:
        import psutil
        physical = psutil.cpu_count(logical=False)
    except ImportError:
        physical = None
    return {"value": round(elems_total / t_total / 1e9, 5), "unit": UNIT,
            "cores": threads, "kind": "oracle",
            "sample": "; ".join(sample_desc) + " (rate scaled to the full step)",
            "cpu_count": os.cpu_count(), "physical_cores": physical,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"), "layers": per_layer,
            "single_thread": {"value": round(elems_total / t_step_1 / 1e9, 6), "unit": UNIT,
                              "sample": "; ".join(desc_1) + " (one thread; rate scaled to the full step)",
                              "seconds": round(secs_1, 3)}}


if __name__ == "__main__":
    main()
