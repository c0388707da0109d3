#!/usr/bin/env python3
"""Benchmark: INT4-g32 W4A16 decode GEMV at M = 1 on 39936 x 6656 (one MI355X).

One step = one call of the layer (host checks + the GEMV kernel, plus the
split-K pass when the shape uses one) on one activation row.  Inputs are
resident in HBM before the timed region.  Consecutive calls read different
copies of the packed weight (ceil(1 GiB / bytes) copies), so the 256 MB
Infinity Cache cannot serve a weight from the previous call.  The calls are
captured in a HIP graph of C = max(200, 2 * copies) calls, and the K timed
calls are ceil(K / C) back-to-back replays (the last one shorter when C does
not divide K), bracketed by device synchronizations; an event on the stream
the kernels run on is recorded between replays, so the whole timed region and
each replay are timed on the GPU's clock.  value = K calls / the whole timed
region; the median, min and p90 of the per-replay time per call are reported
beside it.  Before the W warm-up calls, untimed replays run for --settle-s
seconds (0.5 by default): an idle MI355X holds its graphics clock near 160
MHz and takes a few hundred calls to reach full speed, so a short timed
region right after start-up would time the ramp.  The graphics and memory
clocks, power draw and power cap (amdgpu sysfs, as amd-smi reports them),
read during those replays and after the timed region, are recorded in the
line.  A short spin kernel before the start event keeps the first replay's
submission latency out of the timed region.

Beside the layer, the same rotating buffers are read by a plain streaming
kernel (qg_stream_read: 16-byte non-temporal loads, best of a few grid sizes)
and the line reports the layer's rate as a percentage of that measured read
ceiling (pct_of_stream_ceiling); --op stream_read --bytes N measures the
ceiling alone.

Effective weight bytes per call = N*K/2 (codes) + N*K/32 * 2.5 (fp16 scale +
4-bit zero per group of 32), the packed buffer size.  The roofline is HBM
(8 TB/s peak on MI355X).

The CPU baseline leg times the plain C oracle (tests' reference) on this
host's cores over a bounded sample of the same workload and checks the GPU
result against it.

Other layers of the same path use the same protocol: --op w4a16 with
--m 2..64 (M > 4 runs the matrix-core kernel), --op w4a16_dq (the scale-code
weight, bytes = its packed size; --op w4a8_dq / w4a8_g32_dq the W4A8 forms on it),
--op wn_a16 --bits 5|6 (INT5 / INT6,
M = 1, bytes = the packed size), --op w4a8 / w4a8_g32 (M <= 64; at M > 4 the
activations are quantized once into the workspace and the matrix-core kernel
runs on the int8 codes, one weight pass) and
--op w8a16 (int8 per-channel, bytes = N*K + 2*N); --n/--k pick the shape.  The
offline weight quantizers run the same way: --op quantize_int4 / quantize_int4_dq /
quantize_intn --bits 5|6 (bytes = the
bf16 weight read + the packed weight written) and --op quantize_int8 (bf16
read + int8 codes and bf16 scales written), the bf16 inputs and the outputs
both rotating over >= 1 GiB; their CPU leg runs the oracle quantizer and
compares the bytes.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix-core peak of an MI355X
METRIC = "µs/call and effective weight GB/s (% HBM peak) for INT4-g32 GEMV at M=1"
COUNTERS = os.path.join(ROOT, "profiles", "w4a16_gemv_39936x6656_m1_counters.json")
# The timed kernel's source and the host rules that pick it and its launch
# shape (split table, workgroup shape).
KERNEL_SOURCES = ["gemm_decode_qgemm_amd/csrc/gemv_w4a16.hip", "gemm_decode_qgemm_amd/csrc/w4_common.h",
                  "gemm_decode_qgemm_amd/csrc/qg_common.h", "gemm_decode_qgemm_amd/csrc/dispatch.h"]


def kernel_source_hash() -> str:
    """sha256 over the sources that define the timed kernel and its launch."""
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(n, k, m):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this exact kernel source and workload; else None."""
    try:
        with open(COUNTERS) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash() or c.get("workload") != [n, k, m]:
        return None
    return int(c["hbm_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=1000,
                   help="untimed calls first; the clocks take a few hundred calls to ramp up from idle")
    p.add_argument("--op", choices=("w4a16", "w4a16_dq", "wn_a16", "w4a8", "w4a8_g32", "w4a8_dq", "w4a8_g32_dq", "w8a16",
                                    "quantize_int4", "quantize_int4_dq", "quantize_intn", "quantize_int8",
                                    "stream_read"),
                   default="w4a16")
    p.add_argument("--bits", type=int, default=6, help="code width of --op wn_a16 (5 or 6)")
    p.add_argument("--n", type=int, default=39936)
    p.add_argument("--k", type=int, default=6656)
    p.add_argument("--m", type=int, default=1)
    p.add_argument("--split", type=int, default=0, help="split-K (0 = library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain device-to-device copies of the packed-weight size (for scaling "
                        "the FETCH_SIZE / WRITE_SIZE counters to bytes), then exit")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="rough budget of CPU work for the oracle sample")
    p.add_argument("--settle-s", type=float, default=0.5,
                   help="seconds of untimed calls before the warm-up, so the timed calls run at the "
                        "clocks a busy GPU holds (an idle MI355X sits near 160 MHz and needs a few "
                        "hundred calls to ramp up)")
    p.add_argument("--bytes", type=int, default=0,
                   help="--op stream_read: bytes per read (default: the packed 39936x6656 weight)")
    return p.parse_args()


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this layer is benchmarked "
              "on a single MI355X and the multi-GPU sharding is a design note, not a run.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gemm_decode_qgemm_amd as qg
    import synthetic_inputs as si

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    n, k, m = args.n, args.k, args.m
    op = args.op
    if op.startswith("quantize"):
        return bench_quantizer(args, torch, qg, si, dev)
    if op == "stream_read":
        return bench_stream_read(args, torch, qg, dev)
    if op == "w8a16":
        bytes_eff = n * k + 2 * n
    elif op in ("w4a16_dq", "w4a8_dq", "w4a8_g32_dq"):
        bytes_eff = qg.int4_dq_packed_bytes(n, k)
    elif op == "wn_a16":
        bytes_eff = qg.intn_packed_bytes(n, k, args.bits)
    else:
        bytes_eff = qg.int4_packed_bytes(n, k)
    if args.calibrate_copy:
        return calibrate_copy(torch, dev, bytes_eff)
    copies = max(2, math.ceil((1 << 30) / bytes_eff))
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    split = None
    if op == "w8a16":
        w_cpu, s_cpu, x_cpu = si.int8_layer(n, k, m)
        wq0, sc = w_cpu.to(dev), s_cpu.to(dev)
        wqs = [wq0] + [wq0.clone() for _ in range(copies - 1)]
        x = x_cpu.to(dev)

        def call(i):
            qg.qgemm_w8a16(x, wqs[i % copies], sc, out=y)

        oracle_inputs = (w_cpu, s_cpu, x_cpu)
    else:
        if (n, k) in si.MODEL_SHAPES:
            w_cpu, x_cpu = si.decode_inputs(n, k, m)
        else:
            w_cpu, x_cpu = si.int4_weight(n, k, n ^ k), si.activation(m, k, 9100 + m)
        split = args.split or qg.default_split_k(m, n, k, args.bits if op == "wn_a16" else 4,
                                                 group_scales=op in ("w4a8_g32", "w4a8_g32_dq"))
        if op in ("w4a16_dq", "w4a8_dq", "w4a8_g32_dq"):
            packed0 = qg.quantize_int4_g32_dq(w_cpu.to(dev))
        elif op == "wn_a16":
            packed0 = qg.quantize_intn_g32(w_cpu.to(dev), args.bits)
        else:
            packed0 = qg.quantize_int4_g32(w_cpu.to(dev))
        packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
        x = x_cpu.to(dev)
        ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
        fn = {"w4a16": qg.qgemm_w4a16, "w4a16_dq": qg.qgemm_w4a16_dq, "w4a8": qg.qgemm_w4a8,
              "w4a8_g32": qg.qgemm_w4a8_g32, "w4a8_dq": qg.qgemm_w4a8_dq, "w4a8_g32_dq": qg.qgemm_w4a8_g32_dq,
              "wn_a16": lambda *a, **kw: qg.qgemm_wn_a16(*a[:3], args.bits, **kw)}[op]

        def call(i):
            fn(x, packs[i % copies], n, split_k=split, out=y, workspace=ws)

        oracle_inputs = (w_cpu, None, x_cpu)
    torch.cuda.synchronize()

    # Eager warm-up (also loads the code object), then capture graphs.
    for i in range(min(args.warmup, 20)):
        call(i)
    torch.cuda.synchronize()
    chunk = min(args.steps, max(200, 2 * copies))
    full, rest = divmod(args.steps, chunk)
    stream = torch.cuda.Stream()
    g_warm, g_chunk, g_rest = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), None
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g_warm, stream=stream):
            for i in range(max(args.warmup, 1)):
                call(i)
        with torch.cuda.graph(g_chunk, stream=stream):
            for i in range(chunk):
                call(i)
        if rest:
            g_rest = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rest, stream=stream):
                for i in range(rest):
                    call(i)
    torch.cuda.synchronize()

    replays = [g_chunk] * full + ([g_rest] if rest else [])
    events = [torch.cuda.Event(enable_timing=True) for _ in range(len(replays) + 1)]
    with torch.cuda.stream(stream):
        settle = settle_clocks(torch, g_chunk, chunk, args.settle_s)
        g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        # A short spin kernel holds the stream while the host submits the
        # start event and the graphs, so the timed region holds the K calls
        # back to back and not the submission latency of the first replay.
        torch.cuda._sleep(200_000)
        events[0].record(stream)
        for g, ev in zip(replays, events[1:]):
            g.replay()
            ev.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    state_after = gpu_state()
    ms_total = events[0].elapsed_time(events[-1])
    us_call = ms_total * 1e3 / args.steps
    per_replay = sorted(events[i].elapsed_time(events[i + 1]) * 1e3 / chunk for i in range(full))
    gbs = bytes_eff / (us_call * 1e-6) / 1e9
    y_first = y.clone()

    headline = op == "w4a16" and (n, k, m) == (39936, 6656, 1)
    kernel = "matrix-core GEMM" if (op == "w4a16" and m > 4) else "GEMV"
    label = {"w4a16": "W4A16 INT4-g32 asymmetric",
             "w4a16_dq": "W4A16 INT4-g32 asymmetric, uint8 scale codes x per-row fp16 step",
             "wn_a16": f"W{args.bits}A16 INT{args.bits}-g32 asymmetric",
             "w4a8": "W4A8 INT4-g32 x per-row int8",
             "w4a8_dq": "W4A8 INT4-g32 (scale codes) x per-row int8",
             "w4a8_g32_dq": "W4A8 INT4-g32 (scale codes) x per-group-32 int8",
             "w4a8_g32": "W4A8 INT4-g32 x per-group-32 int8", "w8a16": "W8A16 INT8 per-channel"}[op]
    out = {
        "metric": METRIC if headline else
        f"µs/call and effective weight GB/s (% HBM peak) for {label} {kernel} at M={m}",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us_call / 1e3,
        "us_per_call": round(us_call, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{label} {kernel} {n}x{k} M={m}",
            "op": op, "n": n, "k": k, "m": m, "split_k": split, "bytes_eff_per_call": bytes_eff,
            **({"bits": args.bits} if op == "wn_a16" else {}),
            "codes_only_gbs": round((n * k * {"w8a16": 8, "wn_a16": args.bits}.get(op, 4) / 8)
                                    / (us_call * 1e-6) / 1e9, 2),
            "rotating_weight_copies": copies,
            "timing": f"{full} replays of a {chunk}-call HIP graph" + (f" + one of {rest}" if rest else "")
                      + ", events on its stream",
            "us_per_call_replay": {"median": round(float(np.median(per_replay)), 3) if per_replay else None,
                                   "min": round(per_replay[0], 3) if per_replay else None,
                                   "p90": round(float(np.percentile(per_replay, 90)), 3) if per_replay else None},
            "hip_runtime": torch.version.hip,
            "wall_s": round(wall, 4),
            "clock_settle": {k2: v for k2, v in settle.items() if k2 != "state"},
            "gpu_state": {"during_settle": settle.get("state"), "after_timing": state_after,
                          "note": "amdgpu sysfs readings; they trail the load by a few hundred ms"},
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(n, k, m) if headline else None,
        },
    }
    # The measured read ceiling of the same rotating buffers (a plain 16-byte
    # non-temporal streaming read of bytes_eff each), same clocks and protocol.
    bufs = wqs if op == "w8a16" else packs
    read_bytes = min(bytes_eff, bufs[0].numel() * bufs[0].element_size()) // 16 * 16
    ceiling = stream_ceiling(torch, qg, bufs, read_bytes)
    out["config"]["stream_ceiling"] = ceiling
    out["pct_of_stream_ceiling"] = round(100.0 * gbs / ceiling["gbs"], 2)
    if m > 4:
        tflops = 2.0 * m * n * k / (us_call * 1e-6) / 1e12
        out["roofline"]["matrix_core"] = {"achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, oracle_inputs, y_first, bytes_eff)

    print(json.dumps(out), flush=True)
    return 0


def graph_time(torch, call, steps, warmup, settle_s=0.5):
    """The timing protocol of main(): warm-up graph, then `steps` calls in
    replays of one captured chunk, events on the capture stream.  Returns
    (us per call, per-replay us per call sorted, chunk, full, rest, wall s)."""
    import numpy as np  # noqa: F401

    for i in range(min(warmup, 20)):
        call(i)
    torch.cuda.synchronize()
    chunk = min(steps, 200)
    full, rest = divmod(steps, chunk)
    stream = torch.cuda.Stream()
    g_warm, g_chunk, g_rest = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), None
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g_warm, stream=stream):
            for i in range(max(warmup, 1)):
                call(i)
        with torch.cuda.graph(g_chunk, stream=stream):
            for i in range(chunk):
                call(i)
        if rest:
            g_rest = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_rest, stream=stream):
                for i in range(rest):
                    call(i)
    torch.cuda.synchronize()
    replays = [g_chunk] * full + ([g_rest] if rest else [])
    events = [torch.cuda.Event(enable_timing=True) for _ in range(len(replays) + 1)]
    with torch.cuda.stream(stream):
        settle_clocks(torch, g_chunk, chunk, settle_s)
        g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        torch.cuda._sleep(200_000)
        events[0].record(stream)
        for g, ev in zip(replays, events[1:]):
            g.replay()
            ev.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    us_call = events[0].elapsed_time(events[-1]) * 1e3 / steps
    per_replay = sorted(events[i].elapsed_time(events[i + 1]) * 1e3 / chunk for i in range(full))
    return us_call, per_replay, chunk, full, rest, wall


def gpu_state():
    """Graphics and memory clock, power draw and power cap of the GPU, read
    from the amdgpu driver's sysfs files (the source amd-smi reads; no
    program is started from this GPU process).  The driver refreshes these
    figures every few hundred milliseconds, so a reading trails the load by
    about that much.  None where a file is missing."""
    import glob

    def first(pattern):
        for f in sorted(glob.glob(pattern)):
            try:
                with open(f) as fh:
                    return fh.read()
            except OSError:
                continue
        return None

    def current_mhz(text):
        for line in (text or "").splitlines():
            if line.rstrip().endswith("*"):
                digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                return int(digits) if digits else None
        return None

    def watts(text):
        try:
            return int(text.strip()) / 1e6
        except (AttributeError, ValueError):
            return None

    return {"sclk_mhz": current_mhz(first("/sys/class/drm/card*/device/pp_dpm_sclk")),
            "mclk_mhz": current_mhz(first("/sys/class/drm/card*/device/pp_dpm_mclk")),
            "power_w": watts(first("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")
                             or first("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average")),
            "power_cap_w": watts(first("/sys/class/drm/card*/device/hwmon/hwmon*/power1_cap"))}


def settle_clocks(torch, graph, calls_per_replay, seconds):
    """Replay `graph` (untimed) for at least `seconds`, reading the GPU's
    clocks once while it is busy.  Returns the calls run and that reading."""
    t0 = time.perf_counter()
    replays = 0
    state = None
    while time.perf_counter() - t0 < seconds or replays == 0:
        for _ in range(8):
            graph.replay()
        replays += 8
        if state is None and time.perf_counter() - t0 >= 0.8 * seconds:
            state = gpu_state()            # read while the replays just queued run
        torch.cuda.synchronize()
    return {"calls": replays * calls_per_replay, "s": round(time.perf_counter() - t0, 3),
            "state": state}


STREAM_BLOCKS = (512, 1024, 2048, 4096)


def stream_ceiling(torch, qg, bufs, nbytes, calls=400, replays=3):
    """GB/s of qg_stream_read over the rotating buffers `bufs` (nbytes each),
    best over a few grid sizes, each timed as `replays` replays of a
    `calls`-call graph (clocks already up)."""
    import numpy as np

    dev = bufs[0].device
    sink = torch.empty(max(STREAM_BLOCKS) * 4, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    best = None
    for blocks in STREAM_BLOCKS:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            qg.stream_read(bufs[0], nbytes, sink, blocks)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(calls):
                    qg.stream_read(bufs[i % len(bufs)], nbytes, sink, blocks)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
            ev[0].record(stream)
            for r in range(replays):
                g.replay()
                ev[r + 1].record(stream)
            torch.cuda.synchronize()
        us = float(np.median([ev[r].elapsed_time(ev[r + 1]) * 1e3 / calls for r in range(replays)]))
        gbs = nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 2), "us_per_read": round(us, 3), "blocks": blocks, "bytes": nbytes}
    best["kernel"] = "qg_stream_read: 256 lanes x 2 x 16-byte non-temporal loads per step, grid-strided"
    best["timing"] = f"median of {replays} replays of a {calls}-call graph per grid size {list(STREAM_BLOCKS)}"
    return best


def bench_stream_read(args, torch, qg, dev):
    """The plain streaming-read rate of `--bytes` over rotating copies
    (>= 1 GiB): the ceiling the GEMVs' effective bandwidth is compared with."""
    nbytes = args.bytes or qg.int4_packed_bytes(39936, 6656)
    nbytes -= nbytes % 16
    copies = max(2, math.ceil((1 << 30) / nbytes))
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(copies)]
    torch.cuda.synchronize()
    sink = torch.empty(max(STREAM_BLOCKS) * 4, dtype=torch.int32, device=dev)

    def call(i):
        qg.stream_read(bufs[i % copies], nbytes, sink, 1024)

    # bring the clocks up with untimed reads, then sweep the grid sizes
    settle_t0 = time.perf_counter()
    while time.perf_counter() - settle_t0 < args.settle_s:
        for i in range(50):
            call(i)
        torch.cuda.synchronize()
    best = stream_ceiling(torch, qg, bufs, nbytes, calls=max(args.steps, 2 * copies), replays=3)
    out = {
        "metric": f"streaming-read GB/s (% HBM peak) of {nbytes} bytes per read",
        "value": best["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": best["us_per_read"] / 1e3, "us_per_call": best["us_per_read"],
        "pct_hbm_peak": round(100.0 * best["gbs"] / HBM_PEAK_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"stream read {nbytes} B", "op": "stream_read", "bytes": nbytes,
                   "rotating_copies": copies, **best, "gpu_state": gpu_state()},
        "roofline": {"bound": "hbm", "achieved": best["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(best["gbs"] / HBM_PEAK_GBS, 4), "traffic": None},
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_quantizer(args, torch, qg, si, dev):
    """The offline weight quantizers (INT4 g32 pack, INT8 row-wise) on one
    GPU: HBM-bound streams, bytes = bf16 read + quantized weight written."""
    import numpy as np

    n, k = args.n, args.k
    op = args.op
    int4 = op != "quantize_int8"                  # every packed INT4/5/6 layout
    w_cpu = si.int4_weight(n, k, n ^ k)           # a bf16 weight of the layers' distribution
    if op == "quantize_int4":
        out_bytes, quant = qg.int4_packed_bytes(n, k), qg.quantize_int4_g32
    elif op == "quantize_int4_dq":
        out_bytes, quant = qg.int4_dq_packed_bytes(n, k), qg.quantize_int4_g32_dq
    elif op == "quantize_intn":
        out_bytes = qg.intn_packed_bytes(n, k, args.bits)
        quant = lambda w, out: qg.quantize_intn_g32(w, args.bits, out=out)
    else:
        out_bytes = n * k + 2 * n
    bytes_eff = 2 * n * k + out_bytes
    copies = max(2, math.ceil((1 << 30) / bytes_eff))
    w0 = w_cpu.to(dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    if int4:
        outs = [torch.empty(out_bytes, dtype=torch.uint8, device=dev) for _ in range(copies)]

        def call(i):
            quant(ws[i % copies], out=outs[i % copies])
    else:
        outs = [(torch.empty((n, k), dtype=torch.int8, device=dev), torch.empty(n, dtype=torch.bfloat16, device=dev))
                for _ in range(copies)]

        def call(i):
            qg.quantize_int8_rowwise(ws[i % copies], out=outs[i % copies])
    torch.cuda.synchronize()
    us_call, per_replay, chunk, full, rest, wall = graph_time(torch, call, args.steps, args.warmup, args.settle_s)
    gbs = bytes_eff / (us_call * 1e-6) / 1e9
    name = {"quantize_int4": "INT4-g32 quantize + pack", "quantize_int4_dq": "INT4-g32 quantize + pack with scale codes",
            "quantize_intn": f"INT{args.bits}-g32 quantize + pack", "quantize_int8": "INT8 row-wise quantize"}[op]
    out = {
        "metric": f"µs/call and streamed GB/s (% HBM peak) for the {name} of a bf16 weight",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": us_call / 1e3, "us_per_call": round(us_call, 3),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name} {n}x{k}", "op": args.op, "n": n, "k": k,
                   "bytes_eff_per_call": bytes_eff, "rotating_copies": copies,
                   "timing": f"{full} replays of a {chunk}-call HIP graph" + (f" + one of {rest}" if rest else "")
                             + ", events on its stream",
                   "us_per_call_replay": {"median": round(float(np.median(per_replay)), 3) if per_replay else None,
                                          "min": round(per_replay[0], 3) if per_replay else None},
                   "hip_runtime": torch.version.hip, "wall_s": round(wall, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle

        bits = si.bf16_bits(w_cpu)
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            if op == "quantize_int4":
                c, s, z, _ = oracle.quantize_int4_g32(bits)
                ref = oracle.pack_int4(c, s, z)
            elif op == "quantize_int4_dq":
                c, sc, st, z, _ = oracle.quantize_int4_g32_dq(bits)
                ref = oracle.pack_int4_dq(c, sc, st, z)
            elif op == "quantize_intn":
                c, s, z, _ = oracle.quantize_intn_g32(bits, args.bits)
                ref = oracle.pack_intn(c, s, z, args.bits)
            else:
                ref = oracle.quantize_int8_rowwise(bits)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > args.cpu_seconds:
                break
        t = float(np.median(times))
        if int4:
            same = bool(np.array_equal(outs[0].cpu().numpy(), ref))
        else:
            q_ref, s_ref = ref[0], ref[1]
            same = bool(np.array_equal(outs[0][0].cpu().numpy(), q_ref)
                        and np.array_equal(si.bf16_bits(outs[0][1].cpu()), s_ref))
        out["cpu_baseline"] = {
            "value": round(bytes_eff / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_call": round(t * 1e6, 1),
            "sample": f"{len(times)} full calls ({n}x{k}) in {time.perf_counter() - t_start:.1f} s, median per call",
            "gpu_vs_oracle": {"bit_exact": same},
        }
    print(json.dumps(out), flush=True)
    return 0


def calibrate_copy(torch, dev, nbytes):
    """Plain copies of nbytes each (rotating sources, as the timed GEMV reads
    its weight): under a counter profiler, FETCH_SIZE and WRITE_SIZE of these
    copies give the counters' scale to bytes."""
    copies = max(2, math.ceil((1 << 30) / nbytes))
    src = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(copies)]
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for i in range(3 * copies):
        dst.copy_(src[i % copies])
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_per_copy": nbytes, "copies": 3 * copies}), flush=True)
    return 0


def cpu_baseline(args, oracle_inputs, y_gpu, bytes_eff):
    """Time the C oracle of the same op on the host's cores on a bounded sample
    of the same workload (whole weight, M rows), and check the GPU output
    against it."""
    import numpy as np

    import oracle
    import synthetic_inputs as si

    threads = oracle.hardware_threads()
    w_cpu, s_cpu, x_cpu = oracle_inputs
    xb = si.bf16_bits(x_cpu)
    if args.op == "w8a16":
        wi8 = w_cpu.numpy()
        sb = si.bf16_bits(s_cpu)

        def run():
            return oracle.qgemm_w8a16(xb, wi8, sb, threads=threads)
    elif args.op == "wn_a16":
        codes, scales, zeros, _ = oracle.quantize_intn_g32(si.bf16_bits(w_cpu), args.bits)

        def run():
            return oracle.qgemm_w4a16(xb, codes, scales, zeros, threads=threads)
    elif args.op in ("w4a16_dq", "w4a8_dq", "w4a8_g32_dq"):
        codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w_cpu))
        dq_fn = {"w4a16_dq": oracle.qgemm_w4a16_dq, "w4a8_dq": oracle.qgemm_w4a8_dq,
                 "w4a8_g32_dq": oracle.qgemm_w4a8_g32_dq}[args.op]

        def run():
            return dq_fn(xb, codes, scode, sstep, zeros, threads=threads)
    else:
        codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w_cpu))
        fn = {"w4a16": oracle.qgemm_w4a16, "w4a8": oracle.qgemm_w4a8,
              "w4a8_g32": oracle.qgemm_w4a8_g32}[args.op]

        def run():
            return fn(xb, codes, scales, zeros, threads=threads)
    times = []
    ref = None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ref = run()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > args.cpu_seconds:
            break
    t = float(np.median(times))
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(y - ref)
    mean_ref = float(np.abs(ref).mean())
    # The timed output is bf16: allow half a bf16 ulp of ref on top of the
    # fp32-output bound (the same reading the parity tests use).
    _, e = np.frexp(np.maximum(np.abs(ref), np.finfo(np.float32).tiny))
    within = bool((err <= 1e-2 * mean_ref + 1e-3 + np.ldexp(1.0, e - 9)).all()
                  and err.mean() / mean_ref <= 2e-3)
    return {
        "value": round(bytes_eff / t / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "us_per_call": round(t * 1e6, 1),
        "sample": f"{len(times)} full calls ({args.n}x{args.k}, M={args.m}) in "
                  f"{time.perf_counter() - t_start:.1f} s, median per call",
        "gpu_vs_oracle": {"max_abs_err": float(err.max()),
                          "mean_rel_err": float(err.mean() / mean_ref),
                          "within_tolerance": within},
    }


if __name__ == "__main__":
    sys.exit(main())
