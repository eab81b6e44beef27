"""Benchmark: achieved HBM bandwidth of the packed causal conv on one MI355X.

A step is one call of the whole path (program map, history, taps, SiLU, bf16
planes, state update) on the headline workload: one sequence of 16384 tokens,
dim 4608 = 3 x 1536 packed Q|K|V channels read in place from rows of 9728 bf16
elements, bf16 output planes, FP32 weight and bias, SiLU, FP32 conv state with an
initial state. Inputs are synthetic (seeded, workloads.config3) and resident in
HBM before timing starts. Several complete buffer sets (x, out, state) rotate so
that no step finds its inputs in the 256 MB Infinity Cache from the previous step.

value = algorithmic bytes per step / mean time per step, from HIP events on the
launch stream around the K timed back-to-back steps (synchronised on both sides; a
0.2 ms spin kernel queued ahead of the start event keeps the host's submission of the
first step out of the timed region, see queue_ahead()).
Before the W warm-up steps the same step runs back to back for --settle-ms (100 ms)
of GPU time, because the GPU's power management needs tens of milliseconds of this
load to settle (the settle() docstring has the figures); the K steps timed right
after start-up, before settling, are reported beside it.
Each step is one kernel launch, so roofline.achieved is the same figure: bytes /
mean launch duration. roofline.spread_blocks_of_k gives the median and p10/p90
of the per-launch mean over further blocks of K back-to-back launches timed the
same way. Algorithmic bytes: x read once and out written once (2 B per element
each), the state line read and written (12 B per channel each), weight (16 B per
channel), bias (4 B per channel), metadata (workloads.Workload.algorithmic_bytes).
roofline.traffic: HBM bytes per launch from the committed rocprofv3 counter
summary, when it was taken from the kernel source as it is (else null).

cpu_baseline: the CPU oracle as it stands, single-threaded, on the headline
workload (value); once on each named workload; and on the headline workload
split into channel slices over all the host's cores.

Beside the headline (parity cases and context, not the metric): back-to-back
per-launch times of the four other named workloads, decode batches, fp16 and
FP32 x, and one sequence of 2K, 4K and 8K tokens.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import pathlib
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
METRIC = "achieved HBM GB/s (read+write) and % of peak, 16K tokens × 3×1536 packed conv"
KERNEL_SOURCES = [
    ROOT / "packed_varlen_causal_depthwise_amd" / "csrc" / "kdaconv.hip",
    ROOT / "packed_varlen_causal_depthwise_amd" / "csrc" / "kdaconv_device.h",
]
COUNTERS = ROOT / "profiles" / "packed_conv_kernel_16k_tokens_counters.md"


def kernel_source_hash() -> str:
    """Hash of the kernel sources with // comments and blank lines removed, so that a
    counter summary stays valid across comment-only edits."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        for line in p.read_text().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    summary is absent or was taken from a different kernel source."""
    if not COUNTERS.exists():
        return None
    fields = {}
    for line in COUNTERS.read_text().splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source hash") != kernel_source_hash():
        return None
    try:
        return int(fields["hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def x_tensor(torch, wl, dev):
    """The workload's whole row-strided x buffer on the device, in its format."""
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[wl.x_dtype]
    signed = np.int32 if wl.x.dtype == np.uint32 else np.int16
    return torch.from_numpy(np.ascontiguousarray(wl.x).view(signed)).to(dev).view(dt)


#: Bytes of complete buffer sets rotated across launches: past the 256 MB Infinity Cache,
#: so no launch finds its inputs there from the launch before.
ROTATION_BYTES = 600 << 20


def rotation_sets(set_bytes: int, at_most: int = 64) -> int:
    """Buffer sets to rotate: enough to exceed ROTATION_BYTES, at least 2."""
    return int(min(at_most, max(2, -(-ROTATION_BYTES // max(1, set_bytes)))))


def queue_ahead(torch):
    """Keeps the GPU busy for about 0.2 ms (a spin kernel of 400000 clock cycles) after a
    synchronisation, so that the event starting a timed region and the first launches
    after it queue up behind it. Without it the start event is stamped on an idle GPU and
    the host's time to submit the first launch (the binding's argument checks and the
    launch call) falls inside the timed region: 20 timed steps measured about 0.9 us per
    step slower than the same steps in later blocks."""
    torch.cuda._sleep(400_000)


def graph_replays(torch, step, steps: int, blocks: int):
    """Per-launch times of `blocks` replays of one HIP graph holding `steps` launches (the
    steps captured once on a side stream), timed back to back between events on the
    replay stream. Serving loops launch short kernels this way; the host's time per call
    then falls outside the GPU's critical path."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)  # first use on the capture stream, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    g.replay()  # warm
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    queue_ahead(torch)
    evs[0].record(stream)
    for b in range(blocks):
        g.replay()
        evs[b + 1].record(stream)
    torch.cuda.synchronize()
    del g
    return np.array([evs[b].elapsed_time(evs[b + 1]) * 1e3 / steps for b in range(blocks)])


def back_to_back(torch, stream, step, steps: int, blocks: int):
    """Per-launch times of `blocks` blocks of `steps` back-to-back launches, with an event
    only at each block boundary (events between single launches put an idle gap in front of
    every launch). Returns the per-launch mean of each block in microseconds."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    torch.cuda.synchronize()
    queue_ahead(torch)
    i = 0
    evs[0].record(stream)
    for b in range(blocks):
        for _ in range(steps):
            step(i)
            i += 1
        evs[b + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([evs[b].elapsed_time(evs[b + 1]) * 1e3 / steps for b in range(blocks)])


def settle(torch, step, ms: float, first: int = 0) -> int:
    """Runs back-to-back steps for at least `ms` milliseconds of GPU time and returns how
    many. After an idle period the GPU's power management takes tens of milliseconds
    of this load to settle: the per-launch time of the headline workload measured
    about 56 us for the first launches, 62 us a few milliseconds later, and a steady
    54 us from about 25 ms on, on one box, while a copy-like kernel of the same bytes
    stays flat. The timed region is meant to measure the settled rate."""
    if ms <= 0:
        return 0
    done = 0
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record()
    elapsed = 0.0
    while elapsed < ms:
        for _ in range(50):
            step(first + done)
            done += 1
        z.record()
        torch.cuda.synchronize()
        elapsed = a.elapsed_time(z)
    return done


def summary(nbytes: int, us: np.ndarray) -> dict:
    med = float(np.median(us))
    return {
        "algorithmic_bytes": nbytes,
        "kernel_us_median": round(med, 3),
        "kernel_us_p10_p90": [round(float(np.percentile(us, 10)), 3),
                              round(float(np.percentile(us, 90)), 3)],
        "GB/s": round(nbytes / med / 1e3, 1),
        "pct_of_peak": round(100.0 * nbytes / med / 1e3 / PEAK_HBM_GBS, 2),
    }


def fmt_label(x_dtype: str) -> str:
    return {"bf16": "bf16", "f16": "fp16", "f32": "FP32"}[x_dtype]


def time_config(kd, torch, wl, steps: int, warmup: int, blocks: int = 10, decode: bool = False,
                settle_ms: float = 30.0, x_column: int = 0, graph: bool = False):
    """Back-to-back per-launch times of the conv (or, with decode, of the decode step) on
    one workload, with complete input/output/state sets rotated past the Infinity Cache.
    A ``workloads.Bf16StateDecode`` is timed as the decode step with its bf16 state and
    width-major weight. With x_column > 0, x is read from a buffer whose columns start that
    many elements in (every lane's 8-byte vector of x unaligned). With graph, the
    same steps are also captured in a HIP graph and replayed (``graph``): for launches
    shorter than the binding's host time per call, the eager figure is the host's rate
    and the replayed one the GPU's."""
    dev = torch.device("cuda:0")
    bf16_state = not hasattr(wl, "query_start_loc")
    tokens = wl.batch if bf16_state else wl.num_tokens
    x_dtype = "bf16" if bf16_state else wl.x_dtype
    P = wl.dim // wl.part_dim
    if bf16_state:
        xb = torch.from_numpy(wl.x.view(np.int16)).to(dev).view(torch.bfloat16)
    elif x_column:
        raw = np.zeros((wl.x.shape[0], wl.x.shape[1] + x_column), dtype=wl.x.dtype)
        raw[:, x_column:] = wl.x
        signed = np.int32 if raw.dtype == np.uint32 else np.int16
        dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[wl.x_dtype]
        xb = torch.from_numpy(raw.view(signed)).to(dev).view(dt)[:, x_column:]
    else:
        xb = x_tensor(torch, wl, dev)
    eb = xb.element_size()
    set_bytes = wl.x.nbytes + P * tokens * wl.part_dim * eb + wl.conv_states.nbytes
    sets = rotation_sets(set_bytes)
    bufs = []
    for i in range(sets):
        if x_column:  # a copy of the whole buffer, so that every set keeps the offset
            x = xb if not i else xb.as_strided(
                (xb.shape[0], xb.shape[1] + x_column), (xb.stride(0), 1),
                xb.storage_offset() - x_column).clone()[:, x_column:]
        else:
            x = xb.clone() if i else xb
        st = torch.from_numpy(wl.conv_states.copy().view(np.int16) if bf16_state
                              else wl.conv_states.copy()).to(dev)
        bufs.append(dict(
            x=x[:, : wl.dim],
            st=st.view(torch.bfloat16) if bf16_state else st,
            out=torch.empty((P, tokens, wl.part_dim), dtype=xb.dtype, device=dev),
        ))
    w = torch.from_numpy(wl.weight).to(dev)
    b = None if wl.bias is None else torch.from_numpy(wl.bias).to(dev)
    ci = torch.from_numpy(wl.cache_indices).to(dev)
    if not bf16_state:
        q = torch.from_numpy(wl.query_start_loc).to(dev)
        init = torch.from_numpy(wl.has_initial_state).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = bufs[i % sets]
        if decode or bf16_state:
            kd.packed_causal_conv1d_update(s["x"], w, b, s["st"], ci, wl.part_dim, wl.activation,
                                           wl.null_block_id, out=s["out"])
        else:
            kd.packed_causal_conv1d_fn(s["x"], w, b, s["st"], q, ci, init, wl.part_dim,
                                       wl.activation, wl.null_block_id, out=s["out"])

    n = settle(torch, step, settle_ms)
    for i in range(warmup):
        step(n + i)
    us = back_to_back(torch, stream, step, steps, blocks)
    graph_us = graph_replays(torch, step, steps, blocks) if graph else None
    res = {"workload": wl.name + f", x and out {fmt_label(x_dtype)}"
                       + (f", x from column {x_column} of its buffer" if x_column else ""),
           "buffer_sets_rotated": sets}
    res.update(summary(wl.algorithmic_bytes(), us))
    if graph_us is not None:
        res["graph"] = summary(wl.algorithmic_bytes(), graph_us)
    del bufs
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info(torch, dev) -> dict:
    props = torch.cuda.get_device_properties(dev)
    return {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count,
            "memory_gib": round(props.total_memory / 2**30, 1)}


def clocks_under_load(torch, dev, step, seconds: float = 3.0, first: int = 0) -> dict:
    """The GPU's clocks while the headline workload runs back to back for `seconds`.

    The readings come from amdsmi's GPU metrics (the interface torch.cuda.clock_rate uses
    on ROCm), which the power management refreshes about once a second, so a short
    window would only see the readings from before it. A background thread polls every
    20 ms; only readings refreshed at least 1.1 s into the busy window are kept, one per
    refresh. Reported: the core clock of the socket and of each XCD, the memory clock,
    the socket power and the activity. Best effort: if amdsmi is missing or refuses, the
    error is reported instead."""
    import threading

    try:
        import amdsmi

        handle = torch.cuda._get_amdsmi_handler(dev)
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception as e:  # noqa: BLE001 - reported, not raised
        return {"error": f"{type(e).__name__}: {e}"}
    seen = {}
    stop = threading.Event()
    errors = []
    t0 = time.perf_counter()

    def poll():
        while not stop.wait(0.02):
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            except Exception as e:  # noqa: BLE001
                errors.append(f"{type(e).__name__}: {e}")
                return
            ts = m.get("firmware_timestamp")
            if ts not in seen:
                seen[ts] = (time.perf_counter() - t0, m)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    torch.cuda.synchronize()
    t_busy = time.perf_counter() - t0
    done = 0
    while time.perf_counter() - t0 < t_busy + seconds:
        for _ in range(50):
            step(first + done)
            done += 1
        torch.cuda.synchronize()
    t_end = time.perf_counter() - t0
    stop.set()
    th.join()
    keep = [m for t, m in seen.values() if t_busy + 1.1 <= t <= t_end]

    def num(v):
        return v if isinstance(v, (int, float)) else None

    out = {"source": "amdsmi GPU metrics (refreshed about once a second), during "
                     f"{seconds:.0f} s of back-to-back headline steps after the timed blocks",
           "launches": done, "readings": len(keep)}
    if keep:
        out["gfx_mhz"] = [num(m.get("current_gfxclk")) for m in keep]
        out["gfx_mhz_per_xcd"] = [list(m.get("current_gfxclks") or [])[:8] for m in keep]
        out["memory_clock_mhz"] = [num(m.get("current_uclk")) for m in keep]
        out["socket_power_w"] = [num(m.get("current_socket_power")) for m in keep]
        out["gfx_activity_pct"] = [num(m.get("average_gfx_activity")) for m in keep]
    if errors:
        out["error"] = errors[0]
    return out


def oracle_on_channel_slices(oracle, wl, threads: int):
    """The oracle on `threads` channel slices of the workload at once (Python threads;
    ctypes releases the interpreter lock during the C call). A channel's outputs and
    state depend on that channel only (a pinned invariant), so the slices together are
    the whole result; the oracle itself is unchanged and single-threaded."""
    from concurrent.futures import ThreadPoolExecutor

    import workloads

    dim = wl.dim
    edges = np.linspace(0, dim, threads + 1).astype(int)

    def run(k):
        c0, c1 = int(edges[k]), int(edges[k + 1])
        if c1 <= c0:
            return
        sub = workloads.Workload(wl.name, wl.x[:, c0:c1], c1 - c0,
                                 np.ascontiguousarray(wl.weight[c0:c1]),
                                 None if wl.bias is None else np.ascontiguousarray(wl.bias[c0:c1]),
                                 np.ascontiguousarray(wl.conv_states[:, c0:c1]),
                                 wl.query_start_loc, wl.cache_indices, wl.has_initial_state,
                                 c1 - c0, wl.activation, wl.null_block_id, wl.x_dtype)
        oracle.run_workload(sub)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(threads)))


def cpu_baseline(wl, runs: int, configs: dict):
    """The CPU oracle timed on this host: single-threaded on the headline workload
    (`value`), on each named workload once, and on the headline workload over all the
    host's cores by channel slices."""
    import oracle

    oracle.load()
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle.run_workload(wl)
        times.append(time.perf_counter() - t)
    med = float(np.median(times))
    per_config = {}
    for k, w in configs.items():
        if w is wl:
            dt = med  # the runs above
        else:
            t = time.perf_counter()
            oracle.run_workload(w)
            dt = time.perf_counter() - t
        per_config[str(k)] = {"seconds": round(dt, 4),
                              "GB/s": round(w.algorithmic_bytes() / dt / 1e9, 4), "cores": 1}
    cores = len(os.sched_getaffinity(0))
    par = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle_on_channel_slices(oracle, wl, cores)
        par.append(time.perf_counter() - t)
    pmed = float(np.median(par))
    return {
        "value": round(wl.algorithmic_bytes() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "host_cpus": cores,
        "kind": "oracle",
        "sample": f"the whole headline workload ({wl.num_tokens} tokens x {wl.dim} channels), "
                  f"{runs} runs, median {med:.2f} s per run, single thread",
        "per_config_single_thread": per_config,
        "all_cores": {"value": round(wl.algorithmic_bytes() / pmed / 1e9, 4), "unit": "GB/s",
                      "cores": cores, "seconds_median": round(pmed, 3),
                      "sample": f"the headline workload as {cores} channel slices on {cores} "
                                f"threads, {runs} runs"},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="buffer sets rotated across steps")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="milliseconds of back-to-back steps before the warm-up steps, so that "
                         "the timed region sees the GPU's settled clock")
    ap.add_argument("--spread-blocks", type=int, default=5,
                    help="after the timed region, this many more blocks of K back-to-back steps "
                         "give the median and p10/p90 of the per-launch time")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="seconds of back-to-back steps after the timed blocks during which the "
                         "GPU's clocks are read (0 skips)")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timing of the other workloads, decode, formats and sweep")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warm-up, run a plain device-to-device copy of this many MiB "
                         "three times (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on a single GPU; --gpus above 1 is not supported "
              "(the operation shards over channels or sequences with no communication, "
              "so per-GPU throughput is the single-GPU figure)", file=sys.stderr)
        return 2

    import torch

    import packed_varlen_causal_depthwise_amd as kd
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.config3()
    nbytes = wl.algorithmic_bytes()
    P = wl.dim // wl.part_dim
    xb = torch.from_numpy(wl.x.view(np.int16)).to(dev).view(torch.bfloat16)
    sets = []
    for i in range(args.sets):
        x = xb.clone() if i else xb
        sets.append(dict(
            x=x[:, : wl.dim],
            st=torch.from_numpy(wl.conv_states).to(dev),
            out=torch.empty((P, wl.num_tokens, wl.part_dim), dtype=torch.bfloat16, device=dev),
        ))
    w = torch.from_numpy(wl.weight).to(dev)
    b = torch.from_numpy(wl.bias).to(dev)
    q = torch.from_numpy(wl.query_start_loc).to(dev)
    ci = torch.from_numpy(wl.cache_indices).to(dev)
    init = torch.from_numpy(wl.has_initial_state).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % len(sets)]
        kd.packed_causal_conv1d_fn(s["x"], w, b, s["st"], q, ci, init, wl.part_dim, "silu", None,
                                   out=s["out"])

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    # For comparison only: K steps right after the first W, before the GPU has settled.
    for i in range(args.warmup):
        step(i)
    first_us = back_to_back(torch, stream, step, args.steps, 1)[0]
    settled = settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)

    # The timed region: K back-to-back steps between two events on the launch stream,
    # synchronised on both sides. Every step is one launch of the kernel, so the mean
    # step is also the mean launch duration the roofline uses.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    queue_ahead(torch)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize(dev)
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # Spread: more blocks of K back-to-back steps timed the same way, one per-launch mean
    # per block.
    blocks_us = back_to_back(torch, stream, step, args.steps, args.spread_blocks)
    clocks = clocks_under_load(torch, dev, step, args.clock_seconds) if args.clock_seconds > 0 \
        else {"skipped": True}

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "settle": {"ms": args.settle_ms, "launches": settled,
                   "before_settling_us_per_step": round(float(first_us), 3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "device": device_info(torch, dev),
        "clocks": clocks,
        "config": {
            "workload": "packed varlen causal depthwise conv: 1 sequence x 16384 tokens, "
                        "dim 4608 = 3 x 1536, bf16 x read in place from rows of 9728, bf16 "
                        "output planes (3, 16384, 1536), FP32 weight + bias, SiLU, FP32 conv "
                        "state (8, 4608, 3) with initial state",
            "tokens": wl.num_tokens, "dim": wl.dim, "part_dim": wl.part_dim,
            "x_row_stride": wl.row_stride, "x_and_out": "bf16", "arithmetic": "FP32",
            "algorithmic_bytes_per_step": nbytes, "buffer_sets_rotated": args.sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(value / PEAK_HBM_GBS, 4),
            "traffic": counter_traffic(),
            "kernel": "packed_conv_kernel",
            "kernel_us": round(ms_per_step * 1e3, 3),
            "timing": "mean launch duration over the timed region's K back-to-back launches",
            "spread_blocks_of_k": summary(nbytes, blocks_us),
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    if not args.no_configs:
        # The other workloads are parity cases; their rates are reported beside the
        # headline, not as it.
        result["other_configs"] = {
            str(k): time_config(kd, torch, workloads.CONFIGS[k](), steps=20, warmup=5,
                                graph=k in (1, 2, 5))
            for k in (1, 2, 4, 5)
        }
        # Decode steps (one token per sequence) on the same channels.
        result["decode"] = {
            str(bsz): time_config(kd, torch, workloads.decode_batch(bsz), steps=20, warmup=5,
                                  decode=True, graph=True)
            for bsz in (64, 256, 1024, 4096)
        }
        # Decode steps with the decode kernel page's operands: bf16 state, width-major weight.
        result["decode_bf16_state"] = {
            str(bsz): time_config(kd, torch, workloads.decode_batch_bf16_state(bsz), steps=20,
                                  warmup=5, graph=True)
            for bsz in (64, 256, 1024, 4096)
        }
        # The same 16K-token workload with fp16 and FP32 x (output in x's format).
        result["other_formats"] = {
            fmt: time_config(kd, torch, workloads.config3(x_dtype=fmt), steps=20, warmup=5)
            for fmt in ("f16", "f32")
        }
        # The headline workload with x read from column 1 of its buffer: every lane's
        # 8-byte vector of x starts 2 bytes past an 8-byte boundary.
        result["unaligned_x"] = time_config(kd, torch, wl, steps=20, warmup=5, x_column=1)
        # Context: one sequence of 2K-8K tokens (the first rows of the headline workload).
        result["context_sweep"] = {}
        for tokens in (2048, 4096, 8192):
            sub = dataclasses.replace(wl, name=f"1 x {tokens} tokens, dim 4608, stride 9728",
                                      x=wl.x[:tokens],
                                      query_start_loc=np.array([0, tokens], dtype=np.int32))
            result["context_sweep"][str(tokens)] = time_config(kd, torch, sub, steps=20, warmup=5,
                                                               graph=True)
    if not args.no_cpu_baseline:
        configs = {k: (wl if k == 3 else workloads.CONFIGS[k]()) for k in (1, 2, 3, 4, 5)}
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_runs, configs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
