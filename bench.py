"""Benchmark: achieved HBM bandwidth of the packed causal conv on one MI355X.

A step is one call of the whole path (program map, history, taps, SiLU, bf16
planes, state update) on the headline workload: one sequence of 16384 tokens,
dim 4608 = 3 x 1536 packed Q|K|V channels read in place from rows of 9728
elements, FP32 weight and bias, SiLU, FP32 conv state with an initial state.
Inputs are synthetic (seeded, workloads.config3) and resident in HBM before
timing starts. Several complete buffer sets (x, out, state) rotate so that no
step finds its inputs in the 256 MB Infinity Cache from the previous step.

value = algorithmic bytes per step / mean wall time per step (HIP events around
the K timed steps); roofline.achieved = the same bytes / mean kernel duration
(HIP event pair around each launch, on the launch stream). Algorithmic bytes:
x read once and out written once (2 B per element each), the state line read
and written (12 B per channel each), weight (16 B per channel), bias (4 B per
channel), metadata (workloads.Workload.algorithmic_bytes).

cpu_baseline: the CPU oracle as it stands (single thread) on the same workload.

Beside the headline (parity cases and context, not the metric): per-launch times
of the four other named workloads, decode batches, fp16 and FP32 x, and one
sequence of 2K, 4K and 8K tokens.

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


def time_config(kd, torch, wl, steps: int, warmup: int, sets: int = 2):
    """Per-launch HIP-event times of the kernel on one workload, with `sets` complete
    input/output/state sets rotated (two sets of the 16K-token workloads exceed the
    256 MB Infinity Cache; the small workloads stay cache-resident, as they would in
    use)."""
    dev = torch.device("cuda:0")
    P = wl.dim // wl.part_dim
    xb = x_tensor(torch, wl, dev)
    bufs = []
    for i in range(sets):
        x = xb.clone() if i else xb
        bufs.append(dict(
            x=x[:, : wl.dim],
            st=torch.from_numpy(wl.conv_states.copy()).to(dev),
            out=torch.empty((P, wl.num_tokens, wl.part_dim), dtype=xb.dtype, device=dev),
        ))
    w = torch.from_numpy(wl.weight).to(dev)
    b = None if wl.bias is None else torch.from_numpy(wl.bias).to(dev)
    q = torch.from_numpy(wl.query_start_loc).to(dev)
    ci = torch.from_numpy(wl.cache_indices).to(dev)
    init = torch.from_numpy(wl.has_initial_state).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = bufs[i % sets]
        kd.packed_causal_conv1d_fn(s["x"], w, b, s["st"], q, ci, init, wl.part_dim, wl.activation,
                                   wl.null_block_id, out=s["out"])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, z) in enumerate(evs):
        a.record(stream)
        step(i)
        z.record(stream)
    torch.cuda.synchronize(dev)
    us = np.array([a.elapsed_time(z) for a, z in evs]) * 1e3
    med = float(np.median(us))
    nbytes = wl.algorithmic_bytes()
    return {
        "workload": wl.name + ("" if wl.x_dtype == "bf16" else f", x and out {wl.x_dtype}"),
        "algorithmic_bytes": nbytes,
        "kernel_us_median": round(med, 3),
        "kernel_us_p10_p90": [round(float(np.percentile(us, 10)), 3),
                              round(float(np.percentile(us, 90)), 3)],
        "GB/s": round(nbytes / med / 1e3, 1),
        "pct_of_peak": round(100.0 * nbytes / med / 1e3 / PEAK_HBM_GBS, 2),
    }


def time_decode(kd, torch, wl, steps: int, warmup: int, sets: int = 4):
    """Per-launch HIP-event times of the decode entry point on a decode batch (one
    token per sequence, history from the stored lines)."""
    dev = torch.device("cuda:0")
    P = wl.dim // wl.part_dim
    xb = x_tensor(torch, wl, dev)
    bufs = []
    for i in range(sets):
        x = xb.clone() if i else xb
        bufs.append(dict(
            x=x[:, : wl.dim],
            st=torch.from_numpy(wl.conv_states.copy()).to(dev),
            out=torch.empty((P, wl.num_tokens, wl.part_dim), dtype=xb.dtype, device=dev),
        ))
    w = torch.from_numpy(wl.weight).to(dev)
    b = None if wl.bias is None else torch.from_numpy(wl.bias).to(dev)
    ci = torch.from_numpy(wl.cache_indices).to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = bufs[i % sets]
        kd.packed_causal_conv1d_update(s["x"], w, b, s["st"], ci, wl.part_dim, wl.activation,
                                       wl.null_block_id, out=s["out"])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, z) in enumerate(evs):
        a.record(stream)
        step(i)
        z.record(stream)
    torch.cuda.synchronize(dev)
    us = np.array([a.elapsed_time(z) for a, z in evs]) * 1e3
    med = float(np.median(us))
    nbytes = wl.algorithmic_bytes()
    return {
        "workload": wl.name,
        "algorithmic_bytes": nbytes,
        "kernel_us_median": round(med, 3),
        "kernel_us_p10_p90": [round(float(np.percentile(us, 10)), 3),
                              round(float(np.percentile(us, 90)), 3)],
        "GB/s": round(nbytes / med / 1e3, 1),
        "pct_of_peak": round(100.0 * nbytes / med / 1e3 / PEAK_HBM_GBS, 2),
    }


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


def cpu_baseline(wl, runs: int):
    import oracle

    times = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle.run_workload(wl)
        times.append(time.perf_counter() - t)
    med = float(np.median(times))
    return {
        "value": round(wl.algorithmic_bytes() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"the whole workload ({wl.num_tokens} tokens x {wl.dim} channels), "
                  f"{runs} runs, median {med:.2f} s per run, single thread",
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="buffer sets rotated across steps")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-launch timing of the other four workloads")
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

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)

    # Timed region 1: K back-to-back steps (whole-job throughput).
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize(dev)
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # Timed region 2: an event pair around each launch (kernel duration).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, z) in enumerate(evs):
        a.record(stream)
        step(i)
        z.record(stream)
    torch.cuda.synchronize(dev)
    kern_ms = np.array([a.elapsed_time(z) for a, z in evs])
    kernel_ms = float(kern_ms.mean())

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "device": device_info(torch, dev),
        "config": {
            "workload": "packed varlen causal depthwise conv: 1 sequence x 16384 tokens, "
                        "dim 4608 = 3 x 1536 (x row stride 9728), FP32 weight + bias, SiLU, "
                        "FP32 conv state (8, 4608, 3) with initial state",
            "tokens": wl.num_tokens, "dim": wl.dim, "part_dim": wl.part_dim,
            "x_row_stride": wl.row_stride, "algorithmic_bytes_per_step": nbytes,
            "buffer_sets_rotated": args.sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": counter_traffic(),
            "kernel_us": round(kernel_ms * 1e3, 3),
            "kernel_us_p10_p90": [round(float(np.percentile(kern_ms, 10)) * 1e3, 3),
                                  round(float(np.percentile(kern_ms, 90)) * 1e3, 3)],
            "kernel": "packed_conv_kernel",
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    if not args.no_configs:
        # The other workloads are parity cases; their rates are reported beside the
        # headline, not as it.
        result["other_configs"] = {
            str(k): time_config(kd, torch, workloads.CONFIGS[k](), steps=100, warmup=10)
            for k in (1, 2, 4, 5)
        }
        # Decode steps (one token per sequence) on the same channels.
        result["decode"] = {
            str(bsz): time_decode(kd, torch, workloads.decode_batch(bsz), steps=100, warmup=10)
            for bsz in (64, 256, 1024, 4096)
        }
        # The same 16K-token workload with fp16 and FP32 x (output in x's format).
        result["other_formats"] = {
            fmt: time_config(kd, torch, workloads.config3(x_dtype=fmt), steps=100, warmup=10)
            for fmt in ("f16", "f32")
        }
        # Context: one sequence of 2K-16K tokens (the first rows of the headline workload),
        # enough buffer sets rotated that they exceed the Infinity Cache.
        result["context_sweep"] = {}
        for tokens in (2048, 4096, 8192):
            sub = dataclasses.replace(wl, name=f"1 x {tokens} tokens, dim 4608, stride 9728",
                                      x=wl.x[:tokens],
                                      query_start_loc=np.array([0, tokens], dtype=np.int32))
            set_bytes = tokens * (wl.row_stride + wl.dim) * 2
            result["context_sweep"][str(tokens)] = time_config(
                kd, torch, sub, steps=100, warmup=10, sets=max(2, -(-(600 << 20) // set_bytes)))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_runs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
