"""Benchmark: 16-layer q8 verification attention at 261888 context on one MI355X.

One step is the whole hot path over one batch of synthetic input: for each of
16 distinct layer KV allocations (own block table, own scales), the split
kernel (80 logical splits, FP32 workspace) and the combine kernel, launched
back to back on one stream.  Inputs are resident in HBM before timing starts.

Printed: one JSON line with the headline metric (ms per 16-layer attention),
the roofline of the dominant kernel (split kernel: algorithmic KV bytes per
launch / its average launch time, measured with HIP events on the launch
stream), and the CPU oracle's time on a bounded sample (rank 0, N=1 only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--graph]
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

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
V100_16LAYER_MS = 12.983        # the pages' 16-layer q8 attention on V100 (context only)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")
SPLIT_SRCS = [os.path.join(ROOT, "long_context_split_amd", "csrc", "split_kernel.hip"),
              os.path.join(ROOT, "long_context_split_amd", "csrc", "dfv_common.h"),
              os.path.join(ROOT, "long_context_split_amd", "build.py")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="ctx261888_16layer")
    p.add_argument("--num-q", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="time a captured HIP graph of the step")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after timing, run a plain 512 MiB device-to-device copy (reference for HBM counters)")
    return p.parse_args()


def src_hash() -> str:
    """Hash of everything that shapes the split kernel's binary (source, shared header, flags)."""
    h = hashlib.sha256()
    for p in SPLIT_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_bytes_alg: float):
    """HBM bytes per split launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("split_kernel_sha256_16") != src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(workload: str, num_q: int):
    """Time the FP64 oracle (as it stands) on one full-size layer of the workload."""
    import numpy as np
    from long_context_split_amd import synth
    from oracle import attention as A
    inp = synth.workload_layer(workload, 0, num_q=num_q, device="cpu")
    d = inp.numpy()
    a = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"], d["k_scale"],
         d["v_scale"], d["softmax_scale"])
    t0 = time.perf_counter()
    A.attention(*a)
    m, l, o = A.split_states(*a)
    A.combine(m, l, o)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=round(dt * 16 * 1000.0, 1), unit="ms per 16-layer attention (16 x one layer)",
                cores=min(threads, os.cpu_count() or threads), kind="oracle",
                sample=f"layer 0 of {workload}: unsplit FP64 attention + {A.NUM_SPLITS} split states "
                       f"+ merge at the full context, {dt:.2f} s, scaled x16 layers")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_split_amd import dfv, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dfv.lib()   # fail loudly if the HIP library is missing
    w = synth.WORKLOADS[args.workload]
    nq = args.num_q if args.num_q is not None else w["num_q"][0]
    layers = [synth.workload_layer(args.workload, i, num_q=nq, device="cuda") for i in range(w["layers"])]
    L = w["context"]
    desc = dfv.desc_for(layers[0])
    wss = [dfv.Workspace.allocate(desc) for _ in layers]
    cbufs = [dfv.chunk_buffers(desc) for _ in layers]
    stream = torch.cuda.current_stream()

    def step():
        for inp, ws in zip(layers, wss):
            dfv.run_layer(inp, ws, desc, stream)

    def split_only():
        for inp, ws in zip(layers, wss):
            dfv.attn_split(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                           inp.k_scale, inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.scratch, stream)

    def split_kernel_only():
        for inp, cb in zip(layers, cbufs):
            dfv.attn_split_chunks(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                  inp.context_lens, inp.k_scale, inp.v_scale, *cb, stream)

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    total_ms = timed(run, args.steps)
    ms_per_step = total_ms / args.steps

    # dominant kernel alone (the split kernel writing key-chunk states), then the
    # split stage (split kernel + chunk merge), same stream, same layers
    for _ in range(args.warmup):
        split_kernel_only()
    kernel_ms = timed(split_kernel_only, args.steps) / (args.steps * len(layers))
    split_ms = timed(split_only, args.steps) / (args.steps * len(layers))

    kv_bytes_layer = 2 * L * 256          # K + V E4M3 bytes per layer: 512 B per context token
    nrows = nq * 6
    ws_bytes = nrows * 80 * (256 + 2) * 4
    all_bytes_layer = kv_bytes_layer + nrows * 256 * 2 + (-(-L // 16)) * 4 + 2 * ws_bytes + nrows * 256 * 2
    achieved = kv_bytes_layer / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(kv_bytes_layer)

    line = {
        "metric": "ms per 16-layer q8 verify attention @261888 ctx; achieved HBM GB/s vs peak",
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms_per_step / V100_16LAYER_MS, 5),
        "vs_baseline_note": "value / 12.983 ms, the pages' V100 16-layer figure (other hardware; context only)",
        "dtype": "e4m3 KV, fp16 Q, fp32 accumulate/state",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": len(layers), "context": L, "num_q": nq,
                   "q_heads": 6, "kv_heads": 1, "head_dim": 256, "page_tokens": 16, "splits": 80,
                   "timing": "hip graph replay" if graph else "stream launches"},
        "kv_GBps_whole_step": round(kv_bytes_layer * len(layers) / (ms_per_step * 1e-3) / 1e9, 1),
        "all_bytes_GBps_whole_step": round(all_bytes_layer * len(layers) / (ms_per_step * 1e-3) / 1e9, 1),
        "split_kernel_ms_per_launch": round(kernel_ms, 5),
        "split_stage_ms_per_call": round(split_ms, 5),
        "key_chunks_per_split": dfv.chunks(desc),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "split_kernel",
                     "algorithmic_bytes_per_launch": kv_bytes_layer},
    }
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = 512 << 20
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, nq)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
