"""Benchmark: 16-layer q8 verification attention at 261888 context on one MI355X.

One step is the whole hot path over one batch of synthetic input: for each of
16 distinct layer KV allocations (own block table, own scales), the split
kernel (80 logical splits, FP32 workspace) and the combine kernel, launched
back to back on one stream.  Inputs are resident in HBM before timing starts.

Printed: one JSON line with the headline metric (ms per 16-layer attention;
also its per-step median/p10/p90 and the same step replayed as a captured HIP
graph), the roofline of the dominant kernel (split kernel: algorithmic KV
bytes per launch / its average launch time, measured with HIP events on the
launch stream), the two kernels of a layer each alone (the split kernel and
the merge+combine), the split stage and the combine from a finished
workspace, the small-q sweep
(q = 1..7 over the same KV), the box's page-read ceiling (a probe that streams
exactly the layer's K and V pages in block-table order and computes nothing),
and the CPU oracle's time on a bounded sample (rank 0, N=1 only): layer 0 of
the timed step, whose outputs are then compared with the oracle's.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--graph]
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth
V100_16LAYER_MS = 12.983        # the pages' 16-layer q8 attention on V100 (context only)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_traffic.json")
SPLIT_SRCS = [os.path.join(ROOT, "long_context_split_amd", "csrc", n)
              for n in ("split_kernel.hip", "dfv_common.h", "dfv_device.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="ctx261888_16layer")
    p.add_argument("--num-q", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="report the captured-graph step time as the value")
    p.add_argument("--no-sweep", action="store_true", help="skip the small-q sweep")
    p.add_argument("--no-extras", action="store_true",
                   help="time the step and the split kernel only (no graphs, sweep or probe; for counter runs)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="after timing, run a plain 512 MiB device-to-device copy (reference for HBM counters)")
    return p.parse_args()


def src_hash() -> str:
    """Hash of everything that shapes the split kernel's binary: its source and the
    shared headers with comments and blank lines removed (a comment edit leaves the
    code object unchanged), and the hipcc flags."""
    from long_context_split_amd import build as B
    h = hashlib.sha256()
    for p in SPLIT_SRCS:
        with open(p, "r") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    h.update(" ".join(B.HIPCC_FLAGS).encode())
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


def cpu_baseline(workload: str, d: dict, gpu: dict):
    """Time the FP64 oracle (as it stands) on one full-size layer of the timed
    step (host copies of layer 0's inputs), then compare that layer's outputs
    from the timed step with the oracle's, element by element, with the
    tolerances of the parity tests."""
    import numpy as np
    from oracle import attention as A
    a = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"], d["k_scale"],
         d["v_scale"], d["softmax_scale"])
    t0 = time.perf_counter()
    out = A.attention(*a)
    m, l, o = A.split_states(*a)
    A.combine(m, l, o)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    base = dict(value=round(dt * 16 * 1000.0, 1), unit="ms per 16-layer attention (16 x one layer)",
                cores=min(threads, os.cpu_count() or threads), kind="oracle",
                sample=f"layer 0 of {workload} (the timed step's inputs): unsplit FP64 attention + "
                       f"{A.NUM_SPLITS} split states + merge at the full context, {dt:.2f} s, scaled x16 layers")
    # |out - ref| <= 2e-3 + 2e-3 |ref|; max within 1e-5 max(1, |m|); sum 1e-5 relative;
    # numerator 1e-5 relative in the max norm of each (row, split); empty splits exact
    go = gpu["out"].astype(np.float64)
    out_excess = float(np.max(np.abs(go - out) - (2e-3 + 2e-3 * np.abs(out))))
    full = np.isfinite(m)
    empty_ok = bool(np.array_equal(np.isfinite(gpu["ws_max"]), full) and not gpu["ws_sum"][~full].any()
                    and not gpu["ws_num"][~full].any())
    dm = float(np.max(np.abs(gpu["ws_max"][full] - m[full]) / np.maximum(1.0, np.abs(m[full]))))
    dl = float(np.max(np.abs(gpu["ws_sum"][full] - l[full]) / l[full]))
    do = float(np.max(np.abs(gpu["ws_num"][full] - o[full]).max(axis=-1) / np.abs(o[full]).max(axis=-1)))
    check = dict(layer=0, outputs=int(go.size), split_states=int(full.sum()),
                 out_worst_err_minus_bound=out_excess, ws_max_rel=dm, ws_sum_rel=dl, ws_num_rel=do,
                 ok=bool(np.all(np.isfinite(go)) and out_excess <= 0 and empty_ok and max(dm, dl, do) <= 1e-5))
    return base, check


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
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

    # Every call takes the current stream at call time, so the same functions
    # run eagerly and under graph capture.
    def step():
        for inp, ws in zip(layers, wss):
            dfv.run_layer(inp, ws, desc)

    def split_only():
        for inp, ws in zip(layers, wss):
            dfv.attn_split(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens,
                           inp.k_scale, inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.scratch)

    def combine_only():
        for ws in wss:
            dfv.attn_combine(desc, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out)

    def split_kernel_only():
        for inp, cb in zip(layers, cbufs):
            dfv.attn_split_chunks(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                  inp.context_lens, inp.k_scale, inp.v_scale, *cb)

    def merge_combine_only():
        # the second kernel of dfv_attn: key-chunk states -> workspace and FP16 output
        for cb, ws in zip(cbufs, wss):
            dfv.attn_combine_chunks(desc, *cb, ws.ws_max, ws.ws_sum, ws.ws_num, ws.out)

    def timed(fn, reps):
        """Total ms of `reps` calls, and the ms of each, from HIP events on the stream."""
        cur = torch.cuda.current_stream()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(cur)
        for r in range(reps):
            fn()
            ev[r + 1].record(cur)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[-1]), [ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]

    def settle(fn, ms=60.0):
        """Run fn until `ms` of wall time have passed: after host-side pauses the
        GPU comes back at its idle clock and needs several milliseconds of
        work to reach its working clock (the first ~10 ms of a split-kernel
        loop that follows a 270 MB device-to-host copy ran up to 30% slower).
        Untimed, like the warmup."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1000.0 < ms:
            fn()
            torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        return g

    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream_total, stream_steps = timed(step, args.steps)
    graph_total, graph_steps = (None, None)
    if not args.no_extras or args.graph:
        graph_total, graph_steps = timed(capture(step).replay, args.steps)
    total_ms, per_step = (graph_total, graph_steps) if args.graph else (stream_total, stream_steps)
    ms_per_step = total_ms / args.steps
    q10, q50, q90 = (float(x) for x in np.percentile(np.asarray(per_step), [10, 50, 90]))
    # layer 0 of the timed step, kept on the host for the oracle comparison of
    # the cpu_baseline leg (later measurements rewrite the caches' last rows)
    checked = None
    if not args.no_cpu_baseline:
        checked = (layers[0].numpy(),
                   dict(out=wss[0].out.float().cpu().numpy(), ws_max=wss[0].ws_max.cpu().numpy(),
                        ws_sum=wss[0].ws_sum.cpu().numpy(), ws_num=wss[0].ws_num.cpu().numpy()))

    # dominant kernel alone (the split kernel writing key-chunk states), launched
    # on the stream; then the split stage and the combine alone as graph replays
    settle(split_kernel_only)   # the host copy above left the GPU idle
    for _ in range(args.warmup):
        split_kernel_only()
    kernel_ms = timed(split_kernel_only, args.steps)[0] / (args.steps * len(layers))
    for _ in range(args.warmup):
        merge_combine_only()
    merge_ms = timed(merge_combine_only, args.steps)[0] / (args.steps * len(layers))

    split_ms = combine_ms = None
    if not args.no_extras:
        split_ms = timed(capture(split_only).replay, args.steps)[0] / (args.steps * len(layers))
        combine_ms = timed(capture(combine_only).replay, args.steps)[0] / (args.steps * len(layers))

    # fixed-capacity graph: split size fixed at the capacity rule's 3296 tokens and
    # the launch geometry taken from max_context_len, captured once; the
    # device-side context lengths may change between replays (here they do not)
    fixed_ms = None
    if not (args.no_extras or args.no_sweep):
        dfx = dfv.make_desc(1, nq, layers[0].block_table.shape[1], L, num_splits=80,
                            split_tokens=32 * (-(-(-(-L // 80)) // 32)), softmax_scale=desc.softmax_scale)

        def step_fixed():
            for inp, ws in zip(layers, wss):
                dfv.run_layer(inp, ws, dfx)
        fixed_ms = timed(capture(step_fixed).replay, args.steps)[0] / args.steps

    # small-q sweep: q = 1..7 query tokens over the same KV, block tables and scales
    small_q = {}
    if not (args.no_sweep or args.no_extras) and nq == 8:
        for qn in range(1, 8):
            gen = torch.Generator(device="cuda")
            gen.manual_seed(9000 + qn)
            lq = [dataclasses.replace(inp, q=torch.randn((1, qn, 6, 256), generator=gen, device="cuda")
                                      .to(torch.float16)) for inp in layers]
            dq = dfv.desc_for(lq[0])
            wq = [dfv.Workspace.allocate(dq) for _ in lq]

            def step_q():
                for inp, ws in zip(lq, wq):
                    dfv.run_layer(inp, ws, dq)
            for _ in range(args.warmup):
                step_q()
            small_q[f"q{qn}"] = round(timed(step_q, args.steps)[0] / args.steps, 4)
            del lq, wq

    # page-read ceiling: the same K and V pages in block-table order, no compute
    probe = ctypes.CDLL(os.path.join(ROOT, "long_context_split_amd", "libdfv_probe.so"))
    probe.dfv_probe_page_read.restype = ctypes.c_int
    probe.dfv_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    npages = -(-L // 16)

    def probe_layers():
        for inp in layers:
            rc = probe.dfv_probe_page_read(inp.k_cache.data_ptr(), inp.v_cache.data_ptr(),
                                           inp.block_table.data_ptr(), npages, sink.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"page-read probe failed ({rc})")
    probe_ms = None
    if not args.no_extras:
        for _ in range(args.warmup):
            probe_layers()
        probe_ms = timed(probe_layers, args.steps)[0] / (args.steps * len(layers))

    # QK stage on its own: every FP32 tiled score of every layer (16 distinct
    # score buffers, like the 16 layers' KV)
    qk_ms = None
    qk_tiles = dfv.qk_tiles(desc)
    if not args.no_extras:
        sbufs = [torch.empty((1, qk_tiles, nq * 6, 32), dtype=torch.float32, device="cuda") for _ in layers]

        def qk_only():
            for inp, sb in zip(layers, sbufs):
                dfv.qk_scores(desc, inp.q, inp.k_cache, inp.block_table, inp.context_lens, inp.k_scale,
                              sb, qk_tiles)
        for _ in range(args.warmup):
            qk_only()
        qk_ms = timed(qk_only, args.steps)[0] / (args.steps * len(layers))
        del sbufs

    # KV append of the q new tokens (last q positions of each layer's context),
    # alone and followed by the attention: the whole verification pass.  Runs
    # last among the GPU measurements because it rewrites those cache rows.
    append_us = step_append_ms = None
    if not args.no_extras:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(777)
        kn = [torch.randn((nq, 1, 256), generator=gen, device="cuda").to(torch.float16) for _ in layers]
        vn = [torch.randn((nq, 1, 256), generator=gen, device="cuda").to(torch.float16) for _ in layers]
        pos = torch.arange(L - nq, L, device="cuda")
        slots = [(inp.block_table[0, pos // 16].to(torch.int64) * 16 + pos % 16).contiguous() for inp in layers]

        def append_only():
            for inp, a_k, a_v, sl in zip(layers, kn, vn, slots):
                dfv.kv_append(a_k, a_v, sl, inp.k_scale, inp.v_scale, inp.k_cache, inp.v_cache)

        def step_with_append():
            for inp, ws, a_k, a_v, sl in zip(layers, wss, kn, vn, slots):
                dfv.kv_append(a_k, a_v, sl, inp.k_scale, inp.v_scale, inp.k_cache, inp.v_cache)
                dfv.run_layer(inp, ws, desc)
        append_us = timed(capture(append_only).replay, args.steps)[0] / (args.steps * len(layers)) * 1000
        step_append_ms = timed(capture(step_with_append).replay, args.steps)[0] / args.steps

    kv_bytes_layer = 2 * L * 256          # K + V E4M3 bytes per layer: 512 B per context token
    nrows = nq * 6
    qk_bytes_layer = L * 256 + nrows * 32 * qk_tiles * 4 + nrows * 256 * 2   # K in, scores out, Q in
    ws_bytes = nrows * 80 * (256 + 2) * 4
    all_bytes_layer = kv_bytes_layer + nrows * 256 * 2 + (-(-L // 16)) * 4 + 2 * ws_bytes + nrows * 256 * 2
    achieved = kv_bytes_layer / (kernel_ms * 1e-3) / 1e9
    ceiling = kv_bytes_layer / (probe_ms * 1e-3) / 1e9 if probe_ms else None
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
                   "timing": "hip graph replay" if args.graph else "stream launches"},
        "step_ms_median": round(q50, 4),
        "step_ms_p10": round(q10, 4),
        "step_ms_p90": round(q90, 4),
        "stream_ms_per_step": round(stream_total / args.steps, 4),
        "graph_ms_per_step": round(graph_total / args.steps, 4) if graph_total else None,
        "graph_ms_per_step_fixed_split_tokens": round(fixed_ms, 4) if fixed_ms else None,
        "kv_GBps_whole_step": round(kv_bytes_layer * len(layers) / (ms_per_step * 1e-3) / 1e9, 1),
        "all_bytes_GBps_whole_step": round(all_bytes_layer * len(layers) / (ms_per_step * 1e-3) / 1e9, 1),
        "split_kernel_ms_per_launch": round(kernel_ms, 5),
        "merge_combine_ms_per_launch": round(merge_ms, 5),
        "per_layer_us": {"step_per_layer": round(ms_per_step * 1000 / len(layers), 2),
                         "split_kernel": round(kernel_ms * 1000, 2),
                         "merge_combine_and_launch": round(ms_per_step * 1000 / len(layers) - kernel_ms * 1000, 2),
                         "merge_combine_alone": round(merge_ms * 1000, 2),
                         "what": "a layer of the step = the split kernel (timed alone, back to back, as for the "
                                 "roofline) + the rest of the layer (the chunk merge + combine kernel and the "
                                 "launch gaps; step minus split); the merge alone reads chunk states written long "
                                 "before, in the step it reads the ones just written"},
        "split_stage_ms_per_call": round(split_ms, 5) if split_ms else None,
        "combine_from_workspace_ms_per_call": round(combine_ms, 5) if combine_ms else None,
        "key_chunks_per_split": dfv.chunks(desc),
        "small_q_ms_per_step": small_q or None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "split_kernel",
                     "algorithmic_bytes_per_launch": kv_bytes_layer},
        "kv_append_us_per_call": round(append_us, 2) if append_us else None,
        "graph_ms_per_step_with_kv_append": round(step_append_ms, 4) if step_append_ms else None,
        "qk_stage": {"us_per_launch": round(qk_ms * 1000, 2), "ms_per_16_layers": round(qk_ms * 16, 4),
                     "GBps": round(qk_bytes_layer / (qk_ms * 1e-3) / 1e9, 1),
                     "frac_of_peak": round(qk_bytes_layer / (qk_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "bytes_per_launch": qk_bytes_layer,
                     "what": "dfv_qk_scores alone: the layer's K pages in, every FP32 tiled score out"}
        if qk_ms else None,
        "page_read_ceiling": {"GBps": round(ceiling, 1), "us_per_layer": round(probe_ms * 1000, 2),
                              "frac_of_peak": round(ceiling / HBM_PEAK_GBPS, 4),
                              "split_kernel_frac_of_ceiling": round(achieved / ceiling, 4),
                              "what": "the layer's K and V pages in block-table order through LDS, "
                                      "no compute (libdfv_probe.so)"} if ceiling else None,
    }
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = 512 << 20
    if checked is not None:
        line["cpu_baseline"], line["timed_output_check"] = cpu_baseline(args.workload, *checked)
    else:
        line["cpu_baseline"] = line["timed_output_check"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
