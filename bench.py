#!/usr/bin/env python3
"""Decode MoE layer bench on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload NAME] [--rows M]

A step is one forward of the whole layer (route, top-k, sort, gate/up,
down, blend) over one batch of m synthetic rows, through the C ABI.  The
default workload is the Qwen3-30B-A3B-shaped bf16 layer (H 2048, 128
experts, top-8, I 768) at m = 1; m = 8 is measured too and reported under
"detail".  Weights and inputs are resident in HBM before timing starts.

Calls rotate over R device copies of the layer, each with its own input rows
(so its own expert selection), with R chosen so that at least 600 MB of other
weights stream between two uses of a copy: no call finds its weights in the
256 MB Infinity Cache or the L2.  The headline is HIP-graph replay (decode
steps run graph-captured); stream-launched numbers are reported too.  In that
stream loop every kernel is launched with its own start/stop HIP events
(hipExtLaunchKernelGGL), whose average for the dominant kernel gives the
roofline entry.

Effective bandwidth counts ALGORITHMIC bytes: the experts each call actually
selected (from a one-time readback of the exported indices), router, bias,
shared expert, input and output rows.  The oracle (plain fp64 C, one host
thread) is timed on a bounded sample of the same workload as the CPU
baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE decode layer and effective HBM GB/s (% of peak) at m=1,8"
PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "qwen3_30b_a3b_bf16"
KERNEL_SRC_DIR = os.path.join(ROOT, "mixture_experts_decode_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "gate_up_counters.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--rows", type=int, default=1, help="m of the headline step")
    p.add_argument("--extra-rows", default="8", help="comma list of other m to report")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--all", action="store_true", help="one line per workload and m (analysis)")
    p.add_argument("--grouped-rows", default="",
                   help="with --all: comma list of m > 32 (the grouped path) for the workloads it serves")
    return p.parse_args()


# --------------------------------------------------------------- bytes model

def act_bytes(spec) -> int:
    return 4 if spec.act_fmt == "f32" else 2


def proj_bytes(p) -> int:
    """Stored bytes of one expert's copy of a projection (data + scales + biases)."""
    b = p.data[0].nbytes
    if p.scale is not None:
        b += p.scale[0].nbytes
    if p.bias is not None:
        b += p.bias[0].nbytes
    return b


def layer_bytes(layer, idx, m: int) -> dict:
    """Algorithmic bytes of one call on m rows that selected experts `idx`."""
    spec = layer.spec
    ab = act_bytes(spec)
    distinct = len(set(int(e) for e in idx.reshape(-1)))
    gu = proj_bytes(layer.gate) + proj_bytes(layer.up)
    dn = proj_bytes(layer.down)
    H, Is = spec.hidden, spec.shared_inter if spec.shared else 0
    router = spec.num_experts * H * ab + (spec.num_experts * 4 if spec.routing == "sigmoid_bias" else 0)
    shared_gu = 2 * Is * H * ab
    shared_dn = Is * H * ab
    gate_vec = H * ab if spec.shared_gated else 0
    x_in = m * H * ab
    out = m * H * ab
    te = m * spec.top_k
    total = distinct * (gu + dn) + router + shared_gu + shared_dn + gate_vec + x_in + out
    # gate_up kernel: the active experts' gate+up rows and the shared
    # expert's, the input rows, and the activations it writes.
    gate_up = distinct * gu + shared_gu + x_in + te * spec.inter * 4 + m * Is * 4
    return {"total": total, "distinct": distinct, "gate_up": gate_up,
            "routed_weights": distinct * (gu + dn), "per_expert_gate_up": gu}


def expected_distinct(spec, m: int) -> float:
    return spec.num_experts * (1.0 - (1.0 - spec.top_k / spec.num_experts) ** m)


def copies_for(layer, m: int) -> int:
    spec = layer.spec
    per_expert = proj_bytes(layer.gate) + proj_bytes(layer.up) + proj_bytes(layer.down)
    est = expected_distinct(spec, m) * per_expert + spec.num_experts * spec.hidden * act_bytes(spec)
    if spec.shared:
        est += 3 * spec.shared_inter * spec.hidden * act_bytes(spec)
    r = 1 + math.ceil(600e6 / max(est, 1.0))
    full = per_expert * spec.num_experts + est
    cap = max(1, int(60e9 // full))
    return max(2, min(r, cap, 64))


# ------------------------------------------------------------------ timing

def time_workload(name: str, m: int, steps: int, warmup: int, extra_rows=(), want_stages=True,
                  max_rows=None):
    import numpy as np
    import torch

    from mixture_experts_decode_amd import moe_decode as md
    from mixture_experts_decode_amd import synth
    from mixture_experts_decode_amd.device import DeviceLayer, to_device

    spec = synth.WORKLOADS[name]
    if max_rows:
        spec = spec.replace(rows=(max_rows,))
    layer = synth.make_layer(spec, seed=0)
    rows_all = [m] + [r for r in extra_rows if r != m and r <= spec.max_rows]
    R = max(copies_for(layer, r) for r in rows_all)
    dl = DeviceLayer(layer, max_rows=max(rows_all), copies=R)
    results = {}
    for mm in rows_all:
        xs = [to_device(np.ascontiguousarray(layer.x(block=c)[:mm]), "cuda") for c in range(R)]
        outs = [dl.new_out(mm) for _ in range(R)]
        idx = torch.empty((mm, spec.top_k), dtype=torch.int32, device="cuda")
        bytes_c = []
        for c in range(R):
            dl.forward(xs[c], mm, outs[c], idx, copy=c)
            torch.cuda.synchronize()
            bytes_c.append(layer_bytes(layer, idx.cpu().numpy(), mm))
        B = sum(b["total"] for b in bytes_c) / R
        B_gu = sum(b["gate_up"] for b in bytes_c) / R
        distinct = sum(b["distinct"] for b in bytes_c) / R

        stream = torch.cuda.Stream()
        # One graph holds R consecutive forwards (one per weight copy), as a
        # decode step's graph holds consecutive layers; a second graph holds
        # the remainder, so that exactly `steps` forwards are timed.
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for c in range(n):
                        dl.forward(xs[c], mm, outs[c], copy=c, stream=stream.cuda_stream)
            return g

        g_full = capture(R)
        rem = steps % R
        g_rem = capture(rem) if rem else None
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // R)):
            g_full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps // R):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()
        torch.cuda.synchronize()
        t_graph = (time.perf_counter() - t0) / steps

        # Stream-launched; every kernel carries its own start/stop HIP events.
        nst = md.moe_decode_num_stages(dl.plan)
        evs = []
        with torch.cuda.stream(stream):
            for _ in range(steps):
                row = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)]
                for e in row:
                    e.record(stream)          # materialise the hipEvent_t
                evs.append(row)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(warmup):
                dl.forward(xs[i % R], mm, outs[i % R], copy=i % R, stream=stream.cuda_stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                dl.forward(xs[i % R], mm, outs[i % R], copy=i % R, stream=stream.cuda_stream,
                           events=[e.cuda_event for e in evs[i]])
            torch.cuda.synchronize()
            t_stream = (time.perf_counter() - t0) / steps
        stage_ms = [0.0] * nst
        for row in evs:
            for s in range(nst):
                stage_ms[s] += row[2 * s].elapsed_time(row[2 * s + 1])
        stage_us = {md.moe_decode_stage_name(dl.plan, s): 1e3 * stage_ms[s] / steps for s in range(nst)}
        del g_full, g_rem
        results[mm] = {
            "us_graph": t_graph * 1e6, "us_stream": t_stream * 1e6, "bytes": B,
            "bytes_gate_up": B_gu, "distinct_experts": distinct, "copies": R,
            "gbps_graph": B / t_graph / 1e9, "gbps_stream": B / t_stream / 1e9,
            "stage_us": stage_us,
        }
    return layer, results


def cpu_baseline(layer, m: int, seconds: float):
    import oracle

    x = layer.x(0)[:m]
    oracle.forward(layer, x)                     # warm-up
    n, t0 = 0, time.perf_counter()
    idx = None
    while True:
        r = oracle.forward(layer, x)
        idx = r.idx
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    B = layer_bytes(layer, idx, m)["total"]
    return {"value": round(B / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} oracle calls of the same layer on input block 0, m={m} "
                      f"({dt * 1e3:.1f} ms per call, fp64, single host thread)",
            "us_per_layer": round(dt * 1e6, 1)}


def kernel_source_sha256() -> str:
    """Hash of every file under csrc/ (name and contents, sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        h.update(name.encode())
        with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_entry():
    """Calibrated HBM bytes per gate_up launch (rocprofv3 FETCH_SIZE and
    WRITE_SIZE, scaled by what they read for the plain copy kernel) from the
    committed counter summary, if it was taken on the current kernel sources;
    else None."""
    try:
        data = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if data.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return data.get("traffic_bytes_per_launch")


def stream_read_gbps(gib: int = 4) -> dict:
    """Achievable HBM bandwidth with the library's plain streaming kernels:
    a read of a 4 GiB buffer (moe_decode_bench_read) and a 1 GiB copy
    (moe_decode_bench_copy, 2 GiB moved).  The copy is also the known-size
    reference for the HBM byte counters (one launch reads and writes 1 GiB)."""
    import torch
    from mixture_experts_decode_amd import moe_decode as md

    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    half = 1 << 30
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=10):
        for _ in range(2):
            fn()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    t_read = timed(lambda: md.moe_decode_bench_read(buf.data_ptr(), nbytes, sink.data_ptr(), st))
    t_copy = timed(lambda: md.moe_decode_bench_copy(buf.data_ptr(), buf.data_ptr() + 2 * half, half, st))
    del buf
    torch.cuda.empty_cache()
    return {"read": nbytes / t_read / 1e9, "copy": 2 * half / t_copy / 1e9}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported "
              "(the decode MoE layer here is a single-GPU kernel; see DESIGN.md for how it "
              "would shard)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from mixture_experts_decode_amd import synth

    if args.all:
        for name, spec in synth.WORKLOADS.items():
            layer, res = time_workload(name, spec.rows[0], args.steps, args.warmup, spec.rows[1:])
            for mm, r in res.items():
                print(json.dumps({"workload": name, "m": mm, **{k: (round(v, 3) if isinstance(v, float) else v)
                                                               for k, v in r.items()}}), flush=True)
            del layer
            torch.cuda.empty_cache()
        grows = [int(v) for v in args.grouped_rows.split(",") if v]
        for name, spec in synth.WORKLOADS.items():
            if not grows or spec.act_fmt != "bf16" or spec.expert_fmt not in ("bf16", "mxfp4", "nvfp4", "aff4"):
                continue
            layer, res = time_workload(name, grows[0], args.steps, args.warmup, grows[1:],
                                       max_rows=max(grows))
            for mm, r in res.items():
                print(json.dumps({"workload": name, "m": mm, **{k: (round(v, 3) if isinstance(v, float) else v)
                                                               for k, v in r.items()}}), flush=True)
            del layer
            torch.cuda.empty_cache()
        return

    extra = [int(v) for v in args.extra_rows.split(",") if v]
    spec = synth.WORKLOADS[args.workload]
    # Row counts above the workload's own take the grouped path (m > 32).
    big = max([args.rows] + extra)
    layer, res = time_workload(args.workload, args.rows, args.steps, args.warmup, extra,
                               max_rows=big if big > spec.max_rows else None)
    head = res[args.rows]
    sol = stream_read_gbps()
    read_gbps = sol["read"]
    gu_us = head["stage_us"]["gate_up"]
    achieved = head["bytes_gate_up"] / (gu_us * 1e-6) / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline(layer, args.rows, args.cpu_seconds)
    detail = {}
    for mm, r in res.items():
        detail[f"m{mm}"] = {
            "us_per_layer_graph": round(r["us_graph"], 2), "us_per_layer_stream": round(r["us_stream"], 2),
            "gbps_graph": round(r["gbps_graph"], 1), "gbps_stream": round(r["gbps_stream"], 1),
            "pct_of_peak_graph": round(100 * r["gbps_graph"] / PEAK_HBM_GBPS, 1),
            "pct_of_stream_read": round(100 * r["gbps_graph"] / read_gbps, 1),
            "bytes_per_call": int(r["bytes"]), "distinct_experts": r["distinct_experts"],
            "stage_us": {k: round(v, 2) for k, v in r["stage_us"].items()},
            "copies_rotated": r["copies"],
        }
    line = {
        "metric": METRIC,
        "value": round(head["gbps_graph"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_graph"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.expert_fmt if spec.expert_fmt != "f32" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: decode MoE layer H={spec.hidden} E={spec.num_experts} "
                        f"top-{spec.top_k} I={spec.inter} experts={spec.expert_fmt} "
                        f"routing={spec.routing}" + (f" shared Is={spec.shared_inter}" if spec.shared else ""),
            "rows": args.rows,
            "timing": "HIP graph of consecutive forwards over rotated weight copies (cold caches)",
        },
        "roofline": {
            "bound": "hbm", "kernel": "gate_up", "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic_entry(),
            "bytes_per_launch": int(head["bytes_gate_up"]),
            "avg_launch_us": round(gu_us, 3),
        },
        "cpu_baseline": cpu,
        "detail": detail,
        "stream_read_gbps": round(read_gbps, 1),
        "stream_copy_gbps": round(sol["copy"], 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
