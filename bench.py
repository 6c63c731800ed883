#!/usr/bin/env python3
"""Benchmark: the per-token Q4_0 weight stream through the verify GEMM, one GPU.

One step is one pass over a synthetic 27B-class weight stack: 64 layers, each
with Q4_0 matrices 8192x5120, 5120x8192, 17408x5120 (twice) and 5120x17408
(12.65 GB of codes and scales), each multiplied by that layer's 16-row bf16
draft block -- 320 verify-GEMM calls.  Inputs are drawn on the device with a
seeded generator and resident in HBM before timing starts.

Prints one JSON line: the stream's sustained HBM GB/s at 16 rows (the value),
the same at 1 and 8 rows, rows*weights/s, the verify kernel's roofline
fraction against 8 TB/s, and the CPU oracle timed on a bounded sample of the
same workload.  See the --help text for options.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
LAYERS = 64
SHAPES = ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120), (5120, 17408))
METRIC = "verify GEMM HBM GB/s (% of peak) at N_rows=1/8/16; rows·weights/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q4_0_stream.json")
KERNEL_SOURCES = ("block_quantized_gemm_amd/csrc/verify_gemm.hip", "block_quantized_gemm_amd/csrc/vq_device.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed passes over the stack")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle budget")
    return ap.parse_args()


def build_stack(layers, device):
    import torch
    import workloads as W
    mats = []
    for layer in range(layers):
        for idx, (m, k) in enumerate(SHAPES):
            codes, scales = W.q4_0_device(m, k, W.seed_of(W.CFG_STREAM, layer, 10 * idx), device)
            mats.append((layer, m, k, codes, scales))
    acts = {}
    for layer in range(layers):
        for k in sorted({k for _, k in SHAPES}):
            acts[(layer, k)] = W.act_device(16, k, W.seed_of(W.CFG_STREAM, layer, 1000 + k), device)
    outs = {m: torch.empty((16, m), dtype=torch.bfloat16, device=device) for m in {m for m, _ in SHAPES}}
    torch.cuda.synchronize()
    return mats, acts, outs


def algorithmic_bytes(mats, n_rows):
    w = sum(m * (k // 2) + m * (k // 32) * 2 for _, m, k, _, _ in mats)
    x = sum(n_rows * k * 2 for _, _, k, _, _ in mats)
    y = sum(n_rows * m * 2 for _, m, _, _, _ in mats)
    return w, w + x + y


def time_stream(vq, mats, acts, outs, n_rows, steps, warmup):
    import torch
    stream = torch.cuda.current_stream()
    views = {key: a[:n_rows] for key, a in acts.items()}
    oviews = {m: o[:n_rows] for m, o in outs.items()}

    def one_step():
        for layer, m, k, codes, scales in mats:
            vq.gemm_q4_0(codes, scales, views[(layer, k)], oviews[m], stream=stream)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def cpu_baseline(budget_s):
    """The CPU oracle on a bounded sample of the same workload: for each matrix
    shape of one layer, all 16 rows for the first F output features, with F
    doubled until the budget is used; scaled to GB/s of algorithmic bytes."""
    import numpy as np
    import oracle
    import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    feats, spent, done_bytes, done_rw = 16, 0.0, 0, 0
    sample = []
    mats = [W.stream_matrix(0, i) for i in range(len(SHAPES))]
    act = {k: W.stream_act(0, k) for k in {k for _, k in SHAPES}}
    while spent < budget_s and feats <= 17408:
        t0 = time.perf_counter()
        b = rw = 0
        for mat in mats:
            m, k = mat["M"], mat["K"]
            f = min(feats, m)
            cols = np.arange(f, dtype=np.int64)
            oracle.gemm_q4_0(mat["codes"], mat["scales"], act[k], oracle.BF16, 16, m, k, cols=cols)
            b += f * (k // 2 + (k // 32) * 2) + 16 * k * 2 + 16 * f * 2
            rw += 16 * f * k
        dt = time.perf_counter() - t0
        spent += dt
        done_bytes += b
        done_rw += rw
        sample.append(f)
        feats *= 2
    return dict(value=round(done_bytes / spent / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                rows_weights_per_s=done_rw / spent,
                sample="layer 0 of the stack, 16 rows, output features 0..F-1 of each of its 5 matrices "
                       "for F = %s; %.1f s of fp64 scalar C on %d threads" % (sample, spent, threads))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus %d is not supported" % args.gpus}))
        sys.exit(2)
    import torch
    import block_quantized_gemm_amd as vq
    vq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    mats, acts, outs = build_stack(args.layers, dev)
    n_calls = len(mats)
    ms = {}
    for n in (16, 8, 1):
        ms[n] = time_stream(vq, mats, acts, outs, n, args.steps if n == 16 else max(2, args.steps // 2),
                            args.warmup)
    w_bytes, alg16 = algorithmic_bytes(mats, 16)
    gbs = {n: algorithmic_bytes(mats, n)[1] / (ms[n] * 1e-3) / 1e9 for n in ms}
    n_weights = sum(m * k for _, m, k, _, _ in mats)
    per_launch_us = ms[16] * 1e3 / n_calls
    achieved = alg16 / n_calls / (per_launch_us * 1e-6) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(gbs[16], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms[16], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded on-device draws: Q4_0 codes uniform, fp16 scales U[0.001,0.02], bf16 rows N(0,1))",
        "config": {
            "workload": "Q4_0 per-token weight stream: %d layers x (8192x5120, 5120x8192, 17408x5120 x2, "
                        "5120x17408), %d verify-GEMM calls per step, bf16 draft block of 16 rows per layer"
                        % (args.layers, n_calls),
            "weight_bytes": w_bytes,
            "n_rows": 16,
        },
        "pct_of_hbm_peak": round(100 * gbs[16] / HBM_PEAK_GBS, 2),
        "gbs_by_rows": {str(n): round(gbs[n], 2) for n in (1, 8, 16)},
        "ms_by_rows": {str(n): round(ms[n], 4) for n in (1, 8, 16)},
        "t16_over_t1": round(ms[16] / ms[1], 4),
        "rows_weights_per_s": 16 * n_weights / (ms[16] * 1e-3),
        "roofline": {
            "bound": "hbm",
            "kernel": "vq::verify_kernel (Q4_0, bf16 activations)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(per_launch_us, 3),
            "launches_per_step": n_calls,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
