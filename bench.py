#!/usr/bin/env python3
"""Benchmark: the per-token Q4_0 weight stream through the verify GEMM, one GPU.

One step is one pass over a synthetic 27B-class weight stack: 64 layers, each
with Q4_0 matrices 8192x5120, 5120x8192, 17408x5120 (twice) and 5120x17408
(12.65 GB of codes and scales), each multiplied by that layer's 16-row bf16
draft block -- 320 verify GEMMs.  Inputs are drawn on the device with a seeded
generator and resident in HBM before timing starts.

The weights are held in the library's panel layout (vq_q4_0_to_panel: the same
Q4_0 codes and scales, 12.65 GB, rearranged once into 72 KiB records that a
workgroup reads front to back).  Each layer's five independent GEMMs go to
the library as one grouped call (one kernel launch per layer), and the step's
64 launches are replayed as one HIP graph, as an engine replays its decode
step.  The same step is also timed on the row-major Q4_0 arrays (grouped per
layer, whole-stack grouped calls, one call per matrix eager and
graph-replayed); those figures are reported beside the headline.

Prints one JSON line: the stream's sustained HBM GB/s at 16 rows (the value),
the same at 1 and 8 rows, rows*weights/s, the verify kernel's roofline fraction
against 8 TB/s, measured HBM traffic per launch (from rocprofv3 counters, while
the kernel sources are unchanged since they were taken), and the CPU oracle
timed on a bounded sample of the same workload.

Counter runs (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE) use
`--profile-run`; `--traffic-from FETCH_DIR WRITE_DIR` turns their CSV output
into the stored traffic figure.
"""
from __future__ import annotations

import argparse
import csv
import glob
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
KERNEL_SOURCES = ("block_quantized_gemm_amd/csrc/verify_gemm.hip", "block_quantized_gemm_amd/csrc/vq_device.h",
                  "block_quantized_gemm_amd/csrc/vq_internal.h", "block_quantized_gemm_amd/csrc/vq_api.cpp")
COPY_BYTES = 512 << 20  # calibration copy for the traffic counters


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace do not count,
    any other edit invalidates the stored traffic figure."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed passes over the stack")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the stream: time the prefill-sized W4A8 path (H32 int8 quantizer over 512 "
                         "bf16 rows x 5120, then the W4A8 GEMM against Q4_0 17408 x 5120) and print its "
                         "own JSON line against the int8 MFMA roofline")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline form (grouped per layer, 16 rows), so that a kernel trace of "
                         "this run holds the headline's launches alone")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-oracle budget")
    ap.add_argument("--profile-run", action="store_true",
                    help="a short run for rocprofv3 counters: a few grouped passes at 16 rows, then a "
                         "512 MiB device copy that calibrates the byte counters; prints nothing else")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output of --profile-run and store "
                         "the verify kernel's HBM bytes per launch in profiles/")
    return ap.parse_args()


def build_stack(layers, device):
    """The stack in both layouts: (layer, M, K, codes, scales, panel) per matrix."""
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    mats = []
    for layer in range(layers):
        for idx, (m, k) in enumerate(SHAPES):
            codes, scales = W.q4_0_device(m, k, W.seed_of(W.CFG_STREAM, layer, 10 * idx), device)
            mats.append((layer, m, k, codes, scales, vq.q4_0_to_panel(codes, scales)))
    acts = {}
    for layer in range(layers):
        for k in sorted({k for _, k in SHAPES}):
            acts[(layer, k)] = W.act_device(16, k, W.seed_of(W.CFG_STREAM, layer, 1000 + k), device)
    outs = {m: torch.empty((16, m), dtype=torch.bfloat16, device=device) for m in {m for m, _ in SHAPES}}
    torch.cuda.synchronize()
    return mats, acts, outs


def algorithmic_bytes(mats, n_rows):
    """Codes, scales, activations and outputs of every GEMM (the same for both
    layouts: the panel form holds the same bytes)."""
    w = sum(m * (k // 2) + m * (k // 32) * 2 for _, m, k, *_ in mats)
    x = sum(n_rows * k * 2 for _, _, k, *_ in mats)
    y = sum(n_rows * m * 2 for _, m, *_ in mats)
    return w, w + x + y


class Stream:
    """The step in its launch forms, for a given row count and weight layout
    ("panel" or "row_major")."""

    def __init__(self, vq, mats, acts, outs, n_rows, ws, layout):
        self.vq, self.mats, self.n, self.layout = vq, mats, n_rows, layout
        self.views = {key: a[:n_rows] for key, a in acts.items()}
        self.oviews = {m: o[:n_rows] for m, o in outs.items()}
        self.ws = ws
        layers = sorted({l for l, *_ in mats})

        def problem(l, m, k, c, s, p):
            if layout == "panel":
                return (p, m, self.views[(l, k)], self.oviews[m])
            return (c, s, self.views[(l, k)], self.oviews[m])
        kind = "q4_0_panel" if layout == "panel" else "q4_0"
        self.layer_calls = [vq.GroupedCall(kind, [problem(*t) for t in mats if t[0] == l], workspace=ws)
                            for l in layers]
        self.whole_call = vq.GroupedCall(kind, [problem(*t) for t in mats], workspace=ws)

    def per_call(self, stream):
        for layer, m, k, codes, scales, panel in self.mats:
            if self.layout == "panel":
                self.vq.gemm_q4_0_panel(panel, m, k, self.views[(layer, k)], self.oviews[m], workspace=self.ws,
                                        stream=stream)
            else:
                self.vq.gemm_q4_0(codes, scales, self.views[(layer, k)], self.oviews[m], workspace=self.ws,
                                  stream=stream)

    def per_layer(self, stream):
        for call in self.layer_calls:
            call(stream)

    def whole(self, stream):
        self.whole_call(stream)


def time_ms(fn, stream, steps, warmup, graph):
    """ms per step: HIP events on the launch stream around `steps` steps (or
    replays of one captured step) after `warmup` untimed ones."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            fn(stream)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                g.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            if g is not None:
                g.replay()
            else:
                fn(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


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
        sample.append(feats)
        feats *= 2
    return dict(value=round(done_bytes / spent / 1e9, 4), unit="GB/s", cores=threads, kind="oracle",
                rows_weights_per_s=done_rw / spent,
                sample="layer 0 of the stack, 16 rows, output features 0..min(F, M)-1 of each of its 5 "
                       "matrices for F = %s; %.1f s of fp64 scalar C on %d threads" % (sample, spent, threads))


def _layout_of(kernel_name):
    """The weight layout a walk-kernel dispatch ran on (its last template
    argument is the panel flag), or None for other kernels."""
    if "vq::walk_kernel<" not in kernel_name:
        return None
    return "panel" if kernel_name.split(">")[0].rstrip().endswith("true") else "row_major"


def traffic_from(fetch_dir, write_dir):
    """Per-launch HBM bytes of the verify kernel, per weight layout, from two
    counter runs of --profile-run, each scaled by what the same counter reads
    for the plain copy of COPY_BYTES in that run."""
    def per_kernel(d, counter):
        vals = {"panel": [], "row_major": [], "copy": []}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                lay = _layout_of(name)
                if lay:
                    vals[lay].append(float(r["Counter_Value"]))
                elif "copyBuffer" in name:
                    vals["copy"].append(float(r["Counter_Value"]))
        if not vals["panel"] or not vals["row_major"] or not vals["copy"]:
            raise SystemExit("no %s rows for both verify layouts and the copy in %s" % (counter, d))
        # the calibration copies are the largest device-to-device copies of the run
        top = max(vals["copy"])
        cal = [v for v in vals["copy"] if v >= 0.9 * top]
        avg = {k: sum(v) / len(v) for k, v in vals.items() if k != "copy"}
        return avg, sum(cal) / len(cal)
    fv, fc = per_kernel(fetch_dir, "FETCH_SIZE")
    wv, wc = per_kernel(write_dir, "WRITE_SIZE")
    fetch_scale, write_scale = COPY_BYTES / (fc * 1024), COPY_BYTES / (wc * 1024)
    rec = {
        "kernel_source_hash": kernel_source_hash(),
        "workload": "grouped per-layer launch, 5 stream matrices, 16 bf16 rows",
        "copy_fetch_kib": fc, "copy_write_kib": wc,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
    }
    for lay in ("panel", "row_major"):
        rec[lay] = {
            "hbm_bytes_per_launch": round(fv[lay] * 1024 * fetch_scale + wv[lay] * 1024 * write_scale),
            "read_bytes_per_launch": round(fv[lay] * 1024 * fetch_scale),
            "write_bytes_per_launch": round(wv[lay] * 1024 * write_scale),
            "fetch_kib_raw": fv[lay], "write_kib_raw": wv[lay],
        }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA, published


def fp8_forms(stream, args):
    """The FP8 block-scaled verify GEMM at the FP8 workload's two shapes and
    row counts (1, 4, 16), one call per matrix graph-replayed; enough distinct
    copies of the weights that a step reads more than the 256 MB Infinity
    Cache holds."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    dev = torch.device("cuda:0")
    res = {}
    for m, k in ((5120, 5120), (17408, 5120)):
        f = W.fp8(M=m, K=k, N=16)
        w0 = torch.from_numpy(f["w"]).to(dev)
        s0 = torch.from_numpy(f["tscales"]).to(dev)
        x = torch.from_numpy(f["act"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
        copies = max(1, -(-(600 << 20) // (m * k)))
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        wsp = vq.Workspace(vq.workspace_bytes("fp8", m, k), dev)
        by_rows = {}
        for n in (1, 4, 16):
            per_call = m * k + 4 * ((m + 127) // 128) * (k // 128) + n * k * 2 + n * m * 2
            xn = x[:n].contiguous()
            out = torch.empty((n, m), dtype=torch.bfloat16, device=dev)

            def step(s, ws=ws, s0=s0, xn=xn, out=out, wsp=wsp):
                for w in ws:
                    vq.gemm_fp8_blk128(w, s0, xn, out, workspace=wsp, stream=s)

            t = time_ms(step, stream, max(2, args.steps // 2), args.warmup, graph=True)
            by_rows[str(n)] = round(copies * per_call / (t * 1e-3) / 1e9, 2)
        res["%dx%d" % (m, k)] = by_rows
        del ws
    return res


GREEDY_VOCAB = 151936  # a synthetic vocabulary of 151,936 entries


def greedy_form(stream, args):
    """Greedy verification of a 16-row block over bf16 logits [16][V]: time per
    call, one call per copy graph-replayed over enough copies of the logits
    that a step reads them from HBM; bytes = the logits read once."""
    import torch
    import block_quantized_gemm_amd as vq
    dev = torch.device("cuda:0")
    n, v = 16, GREEDY_VOCAB
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    lg0 = torch.randn((n, v), generator=g, device=dev).to(torch.bfloat16)
    copies = -(-(600 << 20) // lg0.numel() // 2)
    lgs = [lg0] + [lg0.clone() for _ in range(copies - 1)]
    draft = torch.zeros(n - 1, dtype=torch.int32, device=dev)
    tokens = torch.empty(n, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    ws = vq.Workspace(vq.greedy_workspace_bytes(n, v), dev)

    def step(s):
        for lg in lgs:
            vq.greedy_verify(lg, draft, tokens, count, workspace=ws, stream=s)

    t = time_ms(step, stream, max(2, args.steps // 2), args.warmup, graph=True)
    us = t * 1e3 / copies
    gbs = n * v * 2 / (us * 1e-6) / 1e9
    del lgs
    return {"rows": n, "vocab": v, "logits_dtype": "bf16", "us_per_call": round(us, 2), "gbs": round(gbs, 2),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def prefill_bench(args):
    """The prefill-sized W4A8 path on synthetic inputs shaped as its workload."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    vq.lib()
    p = W.prefill()
    N, M, K = p["N"], p["M"], p["K"]
    dev = torch.device("cuda:0")
    codes0 = torch.from_numpy(p["codes"]).to(dev)
    scales0 = torch.from_numpy(p["scales"].view(np.int16).copy()).to(dev).view(torch.float16)
    x = torch.from_numpy(p["act"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
    q = torch.empty((N, K), dtype=torch.int8, device=dev)
    d = torch.empty((N, K // 32), dtype=torch.float16, device=dev)
    out = torch.empty((N, M), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    # the path's weights: the plain Q4_0 matrix rotated once, offline
    codes = torch.empty_like(codes0)
    scales = torch.empty_like(scales0)
    t_rot = time_ms(lambda s: vq.q4_0_rotate_h32(codes0, scales0, codes, scales, stream=s), stream, 3, 1, graph=False)

    def quant(s):
        vq.hadamard32_quant_int8(x, q, d, stream=s)

    def gemm(s):
        vq.gemm_q4_0(codes, scales, q, out, x_scales=d, alpha=1.0 / 32, stream=s)

    def both(s):
        quant(s)
        gemm(s)

    t_q = time_ms(quant, stream, args.steps, args.warmup, graph=True)
    t_g = time_ms(gemm, stream, args.steps, args.warmup, graph=True)
    t_b = time_ms(both, stream, args.steps, args.warmup, graph=True)
    ops = 2.0 * N * M * K
    tops = ops / (t_g * 1e-3) / 1e12
    # error of the rotated W4A8 result against the bf16-row verify GEMM on the
    # plain weights (itself within ~1e-6 of the exact product)
    with torch.cuda.stream(stream):
        both(stream)
    ref = torch.empty((N, M), dtype=torch.float32, device=dev)
    vq.gemm_q4_0(codes0, scales0, x, ref, stream=stream)
    torch.cuda.synchronize()
    rel = float(torch.linalg.norm((out - ref).double()) / torch.linalg.norm(ref.double()))
    # the 4-bit activation codes of the same section (W4A4 numerics): the same
    # GEMM on codes in [-7, 7]
    q4 = torch.empty_like(q)
    d4 = torch.empty_like(d)
    out4 = torch.empty_like(out)

    def quant4(s):
        vq.hadamard32_quant_int4(x, q4, d4, stream=s)

    def gemm4(s):
        vq.gemm_q4_0(codes, scales, q4, out4, x_scales=d4, alpha=1.0 / 32, stream=s)

    t_q4 = time_ms(quant4, stream, args.steps, args.warmup, graph=True)
    t_g4 = time_ms(gemm4, stream, args.steps, args.warmup, graph=True)
    with torch.cuda.stream(stream):
        quant4(stream)
        gemm4(stream)
    torch.cuda.synchronize()
    rel4 = float(torch.linalg.norm((out4 - ref).double()) / torch.linalg.norm(ref.double()))
    tops4 = ops / (t_g4 * 1e-3) / 1e12
    w4a4 = {"workload": "4-bit activation codes (H32, bound 7) of the same rows, the same GEMM",
            "quantizer_us": round(t_q4 * 1e3, 2), "gemm_us": round(t_g4 * 1e3, 2), "tops": round(tops4, 2),
            "rel_error_vs_bf16_rows": round(rel4, 4),
            "roofline": {"bound": "mfma", "achieved": round(tops4, 2), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(tops4 / INT8_MFMA_PEAK_TOPS, 4)}}
    fp8 = fp8_prefill_form(stream, args, N)
    result = {
        "metric": "W4A8 prefill int8-MFMA TOPS",
        "value": round(tops, 2),
        "unit": "TOPS",
        "higher_is_better": True,
        "dtype": "i8",
        "data": "synthetic (Q4_0 codes uniform, fp16 scales lognormal; bf16 rows Student-t with outlier channels)",
        "config": {"workload": "W4A8 prefill: %d bf16 rows x K=%d, H32 int8 quantizer, then Q4_0 %d x %d "
                               "(H32-rotated offline) W4A8 GEMM (exact integer block dots on the 16-bit MFMA), "
                               "fp32 out" % (N, K, M, K)},
        "gemm_us": round(t_g * 1e3, 2),
        "quantizer_us": round(t_q * 1e3, 2),
        "quantizer_plus_gemm_us": round(t_b * 1e3, 2),
        "offline_rotation_us": round(t_rot * 1e3, 2),
        "rel_error_vs_bf16_rows": round(rel, 4),
        "roofline": {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4), "ops_per_launch": ops,
                     # the integer dots run on the fp16 16x16x32 MFMA, whose dense peak is the bf16/fp16 one
                     "mfma_used": "f16 16x16x32", "frac_of_mfma_used": round(tops / BF16_MFMA_PEAK_TFLOPS, 4)},
        "w4a4": w4a4,
        "fp8_prefill": fp8,
    }
    print(json.dumps(result))


def fp8_prefill_form(stream, args, N):
    """The FP8 block-scaled GEMM over N bf16 rows at 17408 x 5120 (the FP8
    workload's distributions) on the MFMA-tiled kernel, against the bf16 MFMA
    peak; the verify kernel on the same rows (16 at a time) for context."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    dev = torch.device("cuda:0")
    f = W.fp8(M=17408, K=5120, N=16)
    M, K = f["M"], f["K"]
    w = torch.from_numpy(f["w"]).to(dev)
    ts = torch.from_numpy(f["tscales"]).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    x = torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((N, M), dtype=torch.bfloat16, device=dev)
    t_p = time_ms(lambda s: vq.gemm_fp8_blk128_prefill(w, ts, x, out, stream=s), stream, args.steps, args.warmup, True)
    t_v = time_ms(lambda s: vq.gemm_fp8_blk128(w, ts, x, out, stream=s), stream, max(2, args.steps // 2),
                  args.warmup, True)
    flops = 2.0 * N * M * K
    tf = flops / (t_p * 1e-3) / 1e12
    return {"workload": "FP8 block-scaled prefill: %d bf16 rows x 17408 x 5120, bf16 out" % N,
            "gemm_us": round(t_p * 1e3, 2), "tflops": round(tf, 2),
            "verify_kernel_us": round(t_v * 1e3, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": flops}}


def main():
    args = parse()
    if args.prefill:
        prefill_bench(args)
        return
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus %d is not supported" % args.gpus}))
        sys.exit(2)
    import torch
    import block_quantized_gemm_amd as vq
    vq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()

    layers = min(args.layers, 8) if args.profile_run else args.layers
    mats, acts, outs = build_stack(layers, dev)
    # one workspace for every call below: the larger of the two layouts' needs
    # (panel tile groups are 256 features wide, their pieces twice the size)
    need = max(vq.GroupedCall("q4_0", [(c, s, acts[(0, k)], outs[m]) for _, m, k, c, s, _ in mats[:32]],
                              workspace=None).workspace_bytes,
               vq.GroupedCall("q4_0_panel", [(p, m, acts[(0, k)], outs[m]) for _, m, k, _, _, p in mats[:32]],
                              workspace="auto").workspace_bytes)
    ws = vq.Workspace(need + (1 << 20), dev)
    streams = {n: Stream(vq, mats, acts, outs, n, ws, "panel") for n in (16, 8, 1)}
    row_major = {n: Stream(vq, mats, acts, outs, n, ws, "row_major") for n in (16, 1)}

    if args.profile_run:
        with torch.cuda.stream(stream):
            for _ in range(3):
                streams[16].per_layer(stream)
            for _ in range(3):
                row_major[16].per_layer(stream)
        torch.cuda.synchronize()
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print("profile run done: %d layers" % layers, flush=True)
        return

    n_launch = len(streams[16].layer_calls)
    ms = {}
    rows = (16,) if args.headline_only else (16, 8, 1)
    for n in rows:
        ms[n] = time_ms(streams[n].per_layer, stream, args.steps if n == 16 else max(2, args.steps // 2),
                        args.warmup, graph=True)
    extra = {"panel_grouped_per_layer_graph": ms[16]}
    rm_ms = {}
    if not args.headline_only:
        half = max(2, args.steps // 2)
        extra["panel_grouped_whole_stack_graph"] = time_ms(streams[16].whole, stream, half, args.warmup, True)
        extra["panel_per_call_graph"] = time_ms(streams[16].per_call, stream, half, args.warmup, True)
        for n in (16, 1):
            rm_ms[n] = time_ms(row_major[n].per_layer, stream, half, args.warmup, True)
        extra["row_major_grouped_per_layer_graph"] = rm_ms[16]
        extra["row_major_grouped_whole_stack_graph"] = time_ms(row_major[16].whole, stream, half, args.warmup,
                                                               True)
        extra["row_major_per_call_graph"] = time_ms(row_major[16].per_call, stream, half, args.warmup, True)
        extra["row_major_per_call_eager"] = time_ms(row_major[16].per_call, stream, half, args.warmup, False)
        extra_fp8 = fp8_forms(stream, args)
        greedy = greedy_form(stream, args)
    w_bytes, alg16 = algorithmic_bytes(mats, 16)
    gbs = {n: algorithmic_bytes(mats, n)[1] / (ms[n] * 1e-3) / 1e9 for n in ms}
    n_weights = sum(m * k for _, m, k, *_ in mats)
    per_launch_us = ms[16] * 1e3 / n_launch
    achieved = alg16 / n_launch / (per_launch_us * 1e-6) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("panel", {}).get("hbm_bytes_per_launch")

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
                        "5120x17408), 16-row bf16 draft block per layer; weights in the library's panel "
                        "layout (same bytes as row-major Q4_0); each layer's 5 GEMMs one grouped call, the "
                        "step's %d launches replayed as one HIP graph" % (args.layers, n_launch),
            "weight_bytes": w_bytes,
            "n_rows": 16,
        },
        "pct_of_hbm_peak": round(100 * gbs[16] / HBM_PEAK_GBS, 2),
        "gbs_by_rows": {str(n): round(gbs[n], 2) for n in rows},
        "ms_by_rows": {str(n): round(ms[n], 4) for n in rows},
        "t16_over_t1": round(ms[16] / ms[1], 4) if 1 in ms else None,
        "row_major_gbs_by_rows": {str(n): round(algorithmic_bytes(mats, n)[1] / (t * 1e-3) / 1e9, 2)
                                  for n, t in rm_ms.items()},
        "row_major_t16_over_t1": round(rm_ms[16] / rm_ms[1], 4) if rm_ms else None,
        "rows_weights_per_s": 16 * n_weights / (ms[16] * 1e-3),
        "launch_forms_gbs_16_rows": {k: round(alg16 / (v * 1e-3) / 1e9, 2) for k, v in extra.items()},
        "fp8_blk128_gbs_by_rows": None if args.headline_only else extra_fp8,
        "greedy_verify": None if args.headline_only else greedy,
        "roofline": {
            "bound": "hbm",
            "kernel": "vq::walk_kernel (Q4_0 panel layout, bf16 activations, grouped per layer)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(per_launch_us, 3),
            "launches_per_step": n_launch,
            "algorithmic_bytes_per_launch": alg16 // n_launch,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
