#!/usr/bin/env python3
"""Benchmark: the block-quantized verify GEMM on one GPU, every workload.

The headline step is one pass over the per-token Q4_0 weight stream: 64
synthetic layers, each with Q4_0 matrices 8192x5120, 5120x8192, 17408x5120
(twice) and 5120x17408 (12.65 GB of codes and scales), each multiplied by that
layer's 16-row bf16 draft block -- 320 verify GEMMs.  The weights are held in
the library's panel layout (the same Q4_0 codes and scales rearranged once
into 72 KiB records), each layer's five GEMMs are one grouped call (one
kernel launch per layer), and the step's 64 launches are replayed as one HIP
graph, as an engine replays its decode step.  The same step runs at 8 and 1
rows (t16/t1) and in other launch forms and on the row-major arrays.

Beside it, in the same run and process:
  tiny     Q4_0 256 x 512, 8 fp16 rows (the correctness config; latency);
  ffn      Q4_0 17408 x 5120 at 1, 8 and 16 bf16 rows, one call per matrix
           over 41 copies of the weights (> 2 GB, far beyond the 256 MB
           Infinity Cache), row-major arrays (vq_gemm_q4_0) and panel layout;
  fp8      FP8 E4M3 with 128 x 128 fp32 tile scales at 5120 x 5120 and
           17408 x 5120, 1, 4 and 16 rows, > 2 GB of copies;
  prefill  512 bf16 rows: H32 int8 quantizer, then the W4A8 GEMM against
           Q4_0 17408 x 5120 rotated offline, against the int8 MFMA peak;
           the 4-bit activation codes through the same GEMM; the FP8
           block-scaled prefill GEMM at the same shape against the bf16 peak;
  greedy   greedy verification of a 16-row block over 151,936 bf16 logits;
  probe    the library's HBM read probe over 2 GiB (the bandwidth a plain read
           reaches on this device).
Every GPU figure is a median over >= 8 repetitions timed with HIP events on
the launch stream (min and max beside it), after discarded warm-ups.  The
CPU oracle (fp64 scalar C, OpenMP over output features, all host threads) is
timed on a bounded sample of each workload.  Inputs are seeded synthetic
draws resident in HBM before any timing starts.

Prints one JSON line.  Counter runs (rocprofv3 --pmc FETCH_SIZE, then
WRITE_SIZE) use `--profile-run`; `--traffic-from FETCH_DIR WRITE_DIR` turns
their CSV output into the stored traffic figure.  `--only PART` runs one part
(for kernel traces).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA, published
LAYERS = 64
SHAPES = ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120), (5120, 17408))
METRIC = "verify GEMM HBM GB/s (% of peak) at N_rows=1/8/16; rows·weights/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q4_0_stream.json")
KERNEL_SOURCES = ("block_quantized_gemm_amd/csrc/verify_gemm.hip", "block_quantized_gemm_amd/csrc/vq_device.h",
                  "block_quantized_gemm_amd/csrc/vq_internal.h", "block_quantized_gemm_amd/csrc/vq_api.cpp")
COPY_BYTES = 512 << 20  # calibration copy for the traffic counters
COPIES_BYTES = 2100 << 20  # weight copies per single-matrix measurement (> 8x the Infinity Cache)
PARTS = ("stream", "tiny", "ffn", "fp8", "fp8stream", "prefill", "greedy", "probe")


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code and the compiler flags: comments and
    whitespace do not count, any other edit invalidates the stored traffic
    figure."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    # the compiler flags shape the machine code too (include paths aside)
    from block_quantized_gemm_amd import build
    flags = [f for f in build.HIPCC_FLAGS if not f.startswith("-I")]
    for src in sorted(build.SOURCE_FLAGS):
        flags += [src, *build.SOURCE_FLAGS[src]]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed passes over the stack (>= 8 recommended)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--reps", type=int, default=10, help="timed repetitions of every other measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="CPU-oracle budget per workload")
    ap.add_argument("--only", choices=PARTS, help="run one part only and print its figures")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline form (grouped per layer, 16 rows), so that a kernel trace of "
                         "this run holds the headline's launches alone")
    ap.add_argument("--profile-run", action="store_true",
                    help="a short run for rocprofv3 counters: a few grouped passes at 16 rows (Q4_0 and E4M3, "
                         "both layouts), then a 512 MiB device copy that calibrates the byte counters; prints "
                         "nothing else")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output of --profile-run and store "
                         "the verify kernels' HBM bytes per launch in profiles/")
    return ap.parse_args()


# ---------------------------------------------------------------------------- timing


def timed(fn, stream, reps, warmup, graph=True, inner=1):
    """Run fn(stream) `warmup` times untimed (then capture it `inner` times
    back to back as one HIP graph if `graph`), then `reps` timed repetitions
    of that graph, each between two HIP events on `stream`.  Returns mean
    (total / reps), median, min and max milliseconds per call of fn (a
    repetition's time / inner).  A graph replay costs tens of microseconds of
    host-side submission, which a kernel shorter than that cannot hide: such
    kernels are timed with inner > 1."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            fn(stream)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(inner):
                fn(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(max(1, warmup)):
                g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for i in range(reps):
            if g is not None:
                g.replay()
            else:
                for _ in range(inner):
                    fn(stream)
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / inner for i in range(reps))
    mid = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    return {"mean_ms": ev[0].elapsed_time(ev[reps]) / reps / inner, "median_ms": mid, "min_ms": per[0],
            "max_ms": per[-1], "reps": reps, "inner": inner}


def rate(t, amount, scale):
    """{median, min, max} of amount / time (ms) / scale, rounded; min rate from
    the slowest repetition."""
    return {"median": round(amount / (t["median_ms"] * 1e-3) / scale, 2),
            "min": round(amount / (t["max_ms"] * 1e-3) / scale, 2),
            "max": round(amount / (t["min_ms"] * 1e-3) / scale, 2)}


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "threads_used": threads}


def smi_clocks(doc):
    """Clock readings of rocm-smi --showclocks --json: {card: {clock: speed}}."""
    if not isinstance(doc, dict):
        return None
    return {card: {k.replace(" clock speed:", "").strip(): v for k, v in vals.items() if "clock speed" in k}
            for card, vals in doc.items() if isinstance(vals, dict) and card.startswith("card")}


def smi_other_processes(doc, own_pid):
    """Processes that rocm-smi --showpids --json lists on the GPU, other than
    own_pid: [(pid, name)].  Entries look like {"PID123": "python3, 1, ..."}."""
    if not isinstance(doc, dict):
        return None
    found = []
    for vals in doc.values():
        if not isinstance(vals, dict):
            continue
        for key, val in vals.items():
            if not key.startswith("PID"):
                continue
            try:
                pid = int(key[3:])
            except ValueError:
                continue
            if pid != own_pid:
                found.append((pid, str(val).split(",")[0].strip()))
    return sorted(found)


def _smi(flag):
    import shutil
    import subprocess
    tool = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    try:
        r = subprocess.run([tool, flag, "--json"], capture_output=True, text=True, timeout=30)
        return json.loads(r.stdout) if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError, ValueError):
        return None


def gpu_state():
    """The GPU's clocks and the other processes on it, as rocm-smi reports them
    (the timings assume an exclusive GPU); None for what the tool could not
    tell (an unprivileged user may not see the process list)."""
    return {"clocks": smi_clocks(_smi("--showclocks")),
            "other_processes": smi_other_processes(_smi("--showpids"), os.getpid())}


def mhz(text):
    """'(2100Mhz)' -> 2100.0, else None."""
    digits = "".join(c for c in str(text) if c.isdigit() or c == ".")
    try:
        return float(digits)
    except ValueError:
        return None


class ClockSampler:
    """Reads the shader and memory clocks with rocm-smi from a host thread,
    again and again, while a timed part runs: the clocks the work ran at."""

    def __init__(self, period_s=0.1):
        import threading
        self.period = period_s
        self.samples = {}
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            clocks = smi_clocks(_smi("--showclocks")) or {}
            for card in clocks.values():
                for name, val in card.items():
                    v = mhz(val)
                    if v is not None:
                        self.samples.setdefault(name, []).append(v)
            self.stop.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join(timeout=60)

    def summary(self):
        import statistics
        return {name + "_mhz": {"median": statistics.median(v), "min": min(v), "max": max(v), "samples": len(v)}
                for name, v in sorted(self.samples.items()) if v}


def cpu_sample(run_f, f0, f_max, budget_s):
    """Calls run_f(F) for F = f0, 2 f0, ... (at most f_max) until budget_s
    seconds are spent; returns (seconds, [F...])."""
    spent, sample, f = 0.0, [], f0
    while spent < budget_s and f <= f_max:
        t0 = time.perf_counter()
        run_f(f)
        spent += time.perf_counter() - t0
        sample.append(f)
        if f == f_max:
            break
        f = min(2 * f, f_max)
    return spent, sample


# ---------------------------------------------------------------------------- the stream (headline)


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


def stream_cpu_baseline(budget_s):
    """The CPU oracle on a bounded sample of the stream: for each matrix shape
    of layer 0, all 16 rows for the first F output features, F doubling until
    the budget is used; scaled to GB/s of algorithmic bytes."""
    import numpy as np
    import oracle
    import workloads as W
    mats = [W.stream_matrix(0, i) for i in range(len(SHAPES))]
    act = {k: W.stream_act(0, k) for k in {k for _, k in SHAPES}}
    done = {"bytes": 0, "rw": 0}

    def run(f):
        for mat in mats:
            m, k = mat["M"], mat["K"]
            fm = min(f, m)
            oracle.gemm_q4_0(mat["codes"], mat["scales"], act[k], oracle.BF16, 16, m, k,
                             cols=np.arange(fm, dtype=np.int64))
            done["bytes"] += fm * (k // 2 + (k // 32) * 2) + 16 * k * 2 + 16 * fm * 2
            done["rw"] += 16 * fm * k
    spent, sample = cpu_sample(run, 16, 17408, budget_s)
    hi = host_info()
    return dict(value=round(done["bytes"] / spent / 1e9, 4), unit="GB/s", cores=hi["threads_used"], kind="oracle",
                rows_weights_per_s=done["rw"] / spent, cpu_model=hi["cpu_model"],
                sample="layer 0 of the stack, 16 rows, output features 0..min(F, M)-1 of each of its 5 "
                       "matrices for F = %s; %.1f s of fp64 scalar C on %d threads" % (sample, spent,
                                                                                      hi["threads_used"]))


def stream_part(args, dev, stream):
    import torch
    import block_quantized_gemm_amd as vq
    layers = min(args.layers, 8) if args.profile_run else args.layers
    mats, acts, outs = build_stack(layers, dev)
    # one workspace for every call below: the larger of the two layouts' needs
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
        # the same passes over the stream's shapes in E4M3, in both layouts
        fmats, facts, fouts = build_fp8_stack(layers, dev, stream)
        for kind in ("fp8_panel", "fp8"):
            calls = fp8_layer_calls(vq, kind, fmats, facts, fouts, 16, ws)
            with torch.cuda.stream(stream):
                for _ in range(3):
                    for c in calls:
                        c(stream)
        torch.cuda.synchronize()
        del fmats, facts, fouts
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print("profile run done: %d layers" % layers, flush=True)
        return None

    n_launch = len(streams[16].layer_calls)
    t = {}
    rows = (16,) if args.headline_only else (16, 8, 1)
    for n in rows:
        t[n] = timed(streams[n].per_layer, stream, args.steps, args.warmup)
    forms = {"panel_grouped_per_layer_graph": t[16]}
    rm = {}
    if not args.headline_only:
        reps = max(8, args.steps // 2)
        forms["panel_grouped_whole_stack_graph"] = timed(streams[16].whole, stream, reps, args.warmup)
        forms["panel_per_call_graph"] = timed(streams[16].per_call, stream, reps, args.warmup)
        for n in (16, 1):
            rm[n] = timed(row_major[n].per_layer, stream, reps, args.warmup)
        forms["row_major_grouped_per_layer_graph"] = rm[16]
        forms["row_major_grouped_whole_stack_graph"] = timed(row_major[16].whole, stream, reps, args.warmup)
        forms["row_major_per_call_graph"] = timed(row_major[16].per_call, stream, reps, args.warmup)
        forms["row_major_per_call_eager"] = timed(row_major[16].per_call, stream, reps, args.warmup, graph=False)
    w_bytes, alg16 = algorithmic_bytes(mats, 16)
    alg = {n: algorithmic_bytes(mats, n)[1] for n in (16, 8, 1)}
    n_weights = sum(m * k for _, m, k, *_ in mats)
    mean16 = t[16]["mean_ms"]
    per_launch_us = mean16 * 1e3 / n_launch
    achieved = alg16 / n_launch / (per_launch_us * 1e-6) / 1e9
    traffic = stored_traffic("panel")
    res = {
        "layers": layers,
        "ms_per_step": mean16,
        "weight_bytes": w_bytes,
        "gbs_by_rows": {str(n): round(alg[n] / (t[n]["mean_ms"] * 1e-3) / 1e9, 2) for n in rows},
        "gbs_by_rows_stats": {str(n): rate(t[n], alg[n], 1e9) for n in rows},
        "ms_by_rows": {str(n): {k: round(v, 4) for k, v in t[n].items() if k.endswith("_ms")} for n in rows},
        "t16_over_t1": round(t[16]["mean_ms"] / t[1]["mean_ms"], 4) if 1 in t else None,
        "row_major_gbs_by_rows": {str(n): round(alg[n] / (v["mean_ms"] * 1e-3) / 1e9, 2) for n, v in rm.items()},
        "row_major_t16_over_t1": round(rm[16]["mean_ms"] / rm[1]["mean_ms"], 4) if rm else None,
        "rows_weights_per_s": 16 * n_weights / (mean16 * 1e-3),
        "launch_forms_gbs_16_rows": {k: round(alg16 / (v["mean_ms"] * 1e-3) / 1e9, 2) for k, v in forms.items()},
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
    del streams, row_major, mats, acts, outs, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- single-matrix configs


def _copies(t, nbytes_each):
    return [t] + [t.clone() for _ in range(max(1, -(-COPIES_BYTES // nbytes_each)) - 1)]


def tiny_part(args, dev, stream):
    """Q4_0 256 x 512, 8 fp16 rows, fp16 out: a latency figure (the whole
    problem fits in cache), the oracle timed in full."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    c = W.tiny()
    M, K, N = c["M"], c["K"], c["N"]
    codes = torch.from_numpy(c["codes"]).to(dev)
    scales = torch.from_numpy(c["scales"].view(np.int16).copy()).to(dev).view(torch.float16)
    x = torch.from_numpy(c["act"].view(np.int16).copy()).to(dev).view(torch.float16)
    out = torch.empty((N, M), dtype=torch.float16, device=dev)
    ws = vq.Workspace(vq.workspace_bytes("q4_0", M, K), dev)
    t = timed(lambda s: vq.gemm_q4_0(codes, scales, x, out, workspace=ws, stream=s), stream, args.reps, args.warmup,
              inner=64)
    res = {"workload": "Q4_0 %d x %d, %d fp16 rows, fp16 out (64 calls back to back per graph replay)" % (M, K, N),
           "us_per_call": {k: round(v * 1e3, 3) for k, v in t.items() if k.endswith("_ms")}}
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 0.5:
            oracle.gemm_q4_0(c["codes"], c["scales"], c["act"], oracle.F16, N, M, K)
            reps += 1
        res["cpu_baseline"] = {"us_per_call": round((time.perf_counter() - t0) / reps * 1e6, 1), "kind": "oracle",
                               "cores": host_info()["threads_used"], "sample": "the whole problem, %d calls" % reps}
    return res


def ffn_part(args, dev, stream):
    """Q4_0 17408 x 5120 at 1, 8 and 16 bf16 rows (Student-t rows with outlier
    channels), bf16 out: one call per matrix over > 2 GB of weight copies,
    graph-replayed; row-major arrays (the vq_gemm_q4_0 entry point) and panel
    layout."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    c = W.ffn(N=16)
    M, K = c["M"], c["K"]
    codes0 = torch.from_numpy(c["codes"]).to(dev)
    scales0 = torch.from_numpy(c["scales"].view(np.int16).copy()).to(dev).view(torch.float16)
    x = torch.from_numpy(c["act"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
    wbytes = M * K // 2 + M * (K // 32) * 2
    codes = _copies(codes0, wbytes)
    scales = [scales0] + [scales0.clone() for _ in range(len(codes) - 1)]
    panels = [vq.q4_0_to_panel(cd, sc) for cd, sc in zip(codes, scales)]
    ncopy = len(codes)
    ws = vq.Workspace(max(vq.workspace_bytes("q4_0", M, K), vq.workspace_bytes("q4_0_panel", M, K)), dev)
    res = {"workload": "Q4_0 %d x %d, bf16 rows (0.5 t(3), 5 channels x 50), bf16 out; one call per matrix over "
                       "%d copies (%.2f GB)" % (M, K, ncopy, ncopy * wbytes / 1e9),
           "row_major": {}, "panel": {}}
    times = {}
    for n in (1, 8, 16):
        xn = x[:n].contiguous()
        out = torch.empty((n, M), dtype=torch.bfloat16, device=dev)
        per_call = wbytes + n * K * 2 + n * M * 2

        def rm_step(s, xn=xn, out=out):
            for cd, sc in zip(codes, scales):
                vq.gemm_q4_0(cd, sc, xn, out, workspace=ws, stream=s)

        def pn_step(s, xn=xn, out=out):
            for p in panels:
                vq.gemm_q4_0_panel(p, M, K, xn, out, workspace=ws, stream=s)
        for lay, fn in (("row_major", rm_step), ("panel", pn_step)):
            t = timed(fn, stream, args.reps, args.warmup)
            times[(lay, n)] = t
            res[lay][str(n)] = {"gbs": rate(t, ncopy * per_call, 1e9),
                                "us_per_call": round(t["median_ms"] * 1e3 / ncopy, 3),
                                "rows_weights_per_s": n * M * K * ncopy / (t["median_ms"] * 1e-3)}
    for lay in ("row_major", "panel"):
        res[lay]["t16_over_t1"] = round(times[(lay, 16)]["median_ms"] / times[(lay, 1)]["median_ms"], 4)
        g16 = res[lay]["16"]["gbs"]["median"]
        res[lay]["roofline"] = {"bound": "hbm", "achieved": g16, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(g16 / HBM_PEAK_GBS, 4)}
    del codes, scales, panels
    if not args.no_cpu_baseline:
        import oracle
        done = {"bytes": 0, "rw": 0}

        def run(f):
            oracle.gemm_q4_0(c["codes"], c["scales"], c["act"], oracle.BF16, 16, M, K,
                             cols=np.arange(f, dtype=np.int64))
            done["bytes"] += f * (K // 2 + (K // 32) * 2) + 16 * K * 2 + 16 * f * 2
            done["rw"] += 16 * f * K
        spent, sample = cpu_sample(run, 16, M, args.cpu_seconds)
        res["cpu_baseline"] = {"value": round(done["bytes"] / spent / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                               "cores": host_info()["threads_used"], "rows_weights_per_s": done["rw"] / spent,
                               "sample": "16 rows, output features 0..F-1 for F = %s; %.1f s" % (sample, spent)}
    return res


def fp8_part(args, dev, stream):
    """FP8 block-scaled verify GEMM at 5120 x 5120 and 17408 x 5120, 1, 4 and
    16 bf16 rows, bf16 out: one call per matrix over > 2 GB of copies, on the
    row-major arrays (the vq_gemm_fp8_blk128 entry point) and, under "panel",
    in the FP8 panel layout."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    res = {}
    for m, k in ((5120, 5120), (17408, 5120)):
        f = W.fp8(M=m, K=k, N=16)
        w0 = torch.from_numpy(f["w"]).to(dev)
        s0 = torch.from_numpy(f["tscales"]).to(dev)
        x = torch.from_numpy(f["act"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
        ws = _copies(w0, m * k)
        pws = [vq.fp8_to_panel(w, stream=stream) for w in ws]
        torch.cuda.synchronize()
        wsp = vq.Workspace(max(vq.workspace_bytes("fp8", m, k), vq.workspace_bytes("fp8_panel", m, k)), dev)
        ent = {"copies": len(ws), "panel": {}}
        times = {}
        for n in (1, 4, 16):
            per_call = m * k + 4 * ((m + 127) // 128) * (k // 128) + n * k * 2 + n * m * 2
            xn = x[:n].contiguous()
            out = torch.empty((n, m), dtype=torch.bfloat16, device=dev)

            def step(s, xn=xn, out=out):
                for w in ws:
                    vq.gemm_fp8_blk128(w, s0, xn, out, workspace=wsp, stream=s)

            def pstep(s, xn=xn, out=out):
                for pw in pws:
                    vq.gemm_fp8_blk128_panel(pw, s0, xn, out, workspace=wsp, stream=s)
            for lay, fn, dst in (("row_major", step, ent), ("panel", pstep, ent["panel"])):
                t = timed(fn, stream, args.reps, args.warmup)
                times[(lay, n)] = t
                dst[str(n)] = {"gbs": rate(t, len(ws) * per_call, 1e9),
                               "us_per_call": round(t["median_ms"] * 1e3 / len(ws), 3)}
        for lay, dst in (("row_major", ent), ("panel", ent["panel"])):
            dst["t16_over_t1"] = round(times[(lay, 16)]["median_ms"] / times[(lay, 1)]["median_ms"], 4)
            g16 = dst["16"]["gbs"]["median"]
            dst["roofline"] = {"bound": "hbm", "achieved": g16, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(g16 / HBM_PEAK_GBS, 4)}
        if not args.no_cpu_baseline and m == 17408:
            import oracle
            done = {"bytes": 0}

            def run(fc, f=f, m=m, k=k):
                oracle.gemm_fp8_blk128(f["w"], f["tscales"], f["act"], oracle.BF16, 16, m, k,
                                       cols=np.arange(fc, dtype=np.int64))
                done["bytes"] += fc * k + 16 * k * 2 + 16 * fc * 2 + 4 * (-(-fc // 128)) * (k // 128)
            spent, sample = cpu_sample(run, 16, m, args.cpu_seconds)
            ent["cpu_baseline"] = {"value": round(done["bytes"] / spent / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                                   "cores": host_info()["threads_used"],
                                   "sample": "16 rows, output features 0..F-1 for F = %s; %.1f s" % (sample, spent)}
        res["%dx%d" % (m, k)] = ent
        del ws, pws
    return res


def prefill_part(args, dev, stream):
    """The prefill-sized W4A8 path: 512 bf16 rows x 5120 (Student-t with
    outlier channels) through the H32 int8 quantizer, then the W4A8 GEMM
    against Q4_0 17408 x 5120 rotated offline by the library; the 4-bit codes
    through the same GEMM; the FP8 block-scaled prefill GEMM at that shape."""
    import numpy as np
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    p = W.prefill()
    N, M, K = p["N"], p["M"], p["K"]
    codes0 = torch.from_numpy(p["codes"]).to(dev)
    scales0 = torch.from_numpy(p["scales"].view(np.int16).copy()).to(dev).view(torch.float16)
    x = torch.from_numpy(p["act"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
    q = torch.empty((N, K), dtype=torch.int8, device=dev)
    d = torch.empty((N, K // 32), dtype=torch.float16, device=dev)
    out = torch.empty((N, M), dtype=torch.float32, device=dev)
    codes = torch.empty_like(codes0)
    scales = torch.empty_like(scales0)
    t_rot = timed(lambda s: vq.q4_0_rotate_h32(codes0, scales0, codes, scales, stream=s), stream, 3, 1, graph=False)

    def quant(s):
        vq.hadamard32_quant_int8(x, q, d, stream=s)

    def gemm(s):
        vq.gemm_q4_0(codes, scales, q, out, x_scales=d, alpha=1.0 / 32, stream=s)

    def both(s):
        quant(s)
        gemm(s)
    t_q = timed(quant, stream, args.reps, args.warmup, inner=64)
    t_g = timed(gemm, stream, args.reps, args.warmup, inner=8)
    t_b = timed(both, stream, args.reps, args.warmup, inner=8)
    ops = 2.0 * N * M * K
    with torch.cuda.stream(stream):
        both(stream)
    ref = torch.empty((N, M), dtype=torch.float32, device=dev)
    vq.gemm_q4_0(codes0, scales0, x, ref, stream=stream)
    torch.cuda.synchronize()
    rel = float(torch.linalg.norm((out - ref).double()) / torch.linalg.norm(ref.double()))
    q4 = torch.empty_like(q)
    d4 = torch.empty_like(d)
    out4 = torch.empty_like(out)

    def quant4(s):
        vq.hadamard32_quant_int4(x, q4, d4, stream=s)

    def gemm4(s):
        vq.gemm_q4_0(codes, scales, q4, out4, x_scales=d4, alpha=1.0 / 32, stream=s)
    t_q4 = timed(quant4, stream, args.reps, args.warmup, inner=64)
    t_g4 = timed(gemm4, stream, args.reps, args.warmup, inner=8)
    with torch.cuda.stream(stream):
        quant4(stream)
        gemm4(stream)
    torch.cuda.synchronize()
    rel4 = float(torch.linalg.norm((out4 - ref).double()) / torch.linalg.norm(ref.double()))
    tops = rate(t_g, ops, 1e12)
    quant_bytes = N * K * 2 + N * K + N * (K // 32) * 2
    res = {
        "workload": "W4A8 prefill: %d bf16 rows x K=%d, H32 int8 quantizer, then Q4_0 %d x %d (H32-rotated "
                    "offline) W4A8 GEMM (exact integer block dots), fp32 out" % (N, K, M, K),
        "gemm_us": {k: round(v * 1e3, 2) for k, v in t_g.items() if k.endswith("_ms")},
        "quantizer_us": {k: round(v * 1e3, 2) for k, v in t_q.items() if k.endswith("_ms")},
        "quantizer_gbs": rate(t_q, quant_bytes, 1e9),
        "quantizer_plus_gemm_us": round(t_b["median_ms"] * 1e3, 2),
        "offline_rotation_us": round(t_rot["median_ms"] * 1e3, 2),
        "tops": tops,
        "rel_error_vs_bf16_rows": round(rel, 4),
        "roofline": {"bound": "mfma", "achieved": tops["median"], "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(tops["median"] / INT8_MFMA_PEAK_TOPS, 4), "ops_per_launch": ops},
        "w4a4": {"workload": "4-bit activation codes (H32, bound 7) of the same rows, the same GEMM",
                 "quantizer_us": round(t_q4["median_ms"] * 1e3, 2), "gemm_us": round(t_g4["median_ms"] * 1e3, 2),
                 "tops": rate(t_g4, ops, 1e12), "rel_error_vs_bf16_rows": round(rel4, 4)},
    }
    # FP8 block-scaled prefill GEMM at the same shape (the FP8 workload's distributions)
    f = W.fp8(M=M, K=K, N=16)
    w8 = torch.from_numpy(f["w"]).to(dev)
    ts = torch.from_numpy(f["tscales"]).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    x8 = torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16)
    o8 = torch.empty((N, M), dtype=torch.bfloat16, device=dev)
    t_p = timed(lambda s: vq.gemm_fp8_blk128_prefill(w8, ts, x8, o8, stream=s), stream, args.reps, args.warmup,
                inner=8)
    tf = rate(t_p, ops, 1e12)
    res["fp8_prefill"] = {
        "workload": "FP8 block-scaled prefill: %d bf16 rows x %d x %d, bf16 out" % (N, M, K),
        "gemm_us": {k: round(v * 1e3, 2) for k, v in t_p.items() if k.endswith("_ms")}, "tflops": tf,
        "roofline": {"bound": "mfma", "achieved": tf["median"], "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf["median"] / BF16_MFMA_PEAK_TFLOPS, 4), "flops_per_launch": ops}}
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        qo, do, _ = oracle.h32_quant_int8(p["act"], oracle.BF16, N, K)
        t_cq = time.perf_counter() - t0
        co, so = oracle.q4_0_rotate_h32(p["codes"], p["scales"], M, K)
        done = {"ops": 0}

        def run(fc):
            oracle.gemm_w4a8(co, so, qo, do, N, M, K, cols=np.arange(fc, dtype=np.int64), alpha=1.0 / 32)
            done["ops"] += 2 * N * fc * K
        spent, sample = cpu_sample(run, 4, M, args.cpu_seconds)
        res["cpu_baseline"] = {"value": round(done["ops"] / spent / 1e12, 6), "unit": "TOPS", "kind": "oracle",
                               "cores": host_info()["threads_used"],
                               "quantizer_ms": round(t_cq * 1e3, 2),
                               "sample": "the quantizer over all %d rows; the W4A8 GEMM on output features "
                                         "0..F-1 for F = %s (%.1f s)" % (N, sample, spent)}
    return res


def build_fp8_stack(layers, dev, stream):
    """The stream's shapes in E4M3 with 128 x 128 fp32 tile scales (E4M3 of
    N(0,1), scales U[1e-3, 1e-2], drawn on the device), each matrix also in
    the FP8 panel layout: (layer, M, K, codes, tile scales, panel) per
    matrix, 16-row activations per (layer, K) and outputs per M."""
    import torch
    import block_quantized_gemm_amd as vq
    import workloads as W
    mats = []
    for layer in range(layers):
        for idx, (m, k) in enumerate(SHAPES):
            g = torch.Generator(device=dev)
            g.manual_seed(W.seed_of(W.CFG_FP8, layer, 10 * idx))
            w = torch.randn((m, k), generator=g, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
            ts = torch.empty(((m + 127) // 128, k // 128), dtype=torch.float32, device=dev).uniform_(1e-3, 1e-2,
                                                                                                      generator=g)
            mats.append((layer, m, k, w, ts, vq.fp8_to_panel(w, stream=stream)))
    acts = {(l, k): W.act_device(16, k, W.seed_of(W.CFG_FP8, l, 1000 + k), dev)
            for l in range(layers) for k in sorted({k for _, k in SHAPES})}
    outs = {m: torch.empty((16, m), dtype=torch.bfloat16, device=dev) for m in {m for m, _ in SHAPES}}
    torch.cuda.synchronize()
    return mats, acts, outs


def fp8_layer_calls(vq, kind, mats, acts, outs, n, ws):
    """One grouped call per layer over its five matrices at n rows, in the
    FP8 panel layout (kind "fp8_panel") or on the row-major arrays ("fp8")."""
    layers = sorted({l for l, *_ in mats})
    calls = []
    for L in layers:
        probs = [(pw if kind == "fp8_panel" else w, ts, acts[(l, k)][:n], outs[m][:n])
                 for l, m, k, w, ts, pw in mats if l == L]
        calls.append(vq.GroupedCall(kind, probs, workspace=ws))
    return calls


def fp8_stream_part(args, dev, stream):
    """The per-token stream's shapes in FP8 E4M3 with 128 x 128 fp32 tile
    scales (E4M3 of N(0,1), scales U[1e-3, 1e-2], drawn on the device): 64
    layers x 5 matrices, 16 bf16 rows per layer, each layer's five GEMMs one
    grouped call, the step's launches replayed as one HIP graph; also at 1 row
    and as whole-stack grouped calls.  The codes in the FP8 panel layout
    (repacked once, before timing) lead; the row-major arrays are timed
    beside them."""
    import torch
    import block_quantized_gemm_amd as vq
    layers = args.layers
    mats, acts, outs = build_fp8_stack(layers, dev, stream)
    wbytes = sum(m * k + 4 * ((m + 127) // 128) * (k // 128) for _, m, k, _, _, _ in mats)
    res = {"workload": "FP8 E4M3 per-token stream: %d layers x (8192x5120, 5120x8192, 17408x5120 x2, 5120x17408), "
                       "128 x 128 fp32 tile scales, 16-row bf16 block per layer; each layer's 5 GEMMs one grouped "
                       "call, the step's launches one HIP graph; codes in the FP8 panel layout" % layers,
           "weight_bytes": wbytes}
    ws = None
    for kind in ("fp8_panel", "fp8"):
        ent = res if kind == "fp8_panel" else res.setdefault("row_major", {})
        times = {}
        for n in (16, 1):
            def problems(sel):
                return [(pw if kind == "fp8_panel" else w, ts, acts[(l, k)][:n], outs[m][:n])
                        for l, m, k, w, ts, pw in mats if sel(l)]
            calls = [vq.GroupedCall(kind, problems(lambda l, L=L: l == L), workspace=ws if ws else "auto")
                     for L in range(layers)]
            big = max((c.ws for c in calls if c.ws is not None), key=lambda w: w.nbytes, default=None)
            if big is not None and (ws is None or big.nbytes > ws.nbytes):
                ws = big
            for c in calls:
                c.ws = ws
            t = timed(lambda st: [c(st) for c in calls], stream, max(8, args.steps // 2), args.warmup)
            alg = wbytes + sum(n * k * 2 + n * m * 2 for _, m, k, _, _, _ in mats)
            times[n] = t
            ent["gbs_%d_rows" % n] = rate(t, alg, 1e9)
            if n == 16:
                whole = [vq.GroupedCall(kind, problems(lambda l, L=L: L <= l < L + 6), workspace=ws)
                         for L in range(0, layers, 6)]
                for c in whole:
                    if c.ws is not ws and c.ws is not None:
                        ws = c.ws
                tw = timed(lambda st: [c(st) for c in whole], stream, max(8, args.steps // 2), args.warmup)
                ent["gbs_16_rows_whole_stack"] = rate(tw, alg, 1e9)
                if kind == "fp8_panel":
                    res["roofline"] = {"bound": "hbm", "achieved": res["gbs_16_rows"]["median"],
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(res["gbs_16_rows"]["median"] / HBM_PEAK_GBS, 4),
                                       "traffic": stored_traffic("fp8_panel"),
                                       "algorithmic_bytes_per_launch": alg // layers}
        ent["t16_over_t1"] = round(times[16]["median_ms"] / times[1]["median_ms"], 4)
    del mats, acts, outs
    torch.cuda.empty_cache()
    return res


GREEDY_VOCAB = 151936  # a synthetic vocabulary of 151,936 entries


def greedy_part(args, dev, stream):
    """Greedy verification of a 16-row block over bf16 logits [16][V]: time per
    call, one call per copy graph-replayed over enough copies of the logits
    that a step reads them from HBM; bytes = the logits read once."""
    import torch
    import block_quantized_gemm_amd as vq
    n, v = 16, GREEDY_VOCAB
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    lg0 = torch.randn((n, v), generator=g, device=dev).to(torch.bfloat16)
    lgs = _copies(lg0, n * v * 2)
    lgs = lgs[:max(1, len(lgs) // 4)]  # > 500 MB
    draft = torch.zeros(n - 1, dtype=torch.int32, device=dev)
    tokens = torch.empty(n, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    ws = vq.Workspace(vq.greedy_workspace_bytes(n, v), dev)

    def step(s):
        for lg in lgs:
            vq.greedy_verify(lg, draft, tokens, count, workspace=ws, stream=s)
    t = timed(step, stream, args.reps, args.warmup)
    us = t["median_ms"] * 1e3 / len(lgs)
    gbs = n * v * 2 / (us * 1e-6) / 1e9
    return {"rows": n, "vocab": v, "logits_dtype": "bf16", "us_per_call": round(us, 2), "gbs": round(gbs, 2),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def probe_part(args, dev, stream):
    """The library's HBM read probe over 2 GiB: one workgroup per 64 KiB, and
    one persistent workgroup per CU in contiguous shares and as a sweeping
    window, with the default and the non-temporal cache policy; then the
    rate of L2 hits (each workgroup re-reading its 64 KiB) and the LDS read
    rate per CU, kept out of best_gbs."""
    import torch
    import block_quantized_gemm_amd as vq
    nbytes = 1 << 31
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {"bytes": nbytes}
    for name, mode, groups, waves, depth, nt in (("blocks_w8_d8", "blocks", 0, 8, 8, False),
                                                 ("blocks_w8_d8_nt", "blocks", 0, 8, 8, True),
                                                 ("shares_%d_w8_d8" % cus, "shares", cus, 8, 8, False),
                                                 ("shares_%d_w8_d8_nt" % cus, "shares", cus, 8, 8, True),
                                                 ("window_%d_w8_d8_nt" % cus, "window", cus, 8, 8, True)):
        t = timed(lambda s: vq.hbm_read_probe(buf, sink, mode=mode, groups=groups, waves_per_group=waves,
                                              depth=depth, nontemporal=nt, stream=s), stream, args.reps, args.warmup,
                  inner=4)
        res[name] = rate(t, nbytes, 1e9)
    res["best_gbs"] = max(v["median"] for k, v in res.items() if isinstance(v, dict))
    # the rate of L2 hits: 64 KiB per workgroup (2 MiB per XCD), read 16 times over in one launch
    small = buf[: cus * (64 << 10)]
    t = timed(lambda s: vq.hbm_read_probe(small, sink, mode="reread", groups=cus, waves_per_group=8, depth=8,
                                          stream=s), stream, args.reps, args.warmup, inner=32)
    res["reread_l2_%d_w8_d8" % cus] = rate(t, small.numel() * vq.PROBE_REREAD_PASSES, 1e9)
    res["reread_l2_gbs_per_cu"] = round(res["reread_l2_%d_w8_d8" % cus]["median"] / cus, 1)
    # the LDS read rate: every workgroup reads 32 MiB from its 64 KiB of LDS
    lds_bytes = 32 << 20
    t = timed(lambda s: vq.hbm_read_probe(buf[:lds_bytes], sink, mode="lds", groups=cus, waves_per_group=8,
                                          depth=8, stream=s), stream, args.reps, args.warmup, inner=4)
    res["lds_read_%d_w8_d8" % cus] = rate(t, cus * lds_bytes, 1e9)
    res["lds_read_gbs_per_cu"] = round(res["lds_read_%d_w8_d8" % cus]["median"] / cus, 1)
    del buf
    return res


# ---------------------------------------------------------------------------- traffic counters


def _layout_of(kernel_name):
    """The format and weight layout a walk-kernel dispatch ran on ("panel",
    "row_major", "fp8_panel", "fp8_row_major"), or None for other kernels.
    The template arguments are the activation type, the FP8 flag, tiles,
    waves, steps ahead and the panel flag."""
    if "vq::walk_kernel<" not in kernel_name:
        return None
    targs = [a.strip() for a in kernel_name.split("vq::walk_kernel<", 1)[1].split(">")[0].split(",")]
    if len(targs) != 6:
        return None
    lay = "panel" if targs[5] == "true" else "row_major"
    return "fp8_" + lay if targs[1] == "true" else lay


def stored_traffic(layout):
    """Measured HBM bytes per grouped-layer launch of a layout from the stored
    counter figure, or None when it is missing or was taken on other kernel
    sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("kernel_source_hash") != kernel_source_hash():
        return None
    return tr.get(layout, {}).get("hbm_bytes_per_launch")


def traffic_from(fetch_dir, write_dir, out_path=TRAFFIC_FILE):
    """Per-launch HBM bytes of the verify kernels, per format and layout, from two
    counter runs of --profile-run, each scaled by what the same counter reads
    for the plain copy of COPY_BYTES in that run."""
    def per_kernel(d, counter):
        vals = {"panel": [], "row_major": [], "fp8_panel": [], "fp8_row_major": [], "copy": []}
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
        avg = {k: sum(v) / len(v) for k, v in vals.items() if k != "copy" and v}
        return avg, sum(cal) / len(cal)
    fv, fc = per_kernel(fetch_dir, "FETCH_SIZE")
    wv, wc = per_kernel(write_dir, "WRITE_SIZE")
    fetch_scale, write_scale = COPY_BYTES / (fc * 1024), COPY_BYTES / (wc * 1024)
    rec = {
        "kernel_source_hash": kernel_source_hash(),
        "workload": "grouped per-layer launch, 5 stream matrices, 16 bf16 rows (Q4_0, and E4M3 with 128 x 128 "
                    "tile scales)",
        "copy_fetch_kib": fc, "copy_write_kib": wc,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
    }
    for lay in ("panel", "row_major", "fp8_panel", "fp8_row_major"):
        if lay not in fv or lay not in wv:
            continue
        rec[lay] = {
            "hbm_bytes_per_launch": round(fv[lay] * 1024 * fetch_scale + wv[lay] * 1024 * write_scale),
            "read_bytes_per_launch": round(fv[lay] * 1024 * fetch_scale),
            "write_bytes_per_launch": round(wv[lay] * 1024 * write_scale),
            "fetch_kib_raw": fv[lay], "write_kib_raw": wv[lay],
        }
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return rec


# ---------------------------------------------------------------------------- main


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus %d is not supported: the verify GEMM "
                                   "would shard along M across GPUs (each its own M/P rows, bit-identical "
                                   "outputs), which is not built here" % args.gpus}))
        sys.exit(2)
    import torch
    import block_quantized_gemm_amd as vq
    vq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    parts = {"tiny": tiny_part, "ffn": ffn_part, "fp8": fp8_part, "fp8stream": fp8_stream_part,
             "prefill": prefill_part, "greedy": greedy_part, "probe": probe_part}
    if args.only and args.only != "stream":
        print(json.dumps({args.only: parts[args.only](args, dev, stream)}))
        return
    if args.profile_run:
        stream_part(args, dev, stream)
        return
    state_before = gpu_state()
    with ClockSampler() as clocks:
        head = stream_part(args, dev, stream)
    if args.only == "stream" or args.headline_only:
        head["clocks_during_timing"] = clocks.summary()
        print(json.dumps(head))
        return
    print("stream timed: %.1f GB/s" % head["gbs_by_rows"]["16"], file=sys.stderr, flush=True)
    configs = {}
    for name in ("tiny", "ffn", "fp8", "fp8stream", "prefill", "greedy", "probe"):
        configs[name] = parts[name](args, dev, stream)
        print("%s timed" % name, file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    probe = configs.pop("probe")
    greedy = configs.pop("greedy")
    g16 = head["gbs_by_rows"]["16"]
    result = {
        "metric": METRIC,
        "value": g16,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded draws: Q4_0 codes uniform, fp16 scales U[0.001,0.02] or lognormal(-5,0.5), "
                "bf16 rows N(0,1) or 0.5 t(3) with outlier channels, E4M3 of N(0,1))",
        "config": {
            "workload": "Q4_0 per-token weight stream: %d layers x (8192x5120, 5120x8192, 17408x5120 x2, "
                        "5120x17408), 16-row bf16 draft block per layer; weights in the library's panel "
                        "layout (same bytes as row-major Q4_0); each layer's 5 GEMMs one grouped call, the "
                        "step's %d launches replayed as one HIP graph" % (head["layers"],
                                                                           head["roofline"]["launches_per_step"]),
            "weight_bytes": head["weight_bytes"],
            "n_rows": 16,
        },
        "pct_of_hbm_peak": round(100 * g16 / HBM_PEAK_GBS, 2),
        "pct_of_probed_hbm": round(100 * g16 / probe["best_gbs"], 2),
    }
    for k in ("gbs_by_rows", "gbs_by_rows_stats", "ms_by_rows", "t16_over_t1", "row_major_gbs_by_rows",
              "row_major_t16_over_t1", "rows_weights_per_s", "launch_forms_gbs_16_rows"):
        result[k] = head[k]
    result["configs"] = configs
    result["greedy_verify"] = greedy
    result["hbm_probe"] = probe
    result["host"] = host_info()
    result["gpu"] = torch.cuda.get_device_properties(dev).name
    result["gpu_state"] = {"before": state_before, "after": gpu_state(),
                           "clocks_during_stream_timing": clocks.summary()}
    result["roofline"] = head["roofline"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = stream_cpu_baseline(args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
