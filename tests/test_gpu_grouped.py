"""Grouped verify GEMMs on the GPU: every problem's output matches the CPU
oracle, is bit-identical for any number of rows, and (in the one-shot form)
bit-identical to its single call."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import accumulation_slack, bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu


def _q4_problem(M, K, N, g, act_dtype=torch.bfloat16, out_dtype=torch.bfloat16):
    codes = W.q4_0_codes(M, K, g)
    scales = W.fp16_scales_lognormal(M, K, g)
    x = 0.5 * g.standard_t(3, size=(N, K))
    bits = W.f32_to_bf16_bits(x) if act_dtype == torch.bfloat16 else W.f32_to_f16_bits(x)
    dev = (to_dev(codes), to_dev(scales, torch.float16), to_dev(bits, act_dtype),
           torch.empty((N, M), dtype=out_dtype, device="cuda"))
    return dict(codes=codes, scales=scales, bits=bits, dev=dev, M=M, K=K, N=N)


def _single(p, workspace):
    out = torch.empty_like(p["dev"][3])
    vq.gemm_q4_0(p["dev"][0], p["dev"][1], p["dev"][2], out, workspace=workspace)
    return out


def _rows(p, r0, r1):
    """Device operands of rows [r0, r1) of a problem, with a fresh output."""
    x = p["dev"][2][r0:r1].contiguous()
    return (p["dev"][0], p["dev"][1], x, torch.empty((r1 - r0, p["M"]), dtype=p["dev"][3].dtype, device="cuda"))


def test_grouped_layer_parity_and_width_invariance():
    """One synthetic layer (the five stream shapes, 16 rows) in one grouped
    call: sampled outputs against the oracle, and each row bit-identical to
    the same grouped call made with that row alone (or 8 rows)."""
    g = np.random.Generator(np.random.PCG64(301))
    probs = [_q4_problem(M, K, 16, g) for M, K in W.STREAM_LAYER_SHAPES]
    ws = vq.Workspace(64 << 20)
    call = vq.GroupedCall("q4_0", [p["dev"] for p in probs], workspace=ws)
    call()
    torch.cuda.synchronize()
    for p in probs:
        cols = np.unique(np.concatenate([[0, p["M"] - 1], g.choice(p["M"], 96, replace=False)]))
        y = out_to_f64(p["dev"][3])[:, cols]
        parity(y, oracle.gemm_q4_0(p["codes"], p["scales"], p["bits"], oracle.BF16, 16, p["M"], p["K"],
                                   cols=cols), "bf16")
    for r0, r1 in ((5, 6), (0, 1), (8, 16)):
        sub = [_rows(p, r0, r1) for p in probs]
        vq.GroupedCall("q4_0", sub, workspace=ws)()
        torch.cuda.synchronize()
        for p, d in zip(probs, sub):
            assert torch.equal(d[3], p["dev"][3][r0:r1]), (r0, p["M"], p["K"])


def test_grouped_many_mixed_problems():
    """More problems than one launch holds, with small-M problems whose launch
    shape differs and K that runs streamed (K % 256 == 0) or one-shot mixed:
    the library splits them over several launches."""
    g = np.random.Generator(np.random.PCG64(302))
    shapes = [(int(g.integers(1, 400)), 32 * int(g.integers(1, 80)) if i % 3 else 256 * int(g.integers(1, 12)))
              for i in range(45)]
    probs = [_q4_problem(M, K, 5, g, torch.float16, torch.float32) for M, K in shapes]
    ws = vq.Workspace(64 << 20)
    vq.gemm_q4_0_grouped([p["dev"] for p in probs], workspace=ws, alpha=0.5)
    torch.cuda.synchronize()
    for i, p in enumerate(probs):
        out = torch.empty_like(p["dev"][3])
        vq.gemm_q4_0(p["dev"][0], p["dev"][1], p["dev"][2], out, workspace=ws, alpha=0.5)
        torch.cuda.synchronize()
        ref = oracle.gemm_q4_0(p["codes"], p["scales"], p["bits"], oracle.F16, 5, p["M"], p["K"], alpha=0.5)
        x = oracle.f16_to_f64(p["bits"])
        w = oracle.q4_0_dequant(p["codes"], p["scales"], p["M"], p["K"])
        slack = 0.5 * accumulation_slack(x, w)
        parity(out_to_f64(p["dev"][3]), ref, "f32", slack=slack)   # grouped
        parity(out_to_f64(out), ref, "f32", slack=slack)           # single


def test_grouped_without_workspace_matches_unsplit_single_calls():
    g = np.random.Generator(np.random.PCG64(303))
    probs = [_q4_problem(M, K, 16, g) for M, K in ((1000, 5120), (300, 2080), (64, 256))]
    vq.gemm_q4_0_grouped([p["dev"] for p in probs], workspace=None)
    torch.cuda.synchronize()
    for p in probs:
        assert torch.equal(p["dev"][3], _single(p, None))


def test_grouped_more_than_16_rows():
    g = np.random.Generator(np.random.PCG64(304))
    probs = [_q4_problem(M, K, 37, g) for M, K in ((520, 4096), (130, 1056))]
    ws = vq.Workspace(16 << 20)
    vq.gemm_q4_0_grouped([p["dev"] for p in probs], workspace=ws)
    torch.cuda.synchronize()
    for p in probs:
        parity(out_to_f64(p["dev"][3]), oracle.gemm_q4_0(p["codes"], p["scales"], p["bits"], oracle.BF16, 37,
                                                         p["M"], p["K"]), "bf16")
    # rows 16..31 are the second group of 16: the same as a 16-row call on them
    sub = [_rows(p, 16, 32) for p in probs]
    vq.gemm_q4_0_grouped(sub, workspace=ws)
    torch.cuda.synchronize()
    for p, d in zip(probs, sub):
        assert torch.equal(d[3], p["dev"][3][16:32])


def test_grouped_fp8():
    g = np.random.Generator(np.random.PCG64(305))
    probs = []
    for M, K in ((5120, 5120), (300, 1280), (17408, 1024)):
        f = W.fp8(M=M, K=K, N=4)
        dev = (to_dev(f["w"]), to_dev(f["tscales"]), to_dev(f["act"], torch.bfloat16),
               torch.empty((4, M), dtype=torch.bfloat16, device="cuda"))
        probs.append((f, dev))
    ws = vq.Workspace(32 << 20)
    vq.gemm_fp8_blk128_grouped([d for _, d in probs], workspace=ws)
    torch.cuda.synchronize()
    for f, d in probs:
        M, K = f["w"].shape
        cols = np.unique(np.concatenate([[0, 127, 128, M - 1], g.choice(M, 64, replace=False)]))
        parity(out_to_f64(d[3])[:, cols], oracle.gemm_fp8_blk128(f["w"], f["tscales"], f["act"], oracle.BF16, 4,
                                                                M, K, cols=cols), "bf16")


def test_grouped_too_small_workspace_rejected():
    g = np.random.Generator(np.random.PCG64(306))
    p = _q4_problem(1024, 5120, 4, g)
    call = vq.GroupedCall("q4_0", [p["dev"]], workspace=None)
    small = vq.Workspace(1024)
    with pytest.raises(vq.VqError) as e:
        vq.lib()  # keep the binding loaded
        st = vq.lib().vq_gemm_q4_0_grouped(call.table, 1, call.act_dtype, call.out_dtype, 4, 1.0, small.ptr(),
                                           small.nbytes, None)
        if st != vq.VQ_OK:
            raise vq.VqError(st, "vq_gemm_q4_0_grouped")
    assert e.value.status == vq.VQ_ERR_WORKSPACE


def test_grouped_graph_replays_match_eager():
    """The grouped call captured in a HIP graph: every replay (with eager work
    on the same workspace and synchronisation between replays) equals the
    eager result."""
    g = np.random.Generator(np.random.PCG64(307))
    probs = [_q4_problem(M, K, 16, g) for M, K in ((2048, 5120), (1024, 8192), (512, 17408))]
    ws = vq.Workspace(64 << 20)
    call = vq.GroupedCall("q4_0", [p["dev"] for p in probs], workspace=ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    eager = [p["dev"][3].clone() for p in probs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call(s)
    for rep in range(4):
        for p in probs:
            p["dev"][3].fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        for i, p in enumerate(probs):
            assert torch.equal(p["dev"][3], eager[i]), (rep, i)
        _single(probs[0], ws)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
