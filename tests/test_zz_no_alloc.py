"""The allocation-free entry point (vq_gemm_q4_0_noalloc) through the C ABI:
the same bits as vq_gemm_q4_0 with a workspace, within the parity bar of the
CPU oracle, on two calls in a row (the second with a smaller input, which
finds the scratch array holding the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(codes, scales, x, out, x_scales=None, alpha=1.0):
    """One call of the C entry point, on torch's current stream."""
    N, K = x.shape
    M = codes.shape[0]
    st = vq.lib().vq_gemm_q4_0_noalloc(
        codes.data_ptr(), scales.data_ptr(), x.data_ptr(), vq._dtype_code(x),
        None if x_scales is None else x_scales.data_ptr(), out.data_ptr(), vq._dtype_code(out),
        N, M, K, ctypes.c_float(alpha), torch.cuda.current_stream().cuda_stream)
    assert st == vq.VQ_OK, vq.status_string(st)


def _case(M, K, N, seed, act="bf16", out_dt=torch.bfloat16):
    g = np.random.Generator(np.random.PCG64(seed))
    codes = W.q4_0_codes(M, K, g)
    scales = W.fp16_scales_lognormal(M, K, g)
    x = 0.5 * g.standard_t(3, size=(N, K))
    bits = W.f32_to_bf16_bits(x) if act == "bf16" else W.f32_to_f16_bits(x)
    return codes, scales, bits


@pytest.mark.parametrize("order", ["large_then_small", "ragged_then_rows"])
def test_noalloc_matches_workspace_call_two_calls_in_a_row(order):
    cases = {"large_then_small": [(17408, 5120, 16, 11), (1000, 2048, 5, 12)],
             "ragged_then_rows": [(5120, 8192, 13, 13), (272, 1024, 40, 14)]}[order]
    ws = vq.Workspace(32 << 20)
    for M, K, N, seed in cases:
        codes_np, scales_np, bits = _case(M, K, N, seed)
        codes, scales = to_dev(codes_np), to_dev(scales_np, torch.float16)
        x = to_dev(bits, torch.bfloat16)
        y_na = torch.full((N, M), float("nan"), dtype=torch.bfloat16, device="cuda")
        y_ws = torch.empty((N, M), dtype=torch.bfloat16, device="cuda")
        _noalloc(codes, scales, x, y_na)
        vq.gemm_q4_0(codes, scales, x, y_ws, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits_u16(y_na), bits_u16(y_ws)), (M, K, N)
        cols = np.unique(np.concatenate([[0, M - 1], np.random.Generator(np.random.PCG64(seed)).choice(M, 256)]))
        ref = oracle.gemm_q4_0(codes_np, scales_np, bits, oracle.BF16, N, M, K, cols=cols)
        parity(out_to_f64(y_na)[:, cols], ref, "bf16")


def test_noalloc_one_shot_shape_and_int8_rows():
    """K % 256 != 0 runs one-shot (no scratch); int8 rows take the W4A8
    kernel (no scratch): both still match the workspace entry point."""
    codes_np, scales_np, bits = _case(300, 96, 7, 21)
    codes, scales = to_dev(codes_np), to_dev(scales_np, torch.float16)
    x = to_dev(bits, torch.bfloat16)
    y_na = torch.empty((7, 300), dtype=torch.float32, device="cuda")
    y_ws = torch.empty_like(y_na)
    _noalloc(codes, scales, x, y_na)
    vq.gemm_q4_0(codes, scales, x, y_ws)
    g = np.random.Generator(np.random.PCG64(22))
    qx = torch.from_numpy(g.integers(-127, 128, size=(7, 96)).astype(np.int8)).cuda()
    dx = to_dev(W.f32_to_f16_bits(g.uniform(0.01, 0.1, size=(7, 3))), torch.float16)
    z_na = torch.empty((7, 300), dtype=torch.float32, device="cuda")
    z_ws = torch.empty_like(z_na)
    _noalloc(codes, scales, qx, z_na, x_scales=dx, alpha=0.5)
    vq.gemm_q4_0(codes, scales, qx, z_ws, x_scales=dx, alpha=0.5)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws) and torch.equal(z_na, z_ws)
    parity(out_to_f64(y_na), oracle.gemm_q4_0(codes_np, scales_np, bits, oracle.BF16, 7, 300, 96), "f32")


def test_noalloc_on_a_side_stream_and_through_the_binding():
    codes_np, scales_np, bits = _case(4100, 5120, 16, 31)
    codes, scales = to_dev(codes_np), to_dev(scales_np, torch.float16)
    x = to_dev(bits, torch.bfloat16)
    y_ws = torch.empty((16, 4100), dtype=torch.bfloat16, device="cuda")
    vq.gemm_q4_0(codes, scales, x, y_ws, workspace=vq.Workspace(32 << 20))
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        y = torch.empty_like(y_ws)
        vq.gemm_q4_0_noalloc(codes, scales, x, y, stream=s)
        outs.append(y)
    s.synchronize()
    for y in outs:
        assert torch.equal(y, y_ws)
