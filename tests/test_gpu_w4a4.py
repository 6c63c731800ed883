"""The 4-bit activation path (W4A4 numerics) on the GPU, through the C ABI:
the H32 4-bit quantizer bit for bit against the CPU oracle, and the W4A8 GEMM
on its codes against the oracle GEMM."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu


def gpu_quant4(x_bits, x_dtype="bf16"):
    N, K = x_bits.shape
    x = to_dev(x_bits, torch.bfloat16 if x_dtype == "bf16" else torch.float16)
    q = torch.empty((N, K), dtype=torch.int8, device="cuda")
    d = torch.empty((N, K // 32), dtype=torch.float16, device="cuda")
    vq.hadamard32_quant_int4(x, q, d)
    torch.cuda.synchronize()
    return q.cpu().numpy(), bits_u16(d)


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_quantizer4_bit_exact_prefill_rows(x_dtype):
    p = W.prefill()
    x = p["act"]
    if x_dtype == "f16":
        x = W.f32_to_f16_bits(torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float().numpy())
    q, d = gpu_quant4(x, x_dtype)
    qo, do, st = oracle.h32_quant_int4(x, oracle.BF16 if x_dtype == "bf16" else oracle.F16, *x.shape)
    assert st == 0
    assert np.array_equal(d, do)
    assert np.array_equal(q, qo)
    assert np.abs(q).max() == 7


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (7, 4128)])
def test_quantizer4_bit_exact_ragged(N, K):
    g = np.random.Generator(np.random.PCG64(7 * N * K))
    x = W.f32_to_bf16_bits(g.standard_normal((N, K)) * np.exp(g.uniform(-8, 8, size=(N, 1))))
    x[0, :32] = 0                      # a zero block
    q, d = gpu_quant4(x)
    qo, do, _ = oracle.h32_quant_int4(x, oracle.BF16, N, K)
    assert np.array_equal(d, do) and np.array_equal(q, qo)
    assert np.all(q[0, :32] == 0) and d[0, 0] == 0


def test_w4a4_prefill_parity_sampled():
    """512 rows x 17408 x 5120: the GPU 4-bit quantizer, then the GEMM on its
    codes (alpha = 1/32), against the oracle GEMM on the same codes."""
    p = W.prefill()
    q, d = gpu_quant4(p["act"])
    M, K, N = p["M"], p["K"], p["N"]
    codes = to_dev(p["codes"])
    scales = to_dev(p["scales"], torch.float16)
    out = torch.empty((N, M), dtype=torch.float32, device="cuda")
    vq.gemm_q4_0(codes, scales, to_dev(q), out, x_scales=to_dev(d, torch.float16), alpha=1.0 / 32)
    torch.cuda.synchronize()
    y = out_to_f64(out)
    g = np.random.Generator(np.random.PCG64(404))
    cols = np.unique(np.concatenate([[0, 287, 288, M - 1], g.choice(M, 160, replace=False)]))
    ref = oracle.gemm_w4a8(p["codes"], p["scales"], q, d, N, M, K, cols=cols, alpha=1.0 / 32)
    fro, worst, ulps = parity(y[:, cols], ref, "f32")
    print("w4a4 prefill: relF %.3e worst %.3e max %.2f ulp" % (fro, worst, ulps))
    assert fro < 1e-5


def test_w4a4_integer_case_exact():
    """4-bit codes, unit scales: every output is an exact integer sum."""
    g = np.random.Generator(np.random.PCG64(405))
    M, K, N = 300, 1024, 130
    codes = W.q4_0_codes(M, K, g)
    q = g.integers(-7, 8, size=(N, K)).astype(np.int8)
    ones_w = np.full((M, K // 32), 0x3C00, dtype=np.uint16)
    ones_x = np.full((N, K // 32), 0x3C00, dtype=np.uint16)
    out = torch.empty((N, M), dtype=torch.float32, device="cuda")
    vq.gemm_q4_0(to_dev(codes), to_dev(ones_w, torch.float16), to_dev(q), out,
                 x_scales=to_dev(ones_x, torch.float16), alpha=1.0)
    torch.cuda.synchronize()
    assert np.array_equal(out_to_f64(out), oracle.gemm_w4a8(codes, ones_w, q, ones_x, N, M, K, alpha=1.0))
