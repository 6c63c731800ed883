"""H32 int8 activation quantizer and the W4A8 int8-MFMA GEMM on the GPU."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu


def gpu_quant(x_bits, x_dtype="bf16"):
    N, K = x_bits.shape
    x = to_dev(x_bits, torch.bfloat16 if x_dtype == "bf16" else torch.float16)
    q = torch.empty((N, K), dtype=torch.int8, device="cuda")
    d = torch.empty((N, K // 32), dtype=torch.float16, device="cuda")
    vq.hadamard32_quant_int8(x, q, d)
    torch.cuda.synchronize()
    return q.cpu().numpy(), bits_u16(d)


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_quantizer_bit_exact_prefill_rows(x_dtype):
    p = W.prefill()
    x = p["act"]
    if x_dtype == "f16":
        x = W.f32_to_f16_bits(torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float().numpy())
    q, d = gpu_quant(x, x_dtype)
    qo, do, st = oracle.h32_quant_int8(x, oracle.BF16 if x_dtype == "bf16" else oracle.F16, *x.shape)
    assert st == 0
    assert np.array_equal(d, do)
    assert np.array_equal(q, qo)


def test_quantizer_rounding_blocks_golden(golden_dir):
    """The hand-worked blocks of tests/golden/quant_rounding_blocks.txt
    (exact ties, division by the stored fp16 scale, the clamp at subnormal
    scales) through both GPU quantizers: codes and scales as worked by hand."""
    from test_oracle_pins import _rounding_blocks
    for name, qmax, rotate, code, bits, dbits, qref in _rounding_blocks(golden_dir):
        if not rotate:
            continue
        x = to_dev(bits.reshape(1, 32), torch.bfloat16 if code == oracle.BF16 else torch.float16)
        q = torch.empty((1, 32), dtype=torch.int8, device="cuda")
        d = torch.empty((1, 1), dtype=torch.float16, device="cuda")
        (vq.hadamard32_quant_int8 if qmax == 127 else vq.hadamard32_quant_int4)(x, q, d)
        torch.cuda.synchronize()
        assert int(bits_u16(d)[0, 0]) == dbits, name
        assert np.array_equal(q.cpu().numpy()[0].astype(np.int64), qref), name


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (7, 4128)])
def test_quantizer_bit_exact_ragged(N, K):
    g = np.random.Generator(np.random.PCG64(N * K))
    x = W.f32_to_bf16_bits(g.standard_normal((N, K)) * np.exp(g.uniform(-8, 8, size=(N, 1))))
    x[0, :32] = 0                      # a zero block
    q, d = gpu_quant(x)
    qo, do, _ = oracle.h32_quant_int8(x, oracle.BF16, N, K)
    assert np.array_equal(d, do) and np.array_equal(q, qo)
    assert np.all(q[0, :32] == 0) and d[0, 0] == 0


class Q4W:
    def __init__(self, codes, scales):
        self.codes_np, self.scales_np = codes, scales
        self.M, self.K = codes.shape[0], codes.shape[1] * 2
        self.codes = to_dev(codes)
        self.scales = to_dev(scales, torch.float16)

    def run(self, q_np, d_bits, alpha, out_dtype=torch.float32):
        qx = to_dev(q_np)
        dx = to_dev(d_bits, torch.float16)
        out = torch.empty((qx.shape[0], self.M), dtype=out_dtype, device="cuda")
        vq.gemm_q4_0(self.codes, self.scales, qx, out, x_scales=dx, alpha=alpha)
        torch.cuda.synchronize()
        return out


def test_w4a8_integer_accumulators_bit_exact():
    g = np.random.Generator(np.random.PCG64(301))
    M, K, N = 96, 5120, 70
    w = Q4W(W.q4_0_codes(M, K, g), np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    qx = g.integers(-127, 128, size=(N, K)).astype(np.int8)
    ones = np.full((N, K // 32), 0x3C00, dtype=np.uint16)
    y = out_to_f64(w.run(qx, ones, 1.0))
    ref = oracle.gemm_w4a8(w.codes_np, w.scales_np, qx, ones, N, M, K, alpha=1.0)
    assert np.array_equal(y, ref)


def test_w4a8_single_block_dots_exact():
    g = np.random.Generator(np.random.PCG64(302))
    M, K, N = 33, 32, 5
    w = Q4W(W.q4_0_codes(M, K, g), np.full((M, 1), 0x3C00, dtype=np.uint16))
    qx = g.integers(-127, 128, size=(N, K)).astype(np.int8)
    y = out_to_f64(w.run(qx, np.full((N, 1), 0x3C00, dtype=np.uint16), 1.0))
    for n in range(N):
        for m in range(M):
            assert y[n, m] == oracle.w4a8_block_dot(w.codes_np, qx, K, n, m, 0)


def test_prefill_config_parity_sampled():
    """512 rows x 17408 x 5120: GPU quantizer then W4A8 GEMM (alpha = 1/32), checked
    against the oracle GEMM on the GPU's own codes and scales."""
    p = W.prefill()
    q, d = gpu_quant(p["act"])
    w = Q4W(p["codes"], p["scales"])
    y = out_to_f64(w.run(q, d, 1.0 / 32))
    g = np.random.Generator(np.random.PCG64(303))
    cols = np.unique(np.concatenate([[0, 15, 16, w.M - 1], g.choice(w.M, 192, replace=False)]))
    ref = oracle.gemm_w4a8(p["codes"], p["scales"], q, d, p["N"], w.M, w.K, cols=cols, alpha=1.0 / 32)
    fro, worst, ulps = parity(y[:, cols], ref, "f32")
    print("prefill: relF %.3e worst %.3e max %.2f ulp" % (fro, worst, ulps))
    assert fro < 1e-5        # only fp32-vs-fp64 scale arithmetic differs


@pytest.mark.parametrize("M,K,N", [(17, 64, 1), (300, 480, 65), (64, 4128, 3), (200, 256, 300), (130, 160, 129),
                                   (1500, 256, 650), (1, 32, 1), (288, 32, 2)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_w4a8_ragged_parity(M, K, N, out_dtype):
    g = np.random.Generator(np.random.PCG64(M + K + N))
    w = Q4W(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    q, d = gpu_quant(x)
    y = out_to_f64(w.run(q, d, 1.0 / 32, out_dtype))
    name = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[out_dtype]
    parity(y, oracle.gemm_w4a8(w.codes_np, w.scales_np, q, d, N, M, K, alpha=1.0 / 32), name)
