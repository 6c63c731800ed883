"""The FP8 block-scaled GEMM for prompt-sized row counts on the GPU, through
the C ABI, against the CPU oracle: parity, exact integer cases, rows
bit-identical for any number of rows."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
ORACLE_DT = {"bf16": oracle.BF16, "f16": oracle.F16}


def _bits(x, dt):
    return W.f32_to_bf16_bits(x) if dt == "bf16" else W.f32_to_f16_bits(x)


def _run(w, ts, bits, act="bf16", out="bf16"):
    x = to_dev(bits, TORCH_DT[act])
    y = torch.empty((x.shape[0], w.shape[0]), dtype=TORCH_DT[out], device="cuda")
    vq.gemm_fp8_blk128_prefill(to_dev(w), to_dev(ts), x, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("N,M,K", [(1, 17, 128), (129, 129, 256), (300, 200, 384), (512, 512, 1024),
                                   (64, 1000, 2048), (1000, 1200, 256), (5, 1, 128), (2, 288, 128)])
def test_ragged_shapes_parity(N, M, K):
    g = np.random.Generator(np.random.PCG64(801 + N + M))
    f = W.fp8(M=M, K=K, N=16)
    x = _bits(g.standard_normal((N, K)), "bf16")
    y = out_to_f64(_run(f["w"], f["tscales"], x))
    parity(y, oracle.gemm_fp8_blk128(f["w"], f["tscales"], x, oracle.BF16, N, M, K), "bf16")


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
def test_dtype_combinations_parity(act, out):
    g = np.random.Generator(np.random.PCG64(810))
    N, M, K = 200, 384, 512
    f = W.fp8(M=M, K=K, N=16)
    x = _bits(g.standard_normal((N, K)), act)
    y = out_to_f64(_run(f["w"], f["tscales"], x, act, out))
    parity(y, oracle.gemm_fp8_blk128(f["w"], f["tscales"], x, ORACLE_DT[act], N, M, K), out)


@pytest.mark.parametrize("N,M,K", [(160, 256, 768), (130, 700, 384), (257, 961, 256)])
def test_integer_case_bit_exact(N, M, K):
    """E4M3 codes of small integers, power-of-two tile scales and integer rows:
    every partial sum is an exact fp32 integer multiple, so the output equals
    the exact oracle bit for bit (one ragged workgroup tile, and several
    320-feature tiles with ragged last ones in both directions)."""
    g = np.random.Generator(np.random.PCG64(811 + M))
    ints = {0x38: 1.0, 0x40: 2.0, 0x44: 3.0, 0x48: 4.0, 0xB8: -1.0, 0xC0: -2.0, 0x00: 0.0}
    w = g.choice(np.array(list(ints), dtype=np.uint8), size=(M, K))
    ts = np.ldexp(1.0, g.integers(-3, 3, size=((M + 127) // 128, K // 128))).astype(np.float32)
    x = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)).astype(np.float32))
    y = out_to_f64(_run(w, ts, x, out="f32"))
    assert np.array_equal(y, oracle.gemm_fp8_blk128(w, ts, x, oracle.BF16, N, M, K))


def test_rows_bit_identical_for_any_row_count():
    g = np.random.Generator(np.random.PCG64(812))
    N, M, K = 512, 640, 1024
    f = W.fp8(M=M, K=K, N=16)
    x = _bits(0.5 * g.standard_t(3, size=(N, K)), "bf16")
    full = bits_u16(_run(f["w"], f["tscales"], x))
    for r0, r1 in ((0, 1), (7, 8), (100, 228), (0, 16), (511, 512)):
        assert np.array_equal(bits_u16(_run(f["w"], f["tscales"], np.ascontiguousarray(x[r0:r1]))), full[r0:r1])


def test_prefill_workload_sampled():
    """512 bf16 rows over the FP8 workload's 17408 x 5120 weights (its
    distributions), sampled output columns against the oracle."""
    g = np.random.Generator(np.random.PCG64(813))
    f = W.fp8(M=17408, K=5120, N=16)
    x = _bits(g.standard_normal((512, 5120)), "bf16")
    y = out_to_f64(_run(f["w"], f["tscales"], x))
    cols = np.unique(np.concatenate([[0, 127, 128, 17407], g.choice(17408, 128, replace=False)]))
    fro, worst, ulps = parity(y[:, cols], oracle.gemm_fp8_blk128(f["w"], f["tscales"], x, oracle.BF16, 512, 17408,
                                                                  5120, cols=cols), "bf16")
    print("fp8 prefill 512x17408x5120: relF %.3e worst %.3e max %.2f ulp" % (fro, worst, ulps))
