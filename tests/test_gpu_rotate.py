"""The offline H32 rotation of Q4_0 weights on the GPU, through the C ABI:
codes and scales bit-identical to the CPU oracle (integer decisions taken in
the same fp32 steps), and the rotated W4A8 path measured against the exact
product of the unrotated weights."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import to_dev

pytestmark = pytest.mark.gpu


def _rotate_dev(codes, scales):
    c, s = vq.q4_0_rotate_h32(to_dev(codes), to_dev(scales, torch.float16))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("M,K", [(1, 32), (17, 96), (300, 480), (256, 5120), (17408, 5120)])
def test_rotation_bit_identical_to_oracle(M, K):
    g = np.random.Generator(np.random.PCG64(701 + M))
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.lognormal(-5, 0.5, size=(M, K // 32)) * g.choice([-1.0, 1.0], size=(M, K // 32)))
    if M >= 17:
        codes[1, :16] = 0x88                       # a block of zeros
        scales[2, 0] = 0x0000                      # a zero scale
        scales[3, 0] = 0x8000                      # a negative zero scale
        codes[4, :16] = 0x8F                       # k = 0..15 at +7 d, k = 16..31 at 0: ties in |H32 x|
        scales[5, 0] = 0x0001                      # the smallest subnormal scale
        scales[6, 0] = 0x7BFF                      # the largest finite scale
    if M == 17408:  # full size: compare a sample of rows
        rows = np.unique(np.concatenate([np.arange(8), g.choice(M, 248, replace=False)]))
    else:
        rows = np.arange(M)
    co, so = _rotate_dev(codes, scales)
    rc, rs = oracle.q4_0_rotate_h32(codes[rows], scales[rows], len(rows), K)
    assert np.array_equal(co[rows], rc)
    assert np.array_equal(so[rows], rs)


def test_rotated_w4a8_error_study():
    """The W4A8 path as the pages run it: weights rotated offline, activations
    rotated and quantized to int8 per 32-block, exact int8 block dots, alpha =
    1/32 -- against the fp64 product of the unrotated weights, next to the
    bf16-activation verify GEMM on the same weights.  Prints the relative
    errors; the bounds are loose sanity limits (a 4-bit requantization adds an
    error comparable to the original 4-bit rounding)."""
    g = np.random.Generator(np.random.PCG64(720))
    p = W.prefill(N=64, M=512, K=5120)
    N, M, K = p["N"], p["M"], p["K"]
    codes, scales, act = p["codes"], p["scales"], p["act"]
    ref = oracle.gemm_q4_0(codes, scales, act, oracle.BF16, N, M, K)
    nref = np.linalg.norm(ref)
    dev = torch.device("cuda:0")
    c = to_dev(codes)
    s = to_dev(scales, torch.float16)
    x = to_dev(act, torch.bfloat16)
    y16 = torch.empty((N, M), dtype=torch.float32, device=dev)
    vq.gemm_q4_0(c, s, x, y16)
    cr, sr = vq.q4_0_rotate_h32(c, s)
    q = torch.empty((N, K), dtype=torch.int8, device=dev)
    d = torch.empty((N, K // 32), dtype=torch.float16, device=dev)
    vq.hadamard32_quant_int8(x, q, d)
    y8 = torch.empty((N, M), dtype=torch.float32, device=dev)
    vq.gemm_q4_0(cr, sr, q, y8, x_scales=d, alpha=1.0 / 32)
    torch.cuda.synchronize()
    e16 = np.linalg.norm(y16.cpu().double().numpy() - ref) / nref
    e8 = np.linalg.norm(y8.cpu().double().numpy() - ref) / nref
    # the weight requantization alone: exact rotated activations times the rotated weights
    crn = cr.cpu().numpy()
    srn = sr.cpu().view(torch.int16).numpy().view(np.uint16)
    wrot = oracle.q4_0_dequant(crn, srn, M, K)
    import scipy.linalg
    H = scipy.linalg.hadamard(32).astype(np.float64)
    xf = torch.from_numpy(act.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    xr = (xf.reshape(N, K // 32, 32) @ H.T).reshape(N, K)
    ew = np.linalg.norm(xr @ wrot.T / 32 - ref) / nref
    print("relative Frobenius error vs the exact unrotated product: bf16 rows %.2e, "
          "rotated weights alone %.3f, rotated W4A8 path %.3f" % (e16, ew, e8))
    assert e16 < 2e-3
    assert ew < 0.25 and e8 < 0.3 and e8 >= ew * 0.9
