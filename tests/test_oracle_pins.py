"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a closed form, an independent library
routine, an exact integer or rational computation, or a hand-written fixture,
chosen so that a plausible slip in the oracle (a dropped offset, a transposed
operand, a wrong block or tile index, a wrong nibble, a wrong Hadamard order)
fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

# ---------------------------------------------------------------- helpers (tests only)


def _np_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _torch_bf16(bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _torch_e4m3(bits):
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _int4_twos_complement(q):
    """Value of the 4-bit pattern (q XOR 8) read as two's complement."""
    v = np.asarray(q, dtype=np.int64) ^ 8
    return np.where(v >= 8, v - 16, v)


def _unpack_codes(codes, K):
    """[M][K] codes 0..15 from packed [M][K/2] bytes, per the layout reading."""
    M = codes.shape[0]
    b = codes.reshape(M, K // 32, 16)
    lo = (b & 0x0F).astype(np.int64)
    hi = (b >> 4).astype(np.int64)
    return np.concatenate([lo, hi], axis=2).reshape(M, K)


def _pack_codes(q):
    """Inverse of _unpack_codes for building test inputs."""
    M, K = q.shape
    b = q.reshape(M, K // 32, 2, 16).astype(np.uint8)
    return (b[:, :, 0, :] | (b[:, :, 1, :] << 4)).reshape(M, K // 2)


def _read_golden(path):
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


# ---------------------------------------------------------------- decoders


def test_f16_decoder_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = _np_f16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bf16_decoder_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = _torch_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decoder_matches_torch_all_256():
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.e4m3_to_f64(bits)
    ref = _torch_e4m3(bits)
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7F and 0xFF only: the FN variant has no infinities
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_spot_values_golden(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_spot_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            got = oracle.e4m3_to_f64([int(code, 16)])[0]
            if val == "nan":
                assert math.isnan(got)
            else:
                assert got == float(val), (code, got, val)


def test_f32_to_f16_rounding_matches_numpy():
    g = np.random.Generator(np.random.PCG64(7))
    # random magnitudes across the whole fp16 range, including subnormals and overflow
    mags = np.exp2(g.uniform(-27, 17, size=20000)).astype(np.float32)
    vals = mags * np.where(g.random(20000) < 0.5, -1, 1).astype(np.float32)
    # exact ties between neighbouring fp16 values, in normal and subnormal range
    h = np.arange(0, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    ties = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    vals = np.concatenate([vals, ties.astype(np.float32), np.float32([0.0, -0.0, 65504, 65519.99, 65520,
                                                                     1e-8, 2.0 ** -25, 2.0 ** -24])])
    got = oracle.f32_to_f16_bits(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- Q4_0 format


def test_q4_0_offset_eight_equals_top_bit_flip():
    """Offset 8 and the top-bit flip to two's complement give the same value
    (1bit serve page, 'Prompt processing: 4-bit activations, rotated first')."""
    K = 32
    for q in range(16):
        codes = np.full((1, 16), q | (q << 4), dtype=np.uint8)
        scales = np.array([[0x3C00]], dtype=np.uint16)  # 1.0
        w = oracle.q4_0_dequant(codes, scales, 1, K)
        assert np.all(w == _int4_twos_complement(q)), q


def test_q4_0_nibble_order_golden(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "q4_0_one_block.txt"))
    codes = np.array([[int(v, 16) for v in g["bytes"]]], dtype=np.uint8)
    scales = np.array([[int(g["scale_bits"][0], 16)]], dtype=np.uint16)
    w = oracle.q4_0_dequant(codes, scales, 1, 32)
    assert np.array_equal(w[0], np.array([float(v) for v in g["weights"]]))


def test_q4_0_block_scale_index():
    """Each 32-wide block of each row takes its own scale: scales 2^(m*8+b)."""
    M, K = 3, 256
    q = np.arange(M * K).reshape(M, K) % 16
    codes = _pack_codes(q)
    sc = np.array([[2.0 ** (-(m * 8 + b)) for b in range(K // 32)] for m in range(M)])
    scales = W.f32_to_f16_bits(sc)
    w = oracle.q4_0_dequant(codes, scales, M, K)
    ref = _int4_twos_complement(q) * np.repeat(sc, 32, axis=1)
    assert np.array_equal(w, ref)


# ---------------------------------------------------------------- Q4_0 verify GEMM


@pytest.mark.parametrize("act_dtype", ["bf16", "f16"])
def test_gemm_q4_0_integer_case_exact(act_dtype):
    """Unit scales and small-integer activations: fp64 is exact, so the oracle
    must equal numpy's int64 product of activations and (q - 8)."""
    g = np.random.Generator(np.random.PCG64(11))
    N, M, K = 5, 37, 320
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = np.full((M, K // 32), 0x3C00, dtype=np.uint16)
    xi = g.integers(-4, 5, size=(N, K))
    bits = W.f32_to_bf16_bits(xi) if act_dtype == "bf16" else W.f32_to_f16_bits(xi)
    dt = oracle.BF16 if act_dtype == "bf16" else oracle.F16
    y = oracle.gemm_q4_0(codes, scales, bits, dt, N, M, K)
    ref = xi @ _int4_twos_complement(_unpack_codes(codes, K)).T
    assert np.array_equal(y, ref.astype(np.float64))


def test_gemm_q4_0_exact_rationals_tiny():
    """Brute force with exact rationals over independently decoded inputs."""
    g = np.random.Generator(np.random.PCG64(12))
    N, M, K = 2, 3, 64
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.uniform(0.001, 0.02, size=(M, K // 32)))
    act = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    xs = _torch_bf16(act)
    ds = _np_f16(scales)
    qs = _int4_twos_complement(_unpack_codes(codes, K))
    y = oracle.gemm_q4_0(codes, scales, act, oracle.BF16, N, M, K, alpha=0.75)
    for n in range(N):
        for m in range(M):
            exact = sum(Fraction(float(xs[n, k])) * Fraction(float(ds[m, k // 32])) * int(qs[m, k])
                        for k in range(K)) * Fraction(3, 4)
            assert abs(Fraction(float(y[n, m])) - exact) <= abs(exact) * Fraction(1, 10 ** 13) + \
                Fraction(1, 10 ** 300)


def test_gemm_q4_0_vs_library_matmul_tiny_config():
    """Full tiny workload: oracle vs numpy BLAS over independently dequantised W."""
    t = W.tiny()
    M, K, N = t["M"], t["K"], t["N"]
    y = oracle.gemm_q4_0(t["codes"], t["scales"], t["act"], oracle.F16, N, M, K)
    w64 = _int4_twos_complement(_unpack_codes(t["codes"], K)) * np.repeat(_np_f16(t["scales"]), 32, axis=1)
    ref = _np_f16(t["act"]) @ w64.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_gemm_q4_0_one_hot_reads_single_weight():
    """Row n of X = e_{k_n}: Y[n][m] must be w[m][k_n] (catches transposed
    operands and wrong k indexing)."""
    g = np.random.Generator(np.random.PCG64(13))
    M, K = 40, 128
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.uniform(0.001, 0.02, size=(M, K // 32)))
    ks = np.array([0, 1, 15, 16, 17, 31, 32, 63, 100, 127])
    x = np.zeros((ks.size, K), dtype=np.float32)
    x[np.arange(ks.size), ks] = 1.0
    y = oracle.gemm_q4_0(codes, scales, W.f32_to_bf16_bits(x), oracle.BF16, ks.size, M, K)
    wref = _int4_twos_complement(_unpack_codes(codes, K)) * np.repeat(_np_f16(scales), 32, axis=1)
    assert np.array_equal(y, wref[:, ks].T)


def test_gemm_q4_0_scale_doubling_adds_one_block():
    g = np.random.Generator(np.random.PCG64(14))
    N, M, K = 3, 8, 160
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.uniform(0.001, 0.02, size=(M, K // 32)))
    act = W.f32_to_bf16_bits(g.integers(-3, 4, size=(N, K)))   # integers: sums stay exact
    y1 = oracle.gemm_q4_0(codes, scales, act, oracle.BF16, N, M, K)
    m, b = 5, 3
    s2 = scales.copy()
    s2[m, b] = W.f32_to_f16_bits(2 * _np_f16(scales[m:m + 1, b:b + 1]))[0, 0]
    y2 = oracle.gemm_q4_0(codes, s2, act, oracle.BF16, N, M, K)
    blk = oracle.gemm_q4_0(codes[:, 16 * b:16 * b + 16], scales[:, b:b + 1],
                           act.reshape(N, K)[:, 32 * b:32 * b + 32], oracle.BF16, N, M, 32)
    others = [c for c in range(M) if c != m]
    assert np.array_equal(y1[:, others], y2[:, others])
    assert np.array_equal(y2[:, m] - y1[:, m], blk[:, m])


def test_gemm_q4_0_column_subset_matches_full():
    t = W.tiny()
    M, K, N = t["M"], t["K"], t["N"]
    full = oracle.gemm_q4_0(t["codes"], t["scales"], t["act"], oracle.F16, N, M, K)
    cols = np.array([255, 0, 17, 128])
    sub = oracle.gemm_q4_0(t["codes"], t["scales"], t["act"], oracle.F16, N, M, K, cols=cols)
    assert np.array_equal(sub, full[:, cols])


def test_gemm_q4_0_linear_in_activations():
    g = np.random.Generator(np.random.PCG64(15))
    N, M, K = 2, 16, 96
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.uniform(0.001, 0.02, size=(M, K // 32)))
    a = g.integers(-8, 9, size=(N, K)).astype(np.float32)
    b = g.integers(-8, 9, size=(N, K)).astype(np.float32)
    ya = oracle.gemm_q4_0(codes, scales, W.f32_to_bf16_bits(a), oracle.BF16, N, M, K)
    yb = oracle.gemm_q4_0(codes, scales, W.f32_to_bf16_bits(b), oracle.BF16, N, M, K)
    yab = oracle.gemm_q4_0(codes, scales, W.f32_to_bf16_bits(a + 2 * b), oracle.BF16, N, M, K)
    assert np.allclose(yab, ya + 2 * yb, rtol=1e-13, atol=1e-13 * np.abs(yab).max())


# ---------------------------------------------------------------- FP8 verify GEMM


def test_fp8_integer_case_exact():
    g = np.random.Generator(np.random.PCG64(21))
    N, M, K = 4, 130, 256
    wi = g.integers(-8, 9, size=(M, K)).astype(np.float32)   # exact in E4M3
    w = W.f32_to_e4m3_bits(wi)
    ts = np.ones(((M + 127) // 128, K // 128), dtype=np.float32)
    xi = g.integers(-4, 5, size=(N, K))
    y = oracle.gemm_fp8_blk128(w, ts, W.f32_to_bf16_bits(xi), oracle.BF16, N, M, K)
    assert np.array_equal(y, (xi @ wi.astype(np.int64).T).astype(np.float64))


def test_fp8_tile_scale_index_one_hot():
    """One-hot rows and distinct power-of-two tile scales: Y[n][m] must be
    e4m3(w[m][k_n]) * s[m // 128][k_n // 128]."""
    g = np.random.Generator(np.random.PCG64(22))
    M, K = 300, 384
    w = W.e4m3_weights(M, K, g)
    ts = np.array([[2.0 ** -(3 * i + j) for j in range(K // 128)] for i in range((M + 127) // 128)],
                  dtype=np.float32)
    ks = np.array([0, 127, 128, 200, 255, 256, 383])
    x = np.zeros((ks.size, K), dtype=np.float32)
    x[np.arange(ks.size), ks] = 1.0
    y = oracle.gemm_fp8_blk128(w, ts, W.f32_to_bf16_bits(x), oracle.BF16, ks.size, M, K)
    wv = _torch_e4m3(w)
    for i, k in enumerate(ks):
        ref = wv[:, k] * ts[np.arange(M) // 128, k // 128].astype(np.float64)
        assert np.array_equal(y[i], ref)


def test_fp8_vs_library_matmul():
    f = W.fp8(M=384, K=512, N=4)
    M, K, N = f["M"], f["K"], f["N"]
    y = oracle.gemm_fp8_blk128(f["w"], f["tscales"], f["act"], oracle.BF16, N, M, K)
    s = np.repeat(np.repeat(f["tscales"].astype(np.float64), 128, axis=0)[:M], 128, axis=1)
    ref = _torch_bf16(f["act"]) @ (_torch_e4m3(f["w"]) * s).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------- Hadamard-32


def test_h32_is_sylvester_hadamard():
    from scipy.linalg import hadamard
    h = oracle.h32_matrix().astype(np.int64)
    assert np.array_equal(h, hadamard(32).astype(np.int64))
    assert np.array_equal(h @ h.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(h, h.T)


def test_fwht_equals_matrix_product_on_integers():
    from scipy.linalg import hadamard
    g = np.random.Generator(np.random.PCG64(31))
    hm = hadamard(32).astype(np.int64)
    for _ in range(20):
        x = g.integers(-1000, 1001, size=32)
        u = oracle.fwht32_f32(x)
        assert np.array_equal(u.astype(np.int64), hm @ x)
        # involution up to the factor 32, and Parseval
        assert np.array_equal(oracle.fwht32_f32(u).astype(np.int64), 32 * x)
        assert int(np.sum(u.astype(np.int64) ** 2)) == 32 * int(np.sum(x ** 2))


def test_quant_zero_block_and_spike():
    K = 64
    x = np.zeros((2, K), dtype=np.float32)
    x[1, 32] = 3.0         # second block of row 1 is 3 * e_0
    x[1, 0] = -0.25        # first block of row 1 is -0.25 * e_0
    q, d, st = oracle.h32_quant_int8(W.f32_to_bf16_bits(x), oracle.BF16, 2, K)
    assert st == 0
    assert np.all(q[0] == 0) and np.all(d[0] == 0)
    # H e_0 is the all-ones vector, so every code of a spiked block has the same magnitude
    for b, v in ((0, -0.25), (1, 3.0)):
        dref = np.float32(np.float32(abs(v)) / np.float32(127)).astype(np.float16)
        assert d[1, b] == dref.view(np.uint16)
        qv = np.clip(np.rint(np.float32(v) / np.float32(dref)), -127, 127)
        assert np.all(q[1, 32 * b:32 * b + 32] == qv)
        assert abs(qv) == 127


def test_quant_math_check_outlier_rows():
    """Codes agree with fp64 H x / d up to rounding; every non-zero block uses
    code magnitude 127; the dequantised block is within d/2 of H x."""
    from scipy.linalg import hadamard
    N, K = 64, 5120
    g = W.rng(W.CFG_PREFILL, 0, W.T_ACT)
    x = W.act_student_outliers(N, K, g, W.rng(W.CFG_PREFILL, 0, W.T_OUTLIER))
    q, d, st = oracle.h32_quant_int8(x, oracle.BF16, N, K)
    assert st == 0
    xs = _torch_bf16(x).reshape(N, K // 32, 32)
    u64 = xs @ hadamard(32).astype(np.float64).T
    dd = _np_f16(d)
    amax = np.abs(u64).max(axis=2)
    # d is amax/127 rounded to fp16 (relative 2^-11), up to fp32 noise in amax
    assert np.all(np.abs(dd - amax / 127) <= dd * (2.0 ** -11) + amax * 1e-6)
    ratio = u64 / dd[:, :, None]
    qq = q.reshape(N, K // 32, 32).astype(np.float64)
    assert np.all(np.abs(qq - ratio) <= 0.5 + 1e-4)
    mism = np.mean(qq != np.clip(np.rint(ratio), -127, 127))
    assert mism < 1e-4
    assert np.all(np.abs(qq).max(axis=2) == 127)


def test_quant4_zero_block_and_spike():
    """4-bit codes: H e_0 is the all-ones vector, so a spiked block quantizes
    to 32 codes of magnitude 7 with d = fp16(|v| / 7); a zero block stays 0."""
    K = 64
    x = np.zeros((2, K), dtype=np.float32)
    x[1, 32] = 3.0
    x[1, 0] = -0.25
    q, d, st = oracle.h32_quant_int4(W.f32_to_bf16_bits(x), oracle.BF16, 2, K)
    assert st == 0
    assert np.all(q[0] == 0) and np.all(d[0] == 0)
    for b, v in ((0, -0.25), (1, 3.0)):
        dref = np.float32(np.float32(abs(v)) / np.float32(7)).astype(np.float16)
        assert d[1, b] == dref.view(np.uint16)
        assert np.all(q[1, 32 * b:32 * b + 32] == (7 if v > 0 else -7))


def test_quant4_math_check_outlier_rows():
    """4-bit codes agree with fp64 H x / d up to rounding, every non-zero
    block reaches magnitude 7 and none exceeds it, d is amax / 7 to fp16."""
    from scipy.linalg import hadamard
    N, K = 64, 2048
    g = W.rng(W.CFG_PREFILL, 0, W.T_ACT)
    x = W.act_student_outliers(N, K, g, W.rng(W.CFG_PREFILL, 0, W.T_OUTLIER))
    q, d, st = oracle.h32_quant_int4(x, oracle.BF16, N, K)
    assert st == 0
    xs = _torch_bf16(x).reshape(N, K // 32, 32)
    u64 = xs @ hadamard(32).astype(np.float64).T
    dd = _np_f16(d)
    amax = np.abs(u64).max(axis=2)
    assert np.all(np.abs(dd - amax / 7) <= dd * (2.0 ** -11) + amax * 1e-6)
    ratio = u64 / dd[:, :, None]
    qq = q.reshape(N, K // 32, 32).astype(np.float64)
    assert np.all(np.abs(qq - np.clip(ratio, -7, 7)) <= 0.5 + 1e-4)
    assert np.all(np.abs(qq).max(axis=2) == 7)


def test_block_quant_without_rotation():
    """The quantizer rule applied to the plain blocks: codes of x / d with
    d = fp16(max |x| / qmax), for both bounds."""
    N, K = 16, 256
    g = np.random.Generator(np.random.PCG64(77))
    x = W.f32_to_bf16_bits(g.standard_normal((N, K)) * np.exp(g.uniform(-3, 3, size=(N, 1))))
    xs = _torch_bf16(x).reshape(N, K // 32, 32)
    for qmax in (127, 7):
        q, d, st = oracle.block_quant(x, oracle.BF16, N, K, qmax, False)
        assert st == 0
        dd = _np_f16(d)
        amax = np.abs(xs).max(axis=2)
        assert np.all(np.abs(dd - amax / qmax) <= dd * (2.0 ** -11))
        qq = q.reshape(N, K // 32, 32).astype(np.float64)
        assert np.all(np.abs(qq - np.clip(xs / dd[:, :, None], -qmax, qmax)) <= 0.5 + 1e-6)
        assert np.all(np.abs(qq).max(axis=2) == qmax)
    q8, d8, _ = oracle.h32_quant_int8(x, oracle.BF16, N, K)
    qr, dr, _ = oracle.block_quant(x, oracle.BF16, N, K, 127, True)
    assert np.array_equal(q8, qr) and np.array_equal(d8, dr)


def _rounding_blocks(golden_dir):
    """The hand-worked blocks of quant_rounding_blocks.txt: (name, qmax,
    rotate, dtype code, input bits [32], expected d bits, expected q [32])."""
    from scipy.linalg import hadamard
    h = hadamard(32).astype(np.float64)
    out = []
    with open(os.path.join(golden_dir, "quant_rounding_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, qmax, rotate, dt, dbits, *ents = line.split()
            u = np.zeros(32)
            q = np.zeros(32, dtype=np.int64)
            for e in ents:
                i, uv, qv = e.split(":")
                u[int(i)] = float.fromhex(uv) if "0x" in uv else float(uv)
                q[int(i)] = int(qv)
            x = h @ u / 32 if rotate == "1" else u
            if dt == "f16":
                bits = W.f32_to_f16_bits(x)
                back = _np_f16(bits)
                code = oracle.F16
            else:
                bits = W.f32_to_bf16_bits(x)
                back = _torch_bf16(bits)
                code = oracle.BF16
            assert np.array_equal(back, x), name  # the fixture's input is exact in its dtype
            out.append((name, int(qmax), rotate == "1", code, bits, int(dbits, 16), q))
    return out


def test_quant_rounding_rules_golden(golden_dir):
    """Hand-worked blocks: ties of u / d go to the even code, the code divides
    by the stored fp16 scale (not the fp32 quotient), and the clamp to
    +-qmax acts where the scale rounds down into the fp16 subnormals.  An
    oracle rounding half away from zero, dividing by fp32(amax / qmax) or
    leaving out the clamp fails here."""
    blocks = _rounding_blocks(golden_dir)
    assert {b[0].rstrip("u") for b in blocks} == {"tie127", "tie7", "stored127", "stored7", "clamp127", "clamp7"}
    for name, qmax, rotate, code, bits, dbits, qref in blocks:
        q, d, st = oracle.block_quant(bits.reshape(1, 32), code, 1, 32, qmax, rotate)
        assert st == 0, name
        assert int(d[0, 0]) == dbits, (name, hex(int(d[0, 0])))
        assert np.array_equal(q[0].astype(np.int64), qref), (name, q[0], qref)
        if rotate:  # the named quantizers are the rotated rule
            fn = oracle.h32_quant_int8 if qmax == 127 else oracle.h32_quant_int4
            q2, d2, _ = fn(bits.reshape(1, 32), code, 1, 32)
            assert np.array_equal(q2, q) and np.array_equal(d2, d), name


def test_quant_clamp_binds_only_below_fp16_normals():
    """The clamp can act only when d = fp16(amax / qmax) rounds down by more
    than half a code: with a normal fp16 d the relative rounding is at most
    2^-11, so |u| / d <= qmax (1 + 2^-10) < qmax + 1/2 and rint never leaves
    the range.  Checked on a sweep of amax over the normal range: every
    block's largest code is exactly qmax and no code exceeds it."""
    g = np.random.Generator(np.random.PCG64(91))
    for qmax in (127, 7):
        amax = np.exp2(g.uniform(-13.5, 15, size=2000)) * qmax
        x = np.zeros((2000, 32))
        x[:, 0] = amax
        x[:, 1:] = g.uniform(-1, 1, size=(2000, 31)) * amax[:, None]
        bits = W.f32_to_bf16_bits(x)
        q, d, st = oracle.block_quant(bits, oracle.BF16, 2000, 32, qmax, False)
        assert st == 0
        assert np.all(_np_f16(d) >= 2.0 ** -14)  # every scale is a normal fp16
        assert np.all(np.abs(q.astype(np.int64)).max(axis=1) == qmax)


def test_activation_rounding_error_study():
    """Prompt-processing numerics on the prefill activations (Student-t rows
    with outlier channels): the error that rounding the activations alone adds
    to a Q4_0 product, for int8 and 4-bit codes, with and without the H32
    rotation (rotated blocks dequantized and rotated back: H H = 32 I).  The
    pages: 4-bit activations are lossy, and the rotation removes about a third
    of that error.  Here: 4-bit 11.4% -> 6.7% with the rotation, int8 1.1% ->
    0.37%."""
    from scipy.linalg import hadamard
    N, K, M = 64, 2048, 256
    x = W.act_student_outliers(N, K, W.rng(W.CFG_PREFILL, 0, W.T_ACT), W.rng(W.CFG_PREFILL, 0, W.T_OUTLIER))
    g = np.random.Generator(np.random.PCG64(5))
    codes, sc = W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g)
    w = oracle.q4_0_dequant(codes, sc, M, K)
    xf = _torch_bf16(x)
    y = xf @ w.T
    h = hadamard(32).astype(np.float64)
    err = {}
    for qmax in (127, 7):
        for rot in (True, False):
            q, d, st = oracle.block_quant(x, oracle.BF16, N, K, qmax, rot)
            assert st == 0
            xh = q.astype(np.float64) * np.repeat(_np_f16(d), 32, axis=1)
            if rot:
                xh = (xh.reshape(N, K // 32, 32) @ h).reshape(N, K) / 32
            err[(qmax, rot)] = np.linalg.norm(xh @ w.T - y) / np.linalg.norm(y)
    print("activation rounding error: int8 %.4f / %.4f, 4-bit %.4f / %.4f (rotated / plain)" % (
        err[(127, True)], err[(127, False)], err[(7, True)], err[(7, False)]))
    assert err[(7, True)] < 0.8 * err[(7, False)]       # the rotation removes a good part of the 4-bit error
    assert err[(127, True)] < err[(127, False)]
    assert err[(7, True)] > 5 * err[(127, True)]          # 4-bit codes stay far lossier than int8


def test_rotation_leaves_block_products_unchanged():
    """(H x_b) . (H w_b) / 32 = x_b . w_b for every block: the reading alpha = 1/32
    restores the product when both sides use the +-1 Sylvester H32."""
    h = oracle.h32_matrix().astype(np.float64)
    t = W.tiny()
    M, K = t["M"], t["K"]
    w = oracle.q4_0_dequant(t["codes"], t["scales"], M, K).reshape(M, K // 32, 32)
    x = _np_f16(t["act"]).reshape(-1, K // 32, 32)
    plain = np.einsum("nbj,mbj->nmb", x, w)
    rot = np.einsum("nbj,mbj->nmb", x @ h.T, w @ h.T) / 32
    assert np.max(np.abs(rot - plain)) <= 1e-12 * np.max(np.abs(plain))


# ---------------------------------------------------------------- W4A8


def test_w4a8_integer_case_exact():
    g = np.random.Generator(np.random.PCG64(41))
    N, M, K = 6, 33, 192
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qx = g.integers(-127, 128, size=(N, K)).astype(np.int8)
    ones_w = np.full((M, K // 32), 0x3C00, dtype=np.uint16)
    ones_x = np.full((N, K // 32), 0x3C00, dtype=np.uint16)
    y = oracle.gemm_w4a8(codes, ones_w, qx, ones_x, N, M, K)
    ref = qx.astype(np.int64) @ _int4_twos_complement(_unpack_codes(codes, K)).T
    assert np.array_equal(y, ref.astype(np.float64))
    # single block dots
    wq = _int4_twos_complement(_unpack_codes(codes, K))
    for (n, m, b) in ((0, 0, 0), (5, 32, 5), (3, 7, 2)):
        ref_b = int(qx[n, 32 * b:32 * b + 32].astype(np.int64) @ wq[m, 32 * b:32 * b + 32])
        assert oracle.w4a8_block_dot(codes, qx, K, n, m, b) == ref_b


def test_w4a8_equals_dequantised_matmul():
    g = np.random.Generator(np.random.PCG64(42))
    N, M, K = 8, 40, 256
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    wsc = W.f32_to_f16_bits(g.lognormal(-5, 0.5, size=(M, K // 32)))
    x = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    qx, dx, st = oracle.h32_quant_int8(x, oracle.BF16, N, K)
    assert st == 0
    y = oracle.gemm_w4a8(codes, wsc, qx, dx, N, M, K, alpha=1 / 32)
    xhat = qx.astype(np.float64) * np.repeat(_np_f16(dx), 32, axis=1)
    what = _int4_twos_complement(_unpack_codes(codes, K)) * np.repeat(_np_f16(wsc), 32, axis=1)
    ref = (xhat @ what.T) / 32
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


# ------------------------------------------------------------ greedy verification


def test_greedy_choice_matches_numpy_argmax():
    """The target's choice per row is numpy's argmax (first maximum, a NaN wins,
    -0 equals +0), for float32 and for the 16-bit formats."""
    g = np.random.Generator(np.random.PCG64(51))
    n, v = 9, 3001
    x = g.standard_normal((n, v)).astype(np.float32)
    x[1, [17, 2000]] = 9.0                  # a tie: the first index
    x[2, 40] = np.nan                       # a NaN: chosen
    x[2, 41] = np.inf
    x[3] = -np.inf
    x[3, [5, 3]] = [-0.0, 0.0]              # -0 == +0: the first of them (3)
    x[4] = np.float32(-1.0)                 # all equal: index 0
    t, _ = oracle.greedy_verify(x, oracle.F32, np.zeros(n - 1, np.int32))
    assert np.array_equal(t, np.argmax(x, axis=1))
    assert t[1] == 17 and t[2] == 40 and t[3] == 3 and t[4] == 0
    for dt, conv in ((oracle.BF16, W.f32_to_bf16_bits), (oracle.F16, W.f32_to_f16_bits)):
        bits = conv(np.nan_to_num(x, nan=0.0, posinf=60000.0, neginf=-60000.0))
        vals = torch.from_numpy(bits.view(np.int16).copy()).view(
            torch.bfloat16 if dt == oracle.BF16 else torch.float16).float().numpy()
        t16, _ = oracle.greedy_verify(bits, dt, np.zeros(n - 1, np.int32))
        assert np.array_equal(t16, np.argmax(vals, axis=1)), dt


def test_greedy_commits_the_accepted_prefix_plus_one():
    """One-hot logits fix the target's choices; the number of committed tokens is
    the length of the matching draft prefix plus the target's own next token."""
    n, v = 16, 50
    choice = np.array([(7 * i + 3) % v for i in range(n)], dtype=np.int32)
    logits = np.full((n, v), -1.0, dtype=np.float32)
    logits[np.arange(n), choice] = 4.0
    for a in (0, 1, 5, 14, 15):
        draft = choice[:n - 1].copy()
        if a < n - 1:
            draft[a] = (draft[a] + 1) % v       # first disagreement at position a
            draft[a + 1:] = 0                   # later proposals do not matter
        t, count = oracle.greedy_verify(logits, oracle.F32, draft)
        assert np.array_equal(t, choice)
        assert count == a + 1
    t, count = oracle.greedy_verify(logits[:1], oracle.F32, np.zeros(0, np.int32))
    assert count == 1 and t[0] == choice[0]   # a block of one row commits the target's token


# ------------------------------------------------------------ offline H32 rotation of Q4_0 weights


def _dequant_np(codes, scales, M, K):
    q = _unpack_codes(codes, K).astype(np.float64)
    return (q - 8) * np.repeat(_np_f16(scales), 32, axis=1)


def test_rotation_requantizes_to_the_nearest_level():
    """Per block: the rotated values are H32 w (exact here: every value is the
    block scale times an integer); the new scale is fp16(m / -8) for the value
    m of largest magnitude; every code is the nearest of the 16 levels d (q - 8)
    (rounding half up, 15 at the top), checked in fp64 away from exact ties."""
    import scipy.linalg
    g = np.random.Generator(np.random.PCG64(61))
    M, K = 24, 256
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.lognormal(-5, 0.5, size=(M, K // 32)) * g.choice([-1, 1], size=(M, K // 32)))
    codes[3, 16:32] = 0x88                       # a block of zeros (codes 8)
    co, so = oracle.q4_0_rotate_h32(codes, scales, M, K)
    H = scipy.linalg.hadamard(32).astype(np.float64)
    w = _dequant_np(codes, scales, M, K).reshape(M, K // 32, 32)
    x = w @ H.T                                   # H32 applied to every block
    qn = _unpack_codes(co, K).reshape(M, K // 32, 32)
    dn = _np_f16(so)
    for m in range(M):
        for b in range(K // 32):
            xb = x[m, b]
            j = int(np.argmax(np.abs(xb)))       # first of the largest magnitudes
            d = xb[j] / -8.0
            assert dn[m, b] == np.float64(np.float16(d)), (m, b)
            if d == 0:
                assert (qn[m, b] == 8).all()
                continue
            t = xb / d + 8.5
            ref = np.minimum(15, np.floor(t))
            near_tie = np.abs(t - np.round(t)) < 1e-5
            assert np.array_equal(qn[m, b][~near_tie], ref[~near_tie]), (m, b)
            assert qn[m, b][j] == 0
    assert dn[3, 1] == 0 and (qn[3, 1] == 8).all()


def test_rotation_round_trips_one_hot_blocks_and_keeps_products():
    """A block c * e_0 rotates to c in every position, which requantizes exactly
    (code 0 at d = c / -8), so H32 of the result / 32 gives the block back; a
    block c * e_j with j > 0 rotates to +-c, and the -c side lands on the top
    code 15 (7 d = -7c/8: the 16 levels stop at +7); for general blocks the
    rotated product / 32 stays within the requantization bound of the plain
    product."""
    import scipy.linalg
    H = scipy.linalg.hadamard(32).astype(np.float64)
    M, K = 8, 32
    codes = np.full((M, K // 2), 0x88, dtype=np.uint8)
    codes[:, 0] = 0x8F                           # code 15 (+7 d) at k = 0
    codes[5, 0] = 0x80                           # code 0 (-8 d) at k = 0
    scales = W.f32_to_f16_bits(np.array([[2.0 ** -e] for e in range(4, 12)]))
    co, so = oracle.q4_0_rotate_h32(codes, scales, M, K)
    w = _dequant_np(codes, scales, M, K)
    wr = _dequant_np(co, so, M, K)
    assert np.array_equal(wr @ H.T / 32, w)
    one = np.full((1, 16), 0x88, dtype=np.uint8)
    one[0, 3] = 0x8F                             # c * e_3
    co, so = oracle.q4_0_rotate_h32(one, np.array([[0x2C00]], np.uint16), 1, 32)
    c = 7 * 2.0 ** -4
    assert np.array_equal(_dequant_np(co, so, 1, 32)[0], np.where(H[:, 3] > 0, c, -7 * c / 8))
    g = np.random.Generator(np.random.PCG64(62))
    M, K = 16, 512
    codes = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    scales = W.f32_to_f16_bits(g.lognormal(-5, 0.5, size=(M, K // 32)))
    co, so = oracle.q4_0_rotate_h32(codes, scales, M, K)
    w = _dequant_np(codes, scales, M, K).reshape(M, K // 32, 32)
    wr = _dequant_np(co, so, M, K).reshape(M, K // 32, 32)
    # requantization error per element: half a level inside the range, and up
    # to a whole level where -m lands on the top code 15; the stored scale is
    # d rounded to fp16, which moves the levels by up to 8 * 2^-11 of a level
    err = np.abs(wr - w @ H.T)
    assert (err <= np.abs(_np_f16(so))[..., None] * 1.005).all()
    xv = g.standard_normal((3, K))
    xr = (xv.reshape(3, K // 32, 32) @ H.T).reshape(3, K)
    plain = xv @ w.reshape(M, K).T
    rotated = xr @ wr.reshape(M, K).T / 32
    bound = (np.abs(xr) @ (np.abs(_np_f16(so)).repeat(32, axis=1)).T) / 32
    assert (np.abs(rotated - plain) <= bound * 1.005).all()
