"""Seeded synthetic inputs for the verify GEMM, shared by tests and the benchmark.

This module holds random draws and input encodings only: it never decodes a
weight, never multiplies, and knows nothing of either the oracle or the HIP
library.  Every tensor is returned as raw bits (uint8 / uint16 / float32 numpy
arrays) so both sides read exactly the same bytes.

Recipes (seed = 1_000_003 * config + 1009 * layer + tensor_id; tensor ids:
0 codes, 1 weight scales, 2 activations, 3 outlier-channel choice,
4 E4M3 values, 5 FP8 tile scales):

  tiny       Q4_0 256 x 512, codes U{0..15}, fp16 scales U[0.001, 0.02],
             8 fp16 activation rows ~ N(0, 1).
  ffn        Q4_0 17408 x 5120, codes U{0..15}, fp16 scales lognormal(-5, 0.5),
             16 bf16 rows 0.5 * Student-t(3) with round(0.001 K) channels x 50.
  fp8        E4M3FN from clip(N(0, 1), +-448) rounded to nearest, fp32 tile
             scales U[1e-3, 1e-2], bf16 rows ~ N(0, 1).
  stream     per layer: Q4_0 8192x5120, 5120x8192, 17408x5120 (x2), 5120x17408,
             codes U{0..15}, fp16 scales U[0.001, 0.02], bf16 rows ~ N(0, 1).
  prefill    512 bf16 rows as in ``ffn``; Q4_0 17408 x 5120 as in ``ffn``.

Uniform Q4_0 codes are drawn as uniform random bytes: two independent uniform
nibbles per byte, so no layout knowledge is needed here.
"""
from __future__ import annotations

import numpy as np

# Shapes of one synthetic layer of the per-token weight stream: (out, in).
STREAM_LAYER_SHAPES = ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120), (5120, 17408))
STREAM_LAYERS = 64

CFG_TINY, CFG_FFN, CFG_FP8, CFG_STREAM, CFG_PREFILL = 1, 2, 3, 4, 5
T_CODES, T_WSCALES, T_ACT, T_OUTLIER, T_E4M3, T_TSCALES = 0, 1, 2, 3, 4, 5


def seed_of(config: int, layer: int, tensor_id: int) -> int:
    return 1_000_003 * config + 1009 * layer + tensor_id


def rng(config: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(config, layer, tensor_id)))


# ------------------------------------------------------------------ encodings

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(a) -> np.ndarray:
    """Round to IEEE binary16 with numpy (nearest, ties to even); return the bits."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_e4m3_bits(a) -> np.ndarray:
    """Round to OCP E4M3FN with torch's CPU conversion; return the bytes."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


# ------------------------------------------------------------------ draws

def q4_0_codes(M: int, K: int, g: np.random.Generator) -> np.ndarray:
    """Packed Q4_0 codes, u8 [M][K/2], every nibble uniform on 0..15."""
    return g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)


def fp16_scales_uniform(M: int, K: int, g, lo=0.001, hi=0.02) -> np.ndarray:
    return f32_to_f16_bits(g.uniform(lo, hi, size=(M, K // 32)))


def fp16_scales_lognormal(M: int, K: int, g, mu=-5.0, sigma=0.5) -> np.ndarray:
    return f32_to_f16_bits(g.lognormal(mu, sigma, size=(M, K // 32)))


def act_normal(N: int, K: int, g, dtype="bf16") -> np.ndarray:
    x = g.standard_normal(size=(N, K)).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else f32_to_f16_bits(x)


def act_student_outliers(N: int, K: int, g, g_out, nu=3.0, scale=0.5, frac=0.001, mult=50.0,
                         dtype="bf16") -> np.ndarray:
    """scale * Student-t(nu), with round(frac * K) distinct channels (columns) x mult."""
    x = (scale * g.standard_t(nu, size=(N, K))).astype(np.float32)
    n_out = int(round(frac * K))
    if n_out > 0:
        ch = g_out.choice(K, size=n_out, replace=False)
        x[:, ch] *= np.float32(mult)
    return f32_to_bf16_bits(x) if dtype == "bf16" else f32_to_f16_bits(x)


def e4m3_weights(M: int, K: int, g) -> np.ndarray:
    x = np.clip(g.standard_normal(size=(M, K)), -448.0, 448.0).astype(np.float32)
    return f32_to_e4m3_bits(x)


def fp8_tile_scales(M: int, K: int, g, lo=1e-3, hi=1e-2) -> np.ndarray:
    return g.uniform(lo, hi, size=((M + 127) // 128, K // 128)).astype(np.float32)


# ------------------------------------------------------------------ named workloads

def tiny(M=256, K=512, N=8):
    """Q4_0 256 x 512, fp16 activations and output."""
    c = CFG_TINY
    return dict(
        codes=q4_0_codes(M, K, rng(c, 0, T_CODES)),
        scales=fp16_scales_uniform(M, K, rng(c, 0, T_WSCALES)),
        act=act_normal(N, K, rng(c, 0, T_ACT), dtype="f16"),
        M=M, K=K, N=N, act_dtype="f16", out_dtype="f16")


def ffn(M=17408, K=5120, N=16):
    """Q4_0 at FFN shape; rows 0..N-1 of one seeded 16-row block."""
    c = CFG_FFN
    act = act_student_outliers(max(N, 16), K, rng(c, 0, T_ACT), rng(c, 0, T_OUTLIER))[:N]
    return dict(
        codes=q4_0_codes(M, K, rng(c, 0, T_CODES)),
        scales=fp16_scales_lognormal(M, K, rng(c, 0, T_WSCALES)),
        act=np.ascontiguousarray(act),
        M=M, K=K, N=N, act_dtype="bf16", out_dtype="bf16")


def fp8(M=5120, K=5120, N=16, layer=0):
    c = CFG_FP8
    act = act_normal(max(N, 16), K, rng(c, layer, T_ACT))[:N]
    return dict(
        w=e4m3_weights(M, K, rng(c, layer, T_E4M3)),
        tscales=fp8_tile_scales(M, K, rng(c, layer, T_TSCALES)),
        act=np.ascontiguousarray(act),
        M=M, K=K, N=N, act_dtype="bf16", out_dtype="bf16")


def stream_matrix(layer: int, idx: int):
    """One Q4_0 matrix of the per-token stream (numpy; use for sampled checks)."""
    M, K = STREAM_LAYER_SHAPES[idx]
    c = CFG_STREAM
    tid = 10 * idx
    return dict(
        codes=q4_0_codes(M, K, rng(c, layer, tid + T_CODES)),
        scales=fp16_scales_uniform(M, K, rng(c, layer, tid + T_WSCALES)),
        M=M, K=K)


def stream_act(layer: int, K: int, N=16):
    """The layer's 16-row bf16 activation block for inputs of width K."""
    return act_normal(N, K, rng(CFG_STREAM, layer, 1000 + K + T_ACT))


def prefill(M=17408, K=5120, N=512):
    c = CFG_PREFILL
    return dict(
        codes=q4_0_codes(M, K, rng(c, 0, T_CODES)),
        scales=fp16_scales_lognormal(M, K, rng(c, 0, T_WSCALES)),
        act=act_student_outliers(N, K, rng(c, 0, T_ACT), rng(c, 0, T_OUTLIER)),
        M=M, K=K, N=N, act_dtype="bf16", out_dtype="f32")


# ------------------------------------------------------------------ device-side draws

def q4_0_device(M: int, K: int, seed: int, device, scale_lo=0.001, scale_hi=0.02):
    """Large Q4_0 matrices drawn straight on the device with a seeded torch generator
    (same distributions as ``stream``).  Returns (codes u8 [M][K/2], scales f16 [M][K/32])."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=device, generator=g)
    scales = torch.empty((M, K // 32), dtype=torch.float32, device=device)
    scales.uniform_(scale_lo, scale_hi, generator=g)
    return codes, scales.to(torch.float16)


def act_device(N: int, K: int, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((N, K), dtype=torch.float32, device=device, generator=g)
    return x.to(torch.bfloat16)
