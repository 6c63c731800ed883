"""FP8 E4M3 block-scaled verify GEMM on the GPU, against the CPU oracle."""
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


class FP8:
    def __init__(self, w, ts):
        self.w_np, self.ts_np = w, ts
        self.M, self.K = w.shape
        self.w = to_dev(w)
        self.ts = to_dev(ts)

    def run(self, act_bits, act_dtype="bf16", out_dtype="bf16", **kw):
        x = to_dev(act_bits, TORCH_DT[act_dtype])
        out = torch.empty((x.shape[0], self.M), dtype=TORCH_DT[out_dtype], device="cuda")
        vq.gemm_fp8_blk128(self.w, self.ts, x, out, **kw)
        torch.cuda.synchronize()
        return out

    def oracle(self, act_bits, act_dtype="bf16", cols=None):
        return oracle.gemm_fp8_blk128(self.w_np, self.ts_np, act_bits, ORACLE_DT[act_dtype],
                                      act_bits.shape[0], self.M, self.K, cols=cols)


@pytest.mark.parametrize("M", [5120, 17408])
@pytest.mark.parametrize("n_rows", [1, 4, 16])
def test_fp8_config_parity_sampled(M, n_rows):
    f = W.fp8(M=M, K=5120, N=16)
    q = FP8(f["w"], f["tscales"])
    a = np.ascontiguousarray(f["act"][:n_rows])
    y = out_to_f64(q.run(a))
    g = np.random.Generator(np.random.PCG64(M + n_rows))
    cols = np.unique(np.concatenate([[0, 127, 128, M - 1], g.choice(M, 512, replace=False)]))
    fro, worst, ulps = parity(y[:, cols], q.oracle(a, cols=cols), "bf16")
    print("fp8 %dx5120 N=%d: relF %.3e worst %.3e max %.2f ulp" % (M, n_rows, fro, worst, ulps))


@pytest.mark.parametrize("act_dtype", ["bf16", "f16"])
def test_fp8_every_code_exact(act_dtype):
    """Each of the 254 finite E4M3 codes (subnormals included) read through
    one-hot activations with unit tile scales: Y = e4m3 value exactly."""
    M, K = 32, 256
    codes = np.arange(256, dtype=np.int64)
    codes = codes[(codes & 0x7F) != 0x7F]             # drop the two NaN codes
    w = np.zeros((M, K), dtype=np.uint8)
    w.reshape(-1)[:codes.size] = codes.astype(np.uint8)
    q = FP8(w, np.ones((1, K // 128), dtype=np.float32))
    ref = oracle.fp8_dequant(w, np.ones((1, K // 128), dtype=np.float32), M, K)
    for k0 in range(0, K, 16):
        x = np.zeros((16, K), dtype=np.float32)
        x[np.arange(16), k0 + np.arange(16)] = 1.0
        bits = W.f32_to_bf16_bits(x) if act_dtype == "bf16" else W.f32_to_f16_bits(x)
        y = out_to_f64(q.run(bits, act_dtype, "f32"))
        assert np.array_equal(y, ref[:, k0:k0 + 16].T), k0


def test_fp8_tile_scale_index_exact():
    g = np.random.Generator(np.random.PCG64(201))
    M, K, N = 300, 384, 16
    wi = g.integers(-8, 9, size=(M, K)).astype(np.float32)
    ts = np.array([[2.0 ** -(3 * i + j) for j in range(K // 128)] for i in range((M + 127) // 128)],
                  dtype=np.float32)
    q = FP8(W.f32_to_e4m3_bits(wi), ts)
    a = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    assert np.array_equal(out_to_f64(q.run(a, "bf16", "f32")), q.oracle(a))


@pytest.mark.parametrize("M", [5120, 17408])
def test_fp8_rows_bit_identical_across_widths(M):
    """Both FP8 workload shapes: every row at N = 1, the 4-row and 8-row
    blocks, a permuted block and junk neighbours give the 16-row call's bits."""
    f = W.fp8(M=M, K=5120, N=16)
    q = FP8(f["w"], f["tscales"])
    x = f["act"]
    full = bits_u16(q.run(x))
    for n in range(16):
        assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[n:n + 1])))[0], full[n]), n
    assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[4:8]))), full[4:8])
    for h in (0, 8):
        assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[h:h + 8]))), full[h:h + 8])
    perm = np.random.Generator(np.random.PCG64(M)).permutation(16)
    assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[perm]))), full[perm])
    junk = W.f32_to_bf16_bits(np.random.Generator(np.random.PCG64(M + 1)).standard_normal((16, 5120)) * 30)
    junk[11] = x[2]
    assert np.array_equal(bits_u16(q.run(junk))[11], full[2])
    assert np.array_equal(bits_u16(q.run(x)), full)
    if M == 17408:
        cols = np.unique(np.concatenate([[0, M - 1], np.random.Generator(np.random.PCG64(3)).choice(M, 300)]))
        parity(out_to_f64(q.run(x))[:, cols], q.oracle(x, cols=cols), "bf16")


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (300, 384, 5), (130, 1280, 33)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_fp8_ragged_parity(M, K, N, out_dtype):
    f = W.fp8(M=M, K=K, N=N)
    q = FP8(f["w"], f["tscales"])
    parity(out_to_f64(q.run(f["act"], "bf16", out_dtype)), q.oracle(f["act"]), out_dtype)


_WS = {}


def big_workspace():
    if "ws" not in _WS:
        _WS["ws"] = vq.Workspace(32 << 20)
    return _WS["ws"]


@pytest.mark.parametrize("tpw", [1, 2, 4])
@pytest.mark.parametrize("wpg", [2, 4, 8])
@pytest.mark.parametrize("groups", [0, 1, 3])
def test_fp8_walk_shapes(tpw, wpg, groups):
    """17 tiles (three 128-row scale tiles, the last partial), 10 steps of K
    (two chunks), every tile/wave shape, tile groups cut between workgroups."""
    f = W.fp8(M=272, K=1280, N=16)
    q = FP8(f["w"], f["tscales"])
    kw = dict(tiles_per_wave=tpw, waves_per_group=wpg, max_groups=groups, workspace=big_workspace())
    parity(out_to_f64(q.run(f["act"], **kw)), q.oracle(f["act"]), "bf16")


@pytest.mark.parametrize("groups", [4, 5])
def test_fp8_walk_long_shares(groups):
    """45 chunks over 4 or 5 workgroups (11.25 and 9 per share): tile groups
    of 5 chunks cut by range edges at several places."""
    f = W.fp8(M=272, K=5120, N=16)
    q = FP8(f["w"], f["tscales"])
    kw = dict(tiles_per_wave=1, waves_per_group=2, max_groups=groups, workspace=big_workspace())
    parity(out_to_f64(q.run(f["act"], **kw)), q.oracle(f["act"]), "bf16")


@pytest.mark.parametrize("tpw", [1, 2, 4])
@pytest.mark.parametrize("wpg", [2, 4, 8])
def test_fp8_one_shot_shapes(tpw, wpg):
    """The same problem in the one-shot form, several LDS chunks per tile group."""
    f = W.fp8(M=272, K=1280, N=16)
    q = FP8(f["w"], f["tscales"])
    kw = dict(tiles_per_wave=tpw, waves_per_group=wpg, workspace=None)
    parity(out_to_f64(q.run(f["act"], **kw)), q.oracle(f["act"]), "bf16")


def test_fp8_without_workspace():
    f = W.fp8(M=1000, K=2560, N=16)
    q = FP8(f["w"], f["tscales"])
    y = q.run(f["act"], workspace=None)
    parity(out_to_f64(y), q.oracle(f["act"]), "bf16")
    one = bits_u16(q.run(np.ascontiguousarray(f["act"][9:10]), workspace=None))
    assert np.array_equal(one[0], bits_u16(y)[9])
