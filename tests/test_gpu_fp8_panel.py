"""FP8 E4M3 weights in the panel layout on the GPU, through the C ABI: the
repack writes the documented bytes, the panel GEMM matches the CPU oracle, and
it returns the bits of the row-major walk form with one tile per wave and
eight waves at the same workgroup cap."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu

REC = 131072
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def panel_bytes_reference(w, M, K):
    """The FP8 panel layout as include/vq.h defines it, built with numpy:
    records of 128 features x 8 steps of 128 k, 1 KiB per (step, tile, half)."""
    P, C = -(-M // 128), -(-K // 1024)
    pad = np.zeros((P * 128, C * 1024), np.uint8)
    pad[:M, :K] = w
    # feature = (p, t, j), k = (c, s, g, h, b)  ->  record order s, t, h, (g, j), b
    v = pad.reshape(P, 8, 16, C, 8, 4, 2, 16).transpose(0, 3, 4, 1, 6, 5, 2, 7)
    return np.ascontiguousarray(v).reshape(-1)


class Fp8Panel:
    """An E4M3 matrix resident on the device in both layouts."""

    def __init__(self, w, ts):
        self.w_np, self.ts_np = w, ts
        self.M, self.K = w.shape
        self.w = to_dev(w)
        self.ts = to_dev(ts)
        self.panel = vq.fp8_to_panel(self.w)
        torch.cuda.synchronize()

    def run(self, bits, act="bf16", out="bf16", **kw):
        x = to_dev(bits, TORCH_DT[act])
        y = torch.empty((x.shape[0], self.M), dtype=TORCH_DT[out], device="cuda")
        vq.gemm_fp8_blk128_panel(self.panel, self.ts, x, y, **kw)
        torch.cuda.synchronize()
        return y

    def run_row_major(self, bits, act="bf16", out="bf16", **kw):
        x = to_dev(bits, TORCH_DT[act])
        y = torch.empty((x.shape[0], self.M), dtype=TORCH_DT[out], device="cuda")
        vq.gemm_fp8_blk128(self.w, self.ts, x, y, **kw)
        torch.cuda.synchronize()
        return y

    def oracle(self, bits, dt=oracle.BF16, cols=None):
        return oracle.gemm_fp8_blk128(self.w_np, self.ts_np, bits, dt, bits.shape[0], self.M, self.K, cols=cols)


_WS = {}


def workspace():
    if "ws" not in _WS:
        _WS["ws"] = vq.Workspace(32 << 20)
    return _WS["ws"]


def _mat(M, K, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return Fp8Panel(W.e4m3_weights(M, K, g), W.fp8_tile_scales(M, K, g)), g


@pytest.mark.parametrize("M,K", [(128, 1024), (1, 128), (300, 1152), (129, 4096), (272, 1280)])
def test_repack_writes_the_documented_layout(M, K):
    p, _ = _mat(M, K, 501)
    assert p.panel.numel() == vq.fp8_panel_bytes(M, K)
    assert np.array_equal(p.panel.cpu().numpy(), panel_bytes_reference(p.w_np, M, K))


def test_repack_into_a_larger_buffer_leaves_the_rest():
    g = np.random.Generator(np.random.PCG64(502))
    M, K = 200, 640
    w = W.e4m3_weights(M, K, g)
    n = vq.fp8_panel_bytes(M, K)
    buf = torch.full((n + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    vq.fp8_to_panel(to_dev(w), buf)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.array_equal(host[:n], panel_bytes_reference(w, M, K))
    assert (host[n:] == 0xA5).all()


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (17, 384, 3), (300, 1280, 5), (272, 1152, 16),
                                   (129, 2176, 16), (1000, 5120, 16), (64, 256, 40)])
def test_ragged_shapes_parity(M, K, N):
    p, g = _mat(M, K, 503)
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    parity(out_to_f64(p.run(a)), p.oracle(a), "bf16")


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
def test_dtype_combinations_parity(act, out):
    p, g = _mat(272, 1024, 504)
    x = g.standard_normal((11, 1024))
    bits = W.f32_to_bf16_bits(x) if act == "bf16" else W.f32_to_f16_bits(x)
    dt = oracle.BF16 if act == "bf16" else oracle.F16
    parity(out_to_f64(p.run(bits, act, out)), p.oracle(bits, dt), out)


@pytest.mark.parametrize("groups", [0, 1, 2, 7, 40])
def test_group_caps_parity_and_exact_integers(groups):
    """Workgroup caps cut panels between workgroups in different places; with
    unit tile scales, small-integer weights and rows every sum is exact, so
    the output must equal the oracle bit for bit (checks the repacked order)."""
    M, K, N = 272, 3328, 16
    p, g = _mat(M, K, 505)
    a = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(N, K)))
    parity(out_to_f64(p.run(a, max_groups=groups, workspace=workspace())), p.oracle(a), "bf16")
    wi = W.f32_to_e4m3_bits(g.integers(-8, 9, size=(M, K)).astype(np.float32))
    pi = Fp8Panel(wi, np.ones(((M + 127) // 128, K // 128), np.float32))
    ai = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    y = out_to_f64(pi.run(ai, out="f32", max_groups=groups, workspace=workspace()))
    assert np.array_equal(y, pi.oracle(ai))


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_every_code_exact(act):
    """Each of the 254 finite E4M3 codes (subnormals included) read through
    one-hot rows with unit tile scales: Y = the code's value exactly."""
    M, K = 32, 256
    codes = np.arange(256, dtype=np.int64)
    codes = codes[(codes & 0x7F) != 0x7F]             # drop the two NaN codes
    w = np.zeros((M, K), dtype=np.uint8)
    w.reshape(-1)[:codes.size] = codes.astype(np.uint8)
    ones = np.ones((1, K // 128), dtype=np.float32)
    p = Fp8Panel(w, ones)
    ref = oracle.fp8_dequant(w, ones, M, K)
    for k0 in range(0, K, 16):
        x = np.zeros((16, K), dtype=np.float32)
        x[np.arange(16), k0 + np.arange(16)] = 1.0
        bits = W.f32_to_bf16_bits(x) if act == "bf16" else W.f32_to_f16_bits(x)
        y = out_to_f64(p.run(bits, act, "f32"))
        assert np.array_equal(y, ref[:, k0:k0 + 16].T), k0


def test_tile_scale_index_exact():
    """Distinct power-of-two scales per 128 x 128 tile, integer weights and
    rows: each step must pick up its own tile's scale."""
    g = np.random.Generator(np.random.PCG64(506))
    M, K, N = 300, 2304, 16
    wi = g.integers(-8, 9, size=(M, K)).astype(np.float32)
    ts = np.array([[2.0 ** -((3 * i + j) % 11) for j in range(K // 128)] for i in range((M + 127) // 128)],
                  dtype=np.float32)
    p = Fp8Panel(W.f32_to_e4m3_bits(wi), ts)
    a = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    assert np.array_equal(out_to_f64(p.run(a, out="f32")), p.oracle(a))


@pytest.mark.parametrize("M,K,groups", [(1000, 2048, 1), (400, 5120, 1), (300, 17408, 1), (400, 5120, 3),
                                         (1000, 5120, 7), (300, 17408, 40), (5120, 5120, 256)])
def test_same_bits_as_row_major_walk(M, K, groups):
    """The panel call performs the arithmetic of the row-major walk form with
    one tile per wave and eight waves (the same loads into the same
    registers, chunks of 8 steps): at the same workgroup cap both cut tile
    groups at the same k and return identical bits."""
    p, g = _mat(M, K, 507)
    a = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    ws = workspace()
    ref = p.run_row_major(a, tiles_per_wave=1, waves_per_group=8, max_groups=groups, workspace=ws)
    assert torch.equal(p.run(a, max_groups=groups, workspace=ws), ref)


@pytest.mark.parametrize("M,K,groups", [(17408, 5120, 0), (5120, 17408, 0), (8192, 5120, 80),
                                         (5120, 8192, 3)])
def test_stream_shapes_parity(M, K, groups):
    """The stream's matrix shapes at full size: sampled outputs within the bar
    of the oracle, tile groups cut between workgroups."""
    p, g = _mat(M, K, 508)
    a = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    cols = np.unique(np.concatenate([[0, 127, 128, M - 1], g.choice(M, 200, replace=False)]))
    parity(out_to_f64(p.run(a, max_groups=groups, workspace=workspace()))[:, cols], p.oracle(a, cols=cols),
           "bf16")


def test_rows_bit_identical_across_widths():
    f = W.fp8(M=17408, K=5120, N=16)
    p = Fp8Panel(f["w"], f["tscales"])
    x = f["act"]
    full = bits_u16(p.run(x))
    for n in range(16):
        assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(x[n:n + 1])))[0], full[n]), n
    for h in (0, 8):
        assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(x[h:h + 8]))), full[h:h + 8])
    perm = np.random.Generator(np.random.PCG64(509)).permutation(16)
    assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(x[perm]))), full[perm])
    junk = W.f32_to_bf16_bits(np.random.Generator(np.random.PCG64(510)).standard_normal((16, 5120)) * 30)
    junk[11] = x[2]
    assert np.array_equal(bits_u16(p.run(junk))[11], full[2])
    cols = np.unique(np.concatenate([[0, 17407], np.random.Generator(np.random.PCG64(511)).choice(17408, 300)]))
    parity(out_to_f64(p.run(x))[:, cols], p.oracle(x, cols=cols), "bf16")


def test_many_row_groups():
    p, g = _mat(200, 640, 512)
    a = W.f32_to_bf16_bits(g.standard_normal((50, 640)))
    y = p.run(a)
    parity(out_to_f64(y), p.oracle(a), "bf16")
    for r0 in (0, 16, 32):
        assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(a[r0:r0 + 16]))), bits_u16(y)[r0:r0 + 16])


def test_missing_workspace_rejected():
    p, g = _mat(64, 256, 513)
    x = to_dev(W.f32_to_bf16_bits(g.standard_normal((2, 256))), torch.bfloat16)
    y = torch.empty((2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vq.VqError) as e:
        vq.gemm_fp8_blk128_panel(p.panel, p.ts, x, y, workspace=vq.Workspace(64))
    assert e.value.status == vq.VQ_ERR_WORKSPACE


_LAYER = {}


def _layer():
    """One layer of the stream shapes in E4M3, both layouts on the device."""
    if "mats" not in _LAYER:
        g = np.random.Generator(np.random.PCG64(514))
        mats = []
        for M, K in W.STREAM_LAYER_SHAPES:
            p = Fp8Panel(W.e4m3_weights(M, K, g), W.fp8_tile_scales(M, K, g))
            bits = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
            mats.append((p, bits, to_dev(bits, torch.bfloat16)))
        _LAYER["mats"] = mats
    return _LAYER["mats"]


def _grouped(kind, mats, xs, ws):
    outs = [torch.empty((x.shape[0], p.M), dtype=torch.bfloat16, device="cuda") for (p, _, _), x in zip(mats, xs)]
    if kind == "fp8_panel":
        probs = [(p.panel, p.ts, x, o) for (p, _, _), x, o in zip(mats, xs, outs)]
    else:
        probs = [(p.w, p.ts, x, o) for (p, _, _), x, o in zip(mats, xs, outs)]
    vq.GroupedCall(kind, probs, workspace=ws)()
    torch.cuda.synchronize()
    return outs


def test_grouped_layer_parity():
    """One grouped call over the layer's five matrices: sampled outputs of
    both layouts within the bar of the oracle."""
    mats = _layer()
    ws = vq.Workspace(64 << 20)
    g = np.random.Generator(np.random.PCG64(515))
    for kind in ("fp8_panel", "fp8"):
        outs = _grouped(kind, mats, [x for _, _, x in mats], ws)
        for (p, bits, _), o in zip(mats, outs):
            cols = np.unique(np.concatenate([[0, 127, 128, p.M - 1], g.choice(p.M, 96, replace=False)]))
            parity(out_to_f64(o)[:, cols], p.oracle(bits, cols=cols), "bf16")


def _grouped_bits(mats, xs, ws):
    return [bits_u16(o) for o in _grouped("fp8_panel", mats, xs, ws)]


def test_grouped_layer_rows_bit_identical_at_every_width():
    """The benchmarked form (one grouped panel call over a layer's five
    matrices) at every width: each row at N = 1, both 8-row halves, a
    permuted block and a block whose other rows are junk return the bits of
    the 16-row call, for all five matrices."""
    mats = _layer()
    ws = vq.Workspace(64 << 20)
    g = np.random.Generator(np.random.PCG64(516))
    full = _grouped_bits(mats, [x for _, _, x in mats], ws)
    for r in range(16):
        one = _grouped_bits(mats, [x[r:r + 1].contiguous() for _, _, x in mats], ws)
        for i, (o, f) in enumerate(zip(one, full)):
            assert np.array_equal(o[0], f[r]), (i, r)
    for h in (0, 8):
        half = _grouped_bits(mats, [x[h:h + 8].contiguous() for _, _, x in mats], ws)
        for i, (o, f) in enumerate(zip(half, full)):
            assert np.array_equal(o, f[h:h + 8]), (i, h)
    perm = g.permutation(16)
    pt = torch.from_numpy(perm).cuda()
    per = _grouped_bits(mats, [x[pt].contiguous() for _, _, x in mats], ws)
    for i, (o, f) in enumerate(zip(per, full)):
        assert np.array_equal(o, f[perm]), i
    xs = []
    for _, _, x in mats:
        j = to_dev(W.f32_to_bf16_bits(40 * g.standard_normal((16, x.shape[1]))), torch.bfloat16)
        j[5] = x[12]
        xs.append(j)
    jk = _grouped_bits(mats, xs, ws)
    for i, (o, f) in enumerate(zip(jk, full)):
        assert np.array_equal(o[5], f[12]), i


@pytest.mark.parametrize("act,out", [("bf16", "bf16"), ("f16", "f32")])
def test_grouped_more_than_16_rows_and_ragged_widths(act, out):
    """A grouped call over ragged matrices with 37 rows (three groups of 16):
    every output within the bar of the oracle, and rows 16..31 equal to a
    16-row call on them."""
    g = np.random.Generator(np.random.PCG64(520))
    mats = [_mat(M, K, 521 + i)[0] for i, (M, K) in enumerate(((520, 4096), (130, 1152), (17, 384)))]
    xs = []
    for p in mats:
        x = g.standard_normal((37, p.K))
        xs.append(W.f32_to_bf16_bits(x) if act == "bf16" else W.f32_to_f16_bits(x))
    ws = vq.Workspace(16 << 20)

    def call(r0, r1):
        outs = [torch.empty((r1 - r0, p.M), dtype=TORCH_DT[out], device="cuda") for p in mats]
        vq.GroupedCall("fp8_panel", [(p.panel, p.ts, to_dev(np.ascontiguousarray(x[r0:r1]), TORCH_DT[act]), o)
                                     for p, x, o in zip(mats, xs, outs)], workspace=ws)()
        torch.cuda.synchronize()
        return outs
    full = call(0, 37)
    dt = oracle.BF16 if act == "bf16" else oracle.F16
    for p, x, y in zip(mats, xs, full):
        parity(out_to_f64(y), p.oracle(x, dt), out)
    for y, z in zip(full, call(16, 32)):
        assert torch.equal(z, y[16:32])


def test_grouped_graph_replays_match_eager():
    mats = []
    for i, (M, K) in enumerate(((2048, 5120), (1024, 8192), (520, 17408))):
        p, g = _mat(M, K, 517 + i)
        x = to_dev(W.f32_to_bf16_bits(g.standard_normal((16, K))), torch.bfloat16)
        mats.append((p, x, torch.empty((16, M), dtype=torch.bfloat16, device="cuda")))
    ws = vq.Workspace(64 << 20)
    call = vq.GroupedCall("fp8_panel", [(p.panel, p.ts, x, o) for p, x, o in mats], workspace=ws)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    eager = [o.clone() for _, _, o in mats]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call(s)
    for rep in range(4):
        for _, _, o in mats:
            o.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        for i, (_, _, o) in enumerate(mats):
            assert torch.equal(o, eager[i]), (rep, i)
        call()  # eager work on the same workspace between replays
        torch.cuda.synchronize()
    assert not ws.tensor[:65536].cpu().numpy().any()  # the counters are back at zero


@pytest.mark.parametrize("count", [9, 10, 14])
def test_grouped_many_problems_exact_integers(count):
    """Grouped calls of 9 problems (every first chunk among the kernel's
    preloaded arguments) and of 10 and 14 (the kernel reads the first chunks
    from the launch record): ragged matrices with unit tile scales,
    small-integer weights and rows, so every output equals the oracle bit for
    bit."""
    g = np.random.Generator(np.random.PCG64(530 + count))
    N = 5
    mats, outs = [], []
    for _ in range(count):
        M, K = int(g.integers(1, 400)), 128 * int(g.integers(1, 24))
        wi = W.f32_to_e4m3_bits(g.integers(-8, 9, size=(M, K)).astype(np.float32))
        p = Fp8Panel(wi, np.ones(((M + 127) // 128, K // 128), np.float32))
        bits = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)).astype(np.float32))
        mats.append((p, bits, to_dev(bits, torch.bfloat16)))
        outs.append(torch.empty((N, M), dtype=torch.float32, device="cuda"))
    vq.GroupedCall("fp8_panel", [(p.panel, p.ts, x, o) for (p, _, x), o in zip(mats, outs)],
                   workspace=vq.Workspace(64 << 20))()
    torch.cuda.synchronize()
    for i, ((p, bits, _), o) in enumerate(zip(mats, outs)):
        assert np.array_equal(out_to_f64(o), p.oracle(bits)), (i, p.M, p.K)
