"""Q4_0 weights in the panel layout on the GPU, through the C ABI: the repack
writes the documented bytes, the panel GEMM matches the CPU oracle, and
where no tile group is cut between workgroups it returns the same bits as the
row-major walk form."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import bits_u16, out_to_f64, parity, to_dev

pytestmark = pytest.mark.gpu

REC = 73728


def panel_bytes_reference(codes, scales, M, K):
    """The panel layout as include/vq.h defines it, built with numpy: records
    of 256 features x 4 steps of 128 k, codes then scales."""
    P, C, NB = -(-M // 256), -(-K // 512), K // 32
    cb = np.zeros((P * 256, C * 16, 16), np.uint8)
    cb[:M, :NB] = codes.reshape(M, NB, 16)
    sc = np.zeros((P * 256, C * 16), np.uint16)
    sc[:M, :NB] = scales
    out = np.zeros((P, C, REC), np.uint8)
    # axes: p, t, j | c, s, q | g, b  ->  record order s, t, (g, j), q, b
    cw = cb.reshape(P, 16, 16, C, 4, 4, 4, 4).transpose(0, 3, 4, 1, 6, 2, 5, 7)
    out[:, :, :65536] = cw.reshape(P, C, 65536)
    sw = np.ascontiguousarray(sc.reshape(P, 16, 16, C, 16).transpose(0, 3, 1, 2, 4))
    out[:, :, 65536:] = sw.reshape(P, C, 4096).view(np.uint8)
    return out.reshape(-1)


class Panel:
    """A Q4_0 matrix resident on the device in both layouts."""

    def __init__(self, codes, scales):
        self.codes_np, self.scales_np = codes, scales
        self.M, self.K = codes.shape[0], codes.shape[1] * 2
        self.codes = to_dev(codes)
        self.scales = to_dev(scales, torch.float16)
        self.panel = vq.q4_0_to_panel(self.codes, self.scales)
        torch.cuda.synchronize()

    def run(self, bits, act=torch.bfloat16, out=torch.bfloat16, **kw):
        x = to_dev(bits, act)
        y = torch.empty((x.shape[0], self.M), dtype=out, device="cuda")
        vq.gemm_q4_0_panel(self.panel, self.M, self.K, x, y, **kw)
        torch.cuda.synchronize()
        return y

    def run_row_major(self, bits, act=torch.bfloat16, out=torch.bfloat16, **kw):
        x = to_dev(bits, act)
        y = torch.empty((x.shape[0], self.M), dtype=out, device="cuda")
        vq.gemm_q4_0(self.codes, self.scales, x, y, **kw)
        torch.cuda.synchronize()
        return y

    def oracle(self, bits, dt=oracle.BF16, cols=None):
        return oracle.gemm_q4_0(self.codes_np, self.scales_np, bits, dt, bits.shape[0], self.M, self.K, cols=cols)


_WS = {}


def workspace():
    if "ws" not in _WS:
        _WS["ws"] = vq.Workspace(32 << 20)
    return _WS["ws"]


@pytest.mark.parametrize("M,K", [(272, 1056), (128, 1024), (1, 32), (300, 2080), (129, 4096)])
def test_repack_writes_the_documented_layout(M, K):
    g = np.random.Generator(np.random.PCG64(401))
    codes, scales = W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g)
    p = Panel(codes, scales)
    assert p.panel.numel() == vq.q4_0_panel_bytes(M, K)
    assert np.array_equal(p.panel.cpu().numpy(), panel_bytes_reference(codes, scales, M, K))


def test_repack_into_a_larger_buffer_leaves_the_rest():
    g = np.random.Generator(np.random.PCG64(402))
    M, K = 200, 640
    codes, scales = W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g)
    n = vq.q4_0_panel_bytes(M, K)
    buf = torch.full((n + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    vq.q4_0_to_panel(to_dev(codes), to_dev(scales, torch.float16), buf)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.array_equal(host[:n], panel_bytes_reference(codes, scales, M, K))
    assert (host[n:] == 0xA5).all()


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (17, 96, 3), (300, 480, 5), (272, 1056, 16), (129, 2080, 16),
                                   (1000, 5120, 16), (64, 160, 40)])
def test_ragged_shapes_parity(M, K, N):
    g = np.random.Generator(np.random.PCG64(403))
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    parity(out_to_f64(p.run(a)), p.oracle(a), "bf16")


@pytest.mark.parametrize("act", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float16, torch.float32])
def test_dtype_combinations_parity(act, out):
    g = np.random.Generator(np.random.PCG64(404))
    M, K, N = 272, 1024, 11
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    x = g.standard_normal((N, K))
    bits = W.f32_to_bf16_bits(x) if act == torch.bfloat16 else W.f32_to_f16_bits(x)
    dt = oracle.BF16 if act == torch.bfloat16 else oracle.F16
    name = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[out]
    parity(out_to_f64(p.run(bits, act, out)), p.oracle(bits, dt), name)


@pytest.mark.parametrize("groups", [0, 1, 2, 7, 40])
def test_group_caps_parity_and_exact_integers(groups):
    """Workgroup caps cut panels between workgroups in different places; with
    unit scales and small-integer rows every sum is exact, so the output must
    equal the oracle bit for bit (checks the repacked code order)."""
    g = np.random.Generator(np.random.PCG64(405))
    M, K, N = 272, 3328, 16
    codes = W.q4_0_codes(M, K, g)
    p = Panel(codes, W.fp16_scales_lognormal(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    parity(out_to_f64(p.run(a, max_groups=groups, workspace=workspace())), p.oracle(a), "bf16")
    pi = Panel(codes, np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    ai = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    y = out_to_f64(pi.run(ai, out=torch.float32, max_groups=groups, workspace=workspace()))
    assert np.array_equal(y, pi.oracle(ai))


def test_one_hot_unpack_every_code():
    """Row n of X = e_k gives q[m][k] - 8 exactly: 16 calls cover every code."""
    g = np.random.Generator(np.random.PCG64(406))
    M, K = 160, 256
    ones = np.full((M, K // 32), 0x3C00, dtype=np.uint16)
    codes = W.q4_0_codes(M, K, g)
    p = Panel(codes, ones)
    ref = oracle.q4_0_dequant(codes, ones, M, K)
    for k0 in range(0, K, 16):
        x = np.zeros((16, K), dtype=np.float32)
        x[np.arange(16), k0 + np.arange(16)] = 1.0
        y = out_to_f64(p.run(W.f32_to_bf16_bits(x), out=torch.float32))
        assert np.array_equal(y, ref[:, k0:k0 + 16].T), k0


def test_block_scales_bit_exact():
    """Distinct power-of-two scales per block with integer rows: each block must
    pick up its own scale from the record's scale rows."""
    g = np.random.Generator(np.random.PCG64(407))
    M, K, N = 200, 2304, 16
    e = g.integers(-6, 3, size=(M, K // 32))
    scales = ((15 + e) << 10).astype(np.uint16)        # fp16 2^e
    p = Panel(W.q4_0_codes(M, K, g), scales)
    a = W.f32_to_bf16_bits(g.integers(-3, 4, size=(N, K)))
    assert np.array_equal(out_to_f64(p.run(a, out=torch.float32)), p.oracle(a))


@pytest.mark.parametrize("M,K", [(1000, 2048), (400, 5120), (300, 17408)])
def test_same_bits_as_row_major_walk_when_uncut(M, K):
    """With one workgroup no tile group is cut, and the panel call performs the
    row-major walk's arithmetic (per block: the offset MFMA, the block MFMA,
    one FMA with the block scale, blocks in order): identical bits."""
    g = np.random.Generator(np.random.PCG64(408))
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    a = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    ws = workspace()
    ref = p.run_row_major(a, tiles_per_wave=1, waves_per_group=8, max_groups=1, workspace=ws)
    assert torch.equal(p.run(a, max_groups=1, workspace=ws), ref)


@pytest.mark.parametrize("M,K,groups", [(400, 5120, 3), (17408, 5120, 0), (300, 17408, 40),
                                         (1000, 5120, 3), (17408, 5120, 80), (300, 17408, 5)])
def test_cut_tile_groups_parity(M, K, groups):
    """Workgroups cut tile groups at chunk boundaries (4 steps of 128 k in the
    panel layout, 8 row-major), with shares from 1.7 to 13.6 chunks: both
    layouts within the bar of the oracle."""
    g = np.random.Generator(np.random.PCG64(409))
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    a = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    ws = workspace()
    cols = np.unique(np.concatenate([[0, M - 1], g.choice(M, min(M, 200), replace=False)]))
    ref = p.oracle(a, cols=cols)
    parity(out_to_f64(p.run(a, max_groups=groups, workspace=ws))[:, cols], ref, "bf16")
    parity(out_to_f64(p.run_row_major(a, max_groups=groups, workspace=ws))[:, cols], ref, "bf16")


def test_rows_bit_identical_across_widths():
    g = np.random.Generator(np.random.PCG64(409))
    M, K = 17408, 5120
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    full = bits_u16(p.run(x))
    for n in (0, 7, 15):
        assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(x[n:n + 1])))[0], full[n])
    assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(x[3:11]))), full[3:11])
    cols = np.unique(np.concatenate([[0, M - 1], g.choice(M, 200, replace=False)]))
    parity(out_to_f64(p.run(x))[:, cols], p.oracle(x, cols=cols), "bf16")


def test_many_row_groups():
    g = np.random.Generator(np.random.PCG64(410))
    M, K, N = 200, 640, 50
    p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    y = p.run(a)
    parity(out_to_f64(y), p.oracle(a), "bf16")
    for r0 in (0, 16, 32):
        assert np.array_equal(bits_u16(p.run(np.ascontiguousarray(a[r0:r0 + 16]))), bits_u16(y)[r0:r0 + 16])


def test_missing_workspace_rejected():
    g = np.random.Generator(np.random.PCG64(411))
    p = Panel(W.q4_0_codes(64, 256, g), W.fp16_scales_uniform(64, 256, g))
    x = to_dev(W.f32_to_bf16_bits(g.standard_normal((2, 256))), torch.bfloat16)
    y = torch.empty((2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vq.VqError) as e:
        vq.gemm_q4_0_panel(p.panel, 64, 256, x, y, workspace=vq.Workspace(64))
    assert e.value.status == vq.VQ_ERR_WORKSPACE


def _layer(g, N=16):
    mats = []
    for M, K in W.STREAM_LAYER_SHAPES:
        codes, scales = W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g)
        bits = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(N, K)))
        p = Panel(codes, scales)
        x = to_dev(bits, torch.bfloat16)
        mats.append((p, bits, x))
    return mats


def test_grouped_layer_parity_and_rows_invariant():
    """One layer of the stream shapes in one grouped call, in both layouts:
    sampled outputs against the oracle; rows invariant to N."""
    g = np.random.Generator(np.random.PCG64(412))
    mats = _layer(g)
    ws = vq.Workspace(64 << 20)
    outs_p = [torch.empty((16, p.M), dtype=torch.bfloat16, device="cuda") for p, _, _ in mats]
    outs_r = [torch.empty_like(o) for o in outs_p]
    vq.GroupedCall("q4_0_panel", [(p.panel, p.M, x, o) for (p, _, x), o in zip(mats, outs_p)], workspace=ws)()
    vq.GroupedCall("q4_0", [(p.codes, p.scales, x, o) for (p, _, x), o in zip(mats, outs_r)], workspace=ws)()
    torch.cuda.synchronize()
    for (p, bits, _), yp, yr in zip(mats, outs_p, outs_r):
        cols = np.unique(np.concatenate([[0, p.M - 1], g.choice(p.M, 96, replace=False)]))
        ref = p.oracle(bits, cols=cols)
        parity(out_to_f64(yp)[:, cols], ref, "bf16")
        parity(out_to_f64(yr)[:, cols], ref, "bf16")
    sub = [torch.empty((1, p.M), dtype=torch.bfloat16, device="cuda") for p, _, _ in mats]
    vq.GroupedCall("q4_0_panel", [(p.panel, p.M, x[6:7].contiguous(), o) for (p, _, x), o in zip(mats, sub)],
                   workspace=ws)()
    torch.cuda.synchronize()
    for o, yp in zip(sub, outs_p):
        assert torch.equal(o[0], yp[6])


def _grouped(kind, mats, xs, ws):
    """One grouped call over the layer's matrices with activations xs[i]."""
    outs = [torch.empty((x.shape[0], p.M), dtype=torch.bfloat16, device="cuda") for (p, _, _), x in zip(mats, xs)]
    if kind == "q4_0_panel":
        probs = [(p.panel, p.M, x, o) for (p, _, _), x, o in zip(mats, xs, outs)]
    else:
        probs = [(p.codes, p.scales, x, o) for (p, _, _), x, o in zip(mats, xs, outs)]
    vq.GroupedCall(kind, probs, workspace=ws)()
    torch.cuda.synchronize()
    return [bits_u16(o) for o in outs]


@pytest.mark.parametrize("kind", ["q4_0_panel", "q4_0"])
def test_grouped_layer_rows_bit_identical_at_every_width(kind):
    """The benchmarked form (one grouped call over a layer's five stream
    matrices) at every width: each row at N = 1, both 8-row halves, a permuted
    block and blocks whose other rows are junk return the bits of the 16-row
    call, for all five matrices."""
    g = np.random.Generator(np.random.PCG64(414))
    mats = _layer(g)
    ws = vq.Workspace(64 << 20)
    full = _grouped(kind, mats, [x for _, _, x in mats], ws)
    for r in range(16):
        one = _grouped(kind, mats, [x[r:r + 1].contiguous() for _, _, x in mats], ws)
        for i, (o, f) in enumerate(zip(one, full)):
            assert np.array_equal(o[0], f[r]), (kind, i, r)
    for h in (0, 8):
        half = _grouped(kind, mats, [x[h:h + 8].contiguous() for _, _, x in mats], ws)
        for i, (o, f) in enumerate(zip(half, full)):
            assert np.array_equal(o, f[h:h + 8]), (kind, i, h)
    perm = g.permutation(16)
    pt = torch.from_numpy(perm).cuda()
    per = _grouped(kind, mats, [x[pt].contiguous() for _, _, x in mats], ws)
    for i, (o, f) in enumerate(zip(per, full)):
        assert np.array_equal(o, f[perm]), (kind, i)
    for tgt, pos in ((0, 15), (9, 4)):
        xs = []
        for _, bits, x in mats:
            j = to_dev(W.f32_to_bf16_bits(40 * g.standard_normal((16, x.shape[1]))), torch.bfloat16)
            j[pos] = x[tgt]
            xs.append(j)
        jk = _grouped(kind, mats, xs, ws)
        for i, (o, f) in enumerate(zip(jk, full)):
            assert np.array_equal(o[pos], f[tgt]), (kind, i, tgt)


def test_grouped_graph_replays_match_eager():
    g = np.random.Generator(np.random.PCG64(413))
    mats = []
    for M, K in ((2048, 5120), (1024, 8192), (520, 17408)):
        p = Panel(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
        x = to_dev(W.f32_to_bf16_bits(g.standard_normal((16, K))), torch.bfloat16)
        mats.append((p, x, torch.empty((16, M), dtype=torch.bfloat16, device="cuda")))
    ws = vq.Workspace(64 << 20)
    call = vq.GroupedCall("q4_0_panel", [(p.panel, p.M, x, o) for p, x, o in mats], workspace=ws)
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
    from the launch record): ragged matrices with unit scales and small-integer
    rows, so every output equals the oracle bit for bit, wherever the
    workgroups' ranges cut the tile groups."""
    g = np.random.Generator(np.random.PCG64(430 + count))
    N = 7
    mats, outs = [], []
    for _ in range(count):
        M, K = int(g.integers(1, 700)), 32 * int(g.integers(1, 100))
        p = Panel(W.q4_0_codes(M, K, g), np.full((M, K // 32), 0x3C00, dtype=np.uint16))
        bits = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)).astype(np.float32))
        mats.append((p, bits, to_dev(bits, torch.bfloat16)))
        outs.append(torch.empty((N, M), dtype=torch.float32, device="cuda"))
    vq.GroupedCall("q4_0_panel", [(p.panel, p.M, x, o) for (p, _, x), o in zip(mats, outs)],
                   workspace=vq.Workspace(64 << 20))()
    torch.cuda.synchronize()
    for i, ((p, bits, _), o) in enumerate(zip(mats, outs)):
        assert np.array_equal(out_to_f64(o), p.oracle(bits)), (i, p.M, p.K)
