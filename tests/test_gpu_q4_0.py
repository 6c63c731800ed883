"""Q4_0 verify GEMM on the GPU, through the C ABI, against the CPU oracle."""
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


def _to_act_bits(x, act_dtype):
    return W.f32_to_bf16_bits(x) if act_dtype == "bf16" else W.f32_to_f16_bits(x)


class Q4:
    """A Q4_0 weight matrix resident on the device."""

    def __init__(self, codes, scales):
        self.codes_np, self.scales_np = codes, scales
        self.M, self.K = codes.shape[0], codes.shape[1] * 2
        self.codes = to_dev(codes)
        self.scales = to_dev(scales, torch.float16)

    def run(self, act_bits, act_dtype="bf16", out_dtype="bf16", alpha=1.0, **kw):
        x = to_dev(act_bits, TORCH_DT[act_dtype])
        out = torch.empty((x.shape[0], self.M), dtype=TORCH_DT[out_dtype], device="cuda")
        vq.gemm_q4_0(self.codes, self.scales, x, out, alpha=alpha, **kw)
        torch.cuda.synchronize()
        return out

    def oracle(self, act_bits, act_dtype="bf16", cols=None, alpha=1.0):
        N = act_bits.shape[0]
        return oracle.gemm_q4_0(self.codes_np, self.scales_np, act_bits, ORACLE_DT[act_dtype],
                                N, self.M, self.K, cols=cols, alpha=alpha)


def _sample_cols(M, n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    edge = np.array([0, 1, 15, 16, M // 2, M - 17, M - 16, M - 1])
    return np.unique(np.concatenate([edge[(edge >= 0) & (edge < M)], g.choice(M, size=min(n, M), replace=False)]))


# ------------------------------------------------------------------ parity


def test_tiny_config_parity():
    t = W.tiny()
    q = Q4(t["codes"], t["scales"])
    y = q.run(t["act"], "f16", "f16")
    ref = q.oracle(t["act"], "f16")
    fro, worst, ulps = parity(out_to_f64(y), ref, "f16")
    print("tiny: relF %.3e worst %.3e max %.2f ulp" % (fro, worst, ulps))


@pytest.fixture(scope="module")
def ffn():
    t = W.ffn(N=16)
    return Q4(t["codes"], t["scales"]), t["act"]


@pytest.mark.parametrize("n_rows", [1, 8, 16])
def test_ffn_config_parity_sampled(ffn, n_rows):
    q, act = ffn
    a = np.ascontiguousarray(act[:n_rows])
    y = out_to_f64(q.run(a))
    cols = _sample_cols(q.M, 768, 5 + n_rows)
    fro, worst, ulps = parity(y[:, cols], q.oracle(a, cols=cols), "bf16")
    print("ffn N=%d: relF %.3e worst %.3e max %.2f ulp" % (n_rows, fro, worst, ulps))


def test_ffn_f16_outlier_rows_f32_out():
    """fp16 activations with the FFN rows' heavy tails and x50 outlier channels,
    fp32 outputs.  The block MFMA adds sum x (1024 + q) and -1032 sum x, two
    terms about 130 times the block dot that mostly cancel, so fp32 rounding
    is amplified by about that factor for fp16 rows (17 for bf16, whose codes
    are 128 + q); the 1 ulp + 1e-4 rms per-element check measures it."""
    t = W.ffn(N=16)
    q = Q4(t["codes"], t["scales"])
    g = W.rng(W.CFG_FFN, 0, W.T_ACT)
    a = W.act_student_outliers(16, q.K, g, W.rng(W.CFG_FFN, 0, W.T_OUTLIER), dtype="f16")
    y = out_to_f64(q.run(a, "f16", "f32"))
    cols = _sample_cols(q.M, 512, 17)
    fro, worst, ulps = parity(y[:, cols], q.oracle(a, "f16", cols=cols), "f32")
    print("ffn f16 rows, f32 out: relF %.3e worst %.3e max %.2f ulp" % (fro, worst, ulps))


def test_auto_workspace_on_a_fresh_side_stream():
    """workspace="auto" on a stream other than torch's current one, from an
    empty cache, then grown by a larger shape on the same stream: the zero fill
    is complete before the first call, and results match the oracle."""
    g = np.random.Generator(np.random.PCG64(118))
    vq._auto_ws.clear()
    s = torch.cuda.Stream()
    for M, K in ((520, 2048), (4100, 5120)):
        q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
        a = W.f32_to_bf16_bits(g.standard_normal((16, K)))
        x = to_dev(a, torch.bfloat16)
        out = torch.empty((16, M), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        vq.gemm_q4_0(q.codes, q.scales, x, out, stream=s)
        s.synchronize()
        parity(out_to_f64(out), q.oracle(a), "bf16")
    key = [k for k in vq._auto_ws if k[1] == s.cuda_stream]
    assert key and not vq._auto_ws[key[0]].tensor[:65536].cpu().numpy().any()


@pytest.mark.parametrize("act_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_dtype_combinations_parity(act_dtype, out_dtype):
    g = np.random.Generator(np.random.PCG64(101))
    M, K, N = 272, 1024, 11
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    a = _to_act_bits(g.standard_normal((N, K)), act_dtype)
    parity(out_to_f64(q.run(a, act_dtype, out_dtype)), q.oracle(a, act_dtype), out_dtype)


# ------------------------------------------------------------------ bit-exact probes


@pytest.mark.parametrize("act_dtype", ["bf16", "f16"])
def test_integer_case_bit_exact(act_dtype):
    """Unit scales and small-integer activations: every partial sum is an integer
    below 2^24, so the fp32 output must equal the exact oracle bit for bit."""
    g = np.random.Generator(np.random.PCG64(102))
    M, K, N = 160, 2048, 16
    q = Q4(W.q4_0_codes(M, K, g), np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    a = _to_act_bits(g.integers(-4, 5, size=(N, K)), act_dtype)
    y = out_to_f64(q.run(a, act_dtype, "f32"))
    assert np.array_equal(y, q.oracle(a, act_dtype))


@pytest.mark.parametrize("act_dtype", ["bf16", "f16"])
def test_one_hot_unpack_every_code(act_dtype):
    """Row n of X = e_k: Y[n][m] = q[m][k] - 8 exactly.  K/16 calls cover every
    code of the matrix (code unpacking must be bit-exact)."""
    t = W.tiny()
    M, K = t["M"], t["K"]
    q = Q4(t["codes"], np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    ref = oracle.q4_0_dequant(t["codes"], np.full((M, K // 32), 0x3C00, dtype=np.uint16), M, K)
    for k0 in range(0, K, 16):
        x = np.zeros((16, K), dtype=np.float32)
        x[np.arange(16), k0 + np.arange(16)] = 1.0
        y = out_to_f64(q.run(_to_act_bits(x, act_dtype), act_dtype, "f32"))
        assert np.array_equal(y, ref[:, k0:k0 + 16].T), k0


def test_block_scales_bit_exact():
    """Distinct power-of-two block scales with integer activations: checks that
    every block picks up its own scale (exact in fp32)."""
    g = np.random.Generator(np.random.PCG64(103))
    M, K, N = 48, 512, 16
    sc = np.array([[2.0 ** -((m + b) % 9) for b in range(K // 32)] for m in range(M)])
    q = Q4(W.q4_0_codes(M, K, g), W.f32_to_f16_bits(sc))
    a = W.f32_to_bf16_bits(g.integers(-3, 4, size=(N, K)))
    assert np.array_equal(out_to_f64(q.run(a, "bf16", "f32")), q.oracle(a))


def test_alpha_power_of_two_is_exact():
    t = W.tiny()
    q = Q4(t["codes"], t["scales"])
    y1 = q.run(t["act"], "f16", "f32").cpu().numpy()
    y4 = q.run(t["act"], "f16", "f32", alpha=0.25).cpu().numpy()
    assert np.array_equal(y4, y1 * np.float32(0.25))


# ------------------------------------------------------------------ width invariance


@pytest.mark.parametrize("act_dtype,shape", [("bf16", (17408, 5120)), ("f16", (256, 512)),
                                              ("bf16", (5120, 17408)), ("bf16", (300, 480))])
def test_rows_bit_identical_across_widths(act_dtype, shape):
    """Each output row is bit-identical whether the call has 1, 8 or 16 rows,
    under row permutation and with junk neighbours (the pages compare verify
    outputs byte for byte across draft widths)."""
    M, K = shape
    g = np.random.Generator(np.random.PCG64(104))
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = _to_act_bits(0.5 * g.standard_t(3, size=(16, K)), act_dtype)
    full = bits_u16(q.run(x, act_dtype, "bf16"))
    for h in (0, 8):
        eight = bits_u16(q.run(np.ascontiguousarray(x[h:h + 8]), act_dtype, "bf16"))
        assert np.array_equal(eight, full[h:h + 8])
    for n in range(16):
        one = bits_u16(q.run(np.ascontiguousarray(x[n:n + 1]), act_dtype, "bf16"))
        assert np.array_equal(one[0], full[n]), n
    perm = g.permutation(16)
    permuted = bits_u16(q.run(np.ascontiguousarray(x[perm]), act_dtype, "bf16"))
    assert np.array_equal(permuted, full[perm])
    junk = _to_act_bits(100.0 * g.standard_normal((16, K)), act_dtype)
    junk[5] = x[5]
    assert np.array_equal(bits_u16(q.run(junk, act_dtype, "bf16"))[5], full[5])


def test_repeat_calls_bit_identical(ffn):
    q, act = ffn
    first = bits_u16(q.run(act))
    for _ in range(3):
        assert np.array_equal(bits_u16(q.run(act)), first)


# ------------------------------------------------------------------ edges and launch shapes


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (17, 96, 3), (300, 480, 5), (64, 160, 40),
                                   (33, 4128, 17), (4096, 32, 16), (16, 8192, 2)])
def test_ragged_shapes_parity(M, K, N):
    g = np.random.Generator(np.random.PCG64(M * 7 + K + N))
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    parity(out_to_f64(q.run(a)), q.oracle(a), "bf16")


_WS = {}


def big_workspace():
    """One 32 MiB workspace shared by the explicit-shape tests (calls are
    ordered on one stream, so sharing it is allowed)."""
    if "ws" not in _WS:
        _WS["ws"] = vq.Workspace(32 << 20)
    return _WS["ws"]


@pytest.mark.parametrize("tpw", [1, 2, 4])
@pytest.mark.parametrize("wpg", [2, 4, 8])
@pytest.mark.parametrize("groups", [0, 1, 2, 7])
def test_every_walk_shape_parity_and_exact_integers(tpw, wpg, groups):
    """17 tiles (partial tile groups) and 10 steps (two chunks, the second of
    2 steps), every tile/wave shape, and workgroup caps that cut tile groups
    between workgroups in different places (1: one workgroup walks it all)."""
    g = np.random.Generator(np.random.PCG64(105))
    M, K, N = 272, 1280, 16
    codes = W.q4_0_codes(M, K, g)
    q = Q4(codes, W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    kw = dict(tiles_per_wave=tpw, waves_per_group=wpg, max_groups=groups, workspace=big_workspace())
    parity(out_to_f64(q.run(a, **kw)), q.oracle(a), "bf16")
    qi = Q4(codes, np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    ai = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    assert np.array_equal(out_to_f64(qi.run(ai, "bf16", "f32", **kw)), qi.oracle(ai))


@pytest.mark.parametrize("groups", [1, 3, 40, 0])
def test_walk_many_pieces(groups):
    """A long K (17 chunks per tile group) over few or many workgroups: tile
    groups cut into up to 17 pieces, combined by the last to arrive."""
    g = np.random.Generator(np.random.PCG64(112))
    M, K, N = 300, 17408, 16
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(N, K)))
    kw = dict(tiles_per_wave=2, waves_per_group=4, max_groups=groups, workspace=big_workspace())
    y = q.run(x, **kw)
    parity(out_to_f64(y), q.oracle(x), "bf16")
    for n in (0, 9):
        assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[n:n + 1]), **kw))[0], bits_u16(y)[n])


@pytest.mark.parametrize("groups", [5, 6])
def test_walk_range_edges_exact(groups):
    """51 chunks over 5 or 6 workgroups (10.2 and 8.5 per share), so range
    edges fall inside tile groups at several places.  With integer weights and
    activations every output is an exact integer, so a step computed twice or
    dropped at a range edge shows; then real scales against the oracle, and
    rows bit-identical alone."""
    g = np.random.Generator(np.random.PCG64(113))
    M, K, N = 300, 17408, 16
    codes = W.q4_0_codes(M, K, g)
    kw = dict(tiles_per_wave=2, waves_per_group=4, max_groups=groups, workspace=big_workspace())
    qi = Q4(codes, np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    ai = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    assert np.array_equal(out_to_f64(qi.run(ai, "bf16", "f32", **kw)), qi.oracle(ai))
    q = Q4(codes, W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(N, K)))
    y = q.run(x, **kw)
    parity(out_to_f64(y), q.oracle(x), "bf16")
    for n in (0, 13):
        assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[n:n + 1]), **kw))[0], bits_u16(y)[n])


@pytest.mark.parametrize("tpw", [1, 2, 4])
@pytest.mark.parametrize("wpg", [2, 4, 8])
def test_every_one_shot_shape_parity_and_exact_integers(tpw, wpg):
    """17 tiles and 33 blocks (a partial last step of 128), staged in several
    LDS chunks, every tile/wave shape, no workspace."""
    g = np.random.Generator(np.random.PCG64(104))
    M, K, N = 272, 1056, 16
    codes = W.q4_0_codes(M, K, g)
    q = Q4(codes, W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    kw = dict(tiles_per_wave=tpw, waves_per_group=wpg, workspace=None)
    parity(out_to_f64(q.run(a, **kw)), q.oracle(a), "bf16")
    qi = Q4(codes, np.full((M, K // 32), 0x3C00, dtype=np.uint16))
    ai = W.f32_to_bf16_bits(g.integers(-4, 5, size=(N, K)))
    assert np.array_equal(out_to_f64(qi.run(ai, "bf16", "f32", **kw)), qi.oracle(ai))


@pytest.mark.parametrize("tpw,wpg", [(3, 4), (1, 1), (1, 16), (4, 3)])
def test_unsupported_launch_shapes_rejected(tpw, wpg):
    g = np.random.Generator(np.random.PCG64(108))
    M, K = 64, 256
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    with pytest.raises(vq.VqError) as e:
        q.run(W.f32_to_bf16_bits(g.standard_normal((4, K))), tiles_per_wave=tpw, waves_per_group=wpg,
              workspace=big_workspace())
    assert e.value.status == vq.VQ_ERR_BAD_CONFIG


def test_group_cap_without_workspace_rejected():
    g = np.random.Generator(np.random.PCG64(109))
    M, K = 64, 1024
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    with pytest.raises(vq.VqError) as e:
        q.run(W.f32_to_bf16_bits(g.standard_normal((4, K))), tiles_per_wave=1, waves_per_group=4, max_groups=4,
              workspace=None)
    assert e.value.status == vq.VQ_ERR_WORKSPACE


@pytest.mark.parametrize("tpw,wpg,groups,K,walk", [
    (4, 4, 0, 2048, True), (2, 8, 3, 2048, True), (1, 2, 0, 2048, True), (4, 2, 5, 2048, True),
    (2, 4, 0, 2048, True), (4, 4, 0, 2080, False), (1, 2, 0, 2080, False), (2, 8, 0, 2048, False)])
def test_launch_shapes_rows_bit_identical_across_widths(tpw, wpg, groups, K, walk):
    """Width invariance holds in every launch shape and form, not only the
    default one."""
    g = np.random.Generator(np.random.PCG64(107))
    M = 400
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    kw = dict(tiles_per_wave=tpw, waves_per_group=wpg, max_groups=groups,
              workspace=big_workspace() if walk else None)
    full = bits_u16(q.run(x, **kw))
    for n in (0, 7, 15):
        one = bits_u16(q.run(np.ascontiguousarray(x[n:n + 1]), **kw))
        assert np.array_equal(one[0], full[n])
    assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(x[3:11]), **kw)), full[3:11])


def test_without_workspace_parity_and_width_invariance():
    """No workspace: the one-shot form (every workgroup walks all of K chunk by
    chunk)."""
    g = np.random.Generator(np.random.PCG64(110))
    M, K = 1000, 5120
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_lognormal(M, K, g))
    x = W.f32_to_bf16_bits(0.5 * g.standard_t(3, size=(16, K)))
    full = q.run(x, workspace=None)
    parity(out_to_f64(full), q.oracle(x), "bf16")
    one = bits_u16(q.run(np.ascontiguousarray(x[5:6]), workspace=None))
    assert np.array_equal(one[0], bits_u16(full)[5])


def test_workspace_reused_across_shapes_and_calls():
    """A workspace left by one call is ready for the next: the arrival counters
    return to zero, and whatever the piece slots hold (another shape's sums,
    or bytes that read as NaN) does not change a result."""
    g = np.random.Generator(np.random.PCG64(111))
    ws = vq.Workspace(32 << 20)
    ws.tensor[65536:].fill_(0xFF)
    mats = []
    for M, K in ((1088, 5120), (320, 8192), (17, 96), (4100, 1024)):
        q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
        x = W.f32_to_bf16_bits(g.standard_normal((16, K)))
        y = q.run(x, workspace=ws)
        parity(out_to_f64(y), q.oracle(x), "bf16")
        mats.append((q, x, bits_u16(y)))
    for rep in range(3):
        for q, x, ref in mats:
            if rep == 1:
                ws.tensor[65536:].fill_(0xFF)
            assert np.array_equal(bits_u16(q.run(x, workspace=ws)), ref)
    assert not ws.tensor[:65536].cpu().numpy().any()  # the counters are back at zero


def test_many_row_groups():
    """N > 16 is processed as groups of 16 rows; each row matches its 16-row call."""
    g = np.random.Generator(np.random.PCG64(106))
    M, K, N = 200, 640, 50
    q = Q4(W.q4_0_codes(M, K, g), W.fp16_scales_uniform(M, K, g))
    a = W.f32_to_bf16_bits(g.standard_normal((N, K)))
    y = bits_u16(q.run(a))
    parity(out_to_f64(q.run(a)), q.oracle(a), "bf16")
    for r0 in (0, 16, 32):
        assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(a[r0:r0 + 16]))), y[r0:r0 + 16])
    assert np.array_equal(bits_u16(q.run(np.ascontiguousarray(a[48:50]))), y[48:50])


def test_full_stream_layer_sampled():
    """One synthetic layer of the per-token weight stream at full size, in the
    library's default launch shapes, 16 rows, sampled outputs vs the oracle."""
    for idx in range(len(W.STREAM_LAYER_SHAPES)):
        m = W.stream_matrix(layer=3, idx=idx)
        q = Q4(m["codes"], m["scales"])
        a = W.stream_act(3, q.K)
        y = out_to_f64(q.run(a))
        cols = _sample_cols(q.M, 256, idx)
        fro, worst, ulps = parity(y[:, cols], q.oracle(a, cols=cols), "bf16")
        print("stream %dx%d: relF %.3e worst %.3e max %.2f ulp" % (q.M, q.K, fro, worst, ulps))
