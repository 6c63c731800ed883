"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments before touching a device (CPU only, no compute calls)."""
import ctypes
import os
import re

import pytest
import torch

import block_quantized_gemm_amd as vq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "vq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert len(names) >= 8, names
    handle = ctypes.CDLL(vq.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(vq.SIGNATURES), "binding and header disagree"


def test_version_and_status_strings():
    assert vq.lib().vq_version() == 400
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert vq.status_string(st) and vq.status_string(st) != "unknown status"
    assert vq.status_string(-99) == "unknown status"


A = 0x10000   # fake, 16-byte-aligned addresses: never dereferenced, validation fails first
B = 0x20000
C = 0x30000
D = 0x40000
E = 0x50000


F = 0x60000   # fake workspace


def _q4(w=A, s=B, x=C, xd=vq.DTYPE_BF16, xs=None, o=D, od=vq.DTYPE_BF16, n=16, m=256, k=512, alpha=1.0,
        ws=None, wsb=0):
    return vq.lib().vq_gemm_q4_0(w, s, x, xd, xs, o, od, n, m, k, alpha, ws, wsb, None)


def test_q4_0_argument_errors():
    assert _q4(w=None) == vq.VQ_ERR_NULL_POINTER
    assert _q4(o=None) == vq.VQ_ERR_NULL_POINTER
    assert _q4(xd=vq.DTYPE_F32) == vq.VQ_ERR_BAD_DTYPE
    assert _q4(od=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert _q4(xs=E) == vq.VQ_ERR_BAD_DTYPE            # float activations carry no scales
    assert _q4(xd=vq.DTYPE_I8, xs=None) == vq.VQ_ERR_NULL_POINTER
    assert _q4(k=500) == vq.VQ_ERR_BAD_SHAPE
    assert _q4(k=0) == vq.VQ_ERR_BAD_SHAPE
    assert _q4(n=0) == vq.VQ_ERR_BAD_SHAPE
    assert _q4(m=-3) == vq.VQ_ERR_BAD_SHAPE
    assert _q4(m=(1 << 24) + 1) == vq.VQ_ERR_BAD_SHAPE
    assert _q4(x=C + 8) == vq.VQ_ERR_MISALIGNED
    assert _q4(w=A + 1) == vq.VQ_ERR_MISALIGNED
    assert _q4(ws=F + 4, wsb=1 << 20) == vq.VQ_ERR_MISALIGNED


def test_fp8_argument_errors():
    f = vq.lib().vq_gemm_fp8_blk128
    assert f(None, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 512, None, 0, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, B, C, vq.DTYPE_I8, D, vq.DTYPE_BF16, 4, 256, 512, None, 0, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 480, None, 0, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B + 4, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 512, None, 0, None) == vq.VQ_ERR_MISALIGNED


def test_quant_argument_errors():
    for f in (vq.lib().vq_hadamard32_quant_int8, vq.lib().vq_hadamard32_quant_int4):
        assert f(None, vq.DTYPE_BF16, B, C, 4, 64, None) == vq.VQ_ERR_NULL_POINTER
        assert f(A, vq.DTYPE_F32, B, C, 4, 64, None) == vq.VQ_ERR_BAD_DTYPE
        assert f(A, vq.DTYPE_BF16, B, C, 4, 48, None) == vq.VQ_ERR_BAD_SHAPE
        assert f(A, vq.DTYPE_BF16, B + 2, C, 4, 64, None) == vq.VQ_ERR_MISALIGNED


def _ex(t, w, s, ws=None, wsb=0, k=512):
    return vq.lib().vq_gemm_q4_0_ex(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 16, 256, k, 1.0, t, w, s,
                                    ws, wsb, None)


def test_explicit_launch_shape_errors():
    assert _ex(3, 4, 0) == vq.VQ_ERR_BAD_CONFIG       # tiles per wave not in {1, 2, 4}
    assert _ex(1, 16, 0) == vq.VQ_ERR_BAD_CONFIG      # waves per group not in {2, 4, 8}
    assert _ex(1, 1, 0) == vq.VQ_ERR_BAD_CONFIG
    assert _ex(-1, 4, 0) == vq.VQ_ERR_BAD_CONFIG
    assert _ex(1, 4, -1) == vq.VQ_ERR_BAD_CONFIG
    assert _ex(1, 4, 2) == vq.VQ_ERR_WORKSPACE        # a group cap asks for the walk form: needs a workspace
    assert _ex(1, 4, 2, ws=F, wsb=64) == vq.VQ_ERR_WORKSPACE
    assert _ex(1, 4, 0, ws=F, wsb=64) == vq.VQ_ERR_WORKSPACE
    # the walk form moves Q4_0 scales in 16-byte pieces: K % 256 == 0
    assert _ex(1, 4, 0, ws=F, wsb=1 << 30, k=544) == vq.VQ_ERR_BAD_CONFIG


def _walk_need(m, k, t, w, chunk_steps=8, cap=1024):
    steps = -(-k // 128)
    chunks = -(-(-(-m // 16)) // (t * w)) * -(-steps // chunk_steps)
    return 64 * 1024 + min(chunks, cap) * 2 * t * w * 1024


def test_workspace_query():
    f = vq.lib().vq_workspace_bytes
    assert f(0, 17408, 5120) > 0 and f(1, 17408, 5120) > 0
    assert f(0, 17408, 5000) == 0 and f(1, 17408, 5120 + 32) == 0 and f(7, 256, 512) == 0
    assert f(0, 17408, 5120 + 32) == 0      # Q4_0 with K % 256 != 0 only runs one-shot
    # counters, then two pieces of a tile group (8 tiles x 1 KiB) per workgroup
    assert f(0, 17408, 5120) == _walk_need(17408, 5120, 1, 8) == 65536 + 680 * 16384
    for m, k in ((256, 512), (17408, 5120), (5120, 17408), (8192, 5120), (5120, 8192)):
        t, w, walk, used = vq.default_launch_shape("q4_0", m, k)
        assert walk == 1 and used == vq.workspace_bytes("q4_0", m, k) == _walk_need(m, k, t, w)
        assert used <= (16 << 20) + 65536
        # without a workspace the default is the one-shot form
        t0, w0, walk0, used0 = vq.default_launch_shape("q4_0", m, k, workspace_bytes=0)
        assert walk0 == 0 and used0 == 0
        # with too little, too
        assert vq.default_launch_shape("q4_0", m, k, workspace_bytes=used - 16)[2] == 0


def test_default_launch_shape_ignores_rows():
    # the shape is a function of (M, K, workspace) only, which keeps rows N-invariant
    for m, k in ((256, 512), (17408, 5120), (5120, 17408), (8192, 5120), (5120, 8192), (17, 96)):
        for kind in ("q4_0", "fp8"):
            if kind == "fp8" and k % 128:
                continue
            t, w, walk, used = vq.default_launch_shape(kind, m, k)
            assert t in (1, 2, 4) and w in (2, 4, 8) and walk in (0, 1)
            assert (used > 0) == (walk == 1)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_arguments_without_device_report_device_error():
    assert _q4() == vq.VQ_ERR_DEVICE


def _table(rows):
    t = (vq.VerifyProblem * len(rows))()
    for i, r in enumerate(rows):
        t[i] = vq.VerifyProblem(*r)
    return t


def test_grouped_argument_errors():
    f = vq.lib().vq_gemm_q4_0_grouped
    good = (A, B, C, D, 256, 512)
    t = _table([good, good])
    assert f(None, 2, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0, None) == vq.VQ_ERR_NULL_POINTER
    assert f(t, 0, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(t, 4097, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(t, 2, vq.DTYPE_BF16, vq.DTYPE_BF16, 0, 1.0, None, 0, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(t, 2, vq.DTYPE_I8, vq.DTYPE_BF16, 16, 1.0, None, 0, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(_table([good, (A, None, C, D, 256, 512)]), 2, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0,
             None) == vq.VQ_ERR_NULL_POINTER
    assert f(_table([good, (A, B, C, D, 256, 500)]), 2, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0,
             None) == vq.VQ_ERR_BAD_SHAPE
    assert f(_table([(A, B, C + 2, D, 256, 512)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0,
             None) == vq.VQ_ERR_MISALIGNED
    # a workspace smaller than the group needs (K = 5120 splits into 5 slices)
    big = _table([(A, B, C, D, 256, 5120)] * 2)
    assert f(big, 2, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, F, 64, None) == vq.VQ_ERR_WORKSPACE
    g = vq.lib().vq_gemm_fp8_blk128_grouped
    assert g(_table([(A, B, C, D, 256, 500)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 4, None, 0,
             None) == vq.VQ_ERR_BAD_SHAPE


def test_grouped_workspace_query():
    f = vq.lib().vq_workspace_bytes_grouped
    layer = [(A, B, C, D, m, k) for m, k in ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120),
                                             (5120, 17408))]
    need = f(vq.KIND_Q4_0, _table(layer), 5)
    # one launch over every problem's chunks
    chunks = sum(-(-m // 128) * (k // 1024) for *_, m, k in layer)
    assert need == 65536 + min(chunks, 1024) * 16384
    # a one-shot problem needs no workspace
    assert f(vq.KIND_Q4_0, _table(layer + [(A, B, C, D, 4096, 4128)]), 6) == need
    assert f(vq.KIND_Q4_0, _table(layer + [(A, B, C, D, 17, 100)]), 6) == 0   # K % 32 != 0
    assert f(9, _table(layer), 5) == 0


def test_panel_size_query():
    f = vq.lib().vq_q4_0_panel_bytes
    # records of 256 features x 512 k: 64 KiB of codes + 8 KiB of scales
    assert f(17408, 5120) == 68 * 10 * 73728 == 17408 * 5120 // 2 * 9 // 8
    assert f(256, 512) == 73728
    assert f(128, 1024) == 2 * 73728
    assert f(257, 544) == 2 * 2 * 73728      # ragged M and K round up to whole records
    assert f(1, 32) == 73728
    assert f(0, 1024) == 0 and f(128, 1000) == 0 and f(128, (1 << 24) + 32) == 0
    assert vq.q4_0_panel_bytes(5120, 17408) == 20 * 34 * 73728


def _pk(c=A, s=B, m=256, k=512, p=C, pb=1 << 20):
    return vq.lib().vq_q4_0_to_panel(c, s, m, k, p, pb, None)


def _pg(w=A, x=C, xd=vq.DTYPE_BF16, o=D, od=vq.DTYPE_BF16, n=16, m=256, k=512, groups=0, ws=F, wsb=1 << 30):
    return vq.lib().vq_gemm_q4_0_panel_ex(w, x, xd, o, od, n, m, k, 1.0, groups, ws, wsb, None)


def test_panel_argument_errors():
    assert _pk(c=None) == vq.VQ_ERR_NULL_POINTER
    assert _pk(p=None) == vq.VQ_ERR_NULL_POINTER
    assert _pk(k=500) == vq.VQ_ERR_BAD_SHAPE
    assert _pk(pb=73728 - 16) == vq.VQ_ERR_BAD_SHAPE         # (256, 512) needs one whole record
    assert _pk(m=257, pb=2 * 73728 - 16) == vq.VQ_ERR_BAD_SHAPE  # (257, 512) needs two
    assert _pk(s=B + 2) == vq.VQ_ERR_MISALIGNED
    assert _pg(w=None) == vq.VQ_ERR_NULL_POINTER
    assert _pg(xd=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert _pg(od=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert _pg(k=500) == vq.VQ_ERR_BAD_SHAPE
    assert _pg(n=0) == vq.VQ_ERR_BAD_SHAPE
    assert _pg(x=C + 8) == vq.VQ_ERR_MISALIGNED
    assert _pg(groups=-1) == vq.VQ_ERR_BAD_CONFIG
    assert _pg(ws=None) == vq.VQ_ERR_WORKSPACE            # panels always walk
    assert _pg(wsb=64) == vq.VQ_ERR_WORKSPACE
    assert _pg(ws=F + 4) == vq.VQ_ERR_MISALIGNED
    g = vq.lib().vq_gemm_q4_0_panel
    assert g(A, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 16, 256, 512, 1.0, None, 0, None) == vq.VQ_ERR_WORKSPACE
    h = vq.lib().vq_gemm_q4_0_panel_grouped
    t = _table([(A, None, C, D, 256, 512)])
    assert h(t, 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, None, 0, None) == vq.VQ_ERR_WORKSPACE
    assert h(_table([(A, None, C, D, 256, 500)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, F, 1 << 30,
             None) == vq.VQ_ERR_BAD_SHAPE
    assert h(_table([(None, None, C, D, 256, 512)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, 1.0, F, 1 << 30,
             None) == vq.VQ_ERR_NULL_POINTER


def test_panel_workspace_and_shape_queries():
    # any K % 32 == 0 walks; one 256-feature panel of 8 two-tile waves per
    # workgroup, chunks of 4 steps (one record)
    for m, k in ((256, 512), (17408, 5120), (1, 32), (129, 1056), (5120, 17408)):
        t, w, walk, used = vq.default_launch_shape("q4_0_panel", m, k)
        assert (t, w, walk) == (2, 8, 1)
        assert used == vq.workspace_bytes("q4_0_panel", m, k) == _walk_need(m, k, 2, 8, chunk_steps=4)
    # the same chunk count as the row-major walk (72 KiB chunks), twice the piece size
    assert vq.workspace_bytes("q4_0_panel", 17408, 5120) - 65536 == 2 * (vq.workspace_bytes("q4_0", 17408, 5120) - 65536)
    f = vq.lib().vq_workspace_bytes_grouped
    layer = [(A, None, C, D, m, k) for m, k in ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120),
                                                (5120, 17408))]
    # 2680 chunks, capped at 1024 workgroups
    assert f(vq.KIND_Q4_0_PANEL, _table(layer), 5) == 65536 + 1024 * 2 * 16 * 1024


def test_fp8_panel_size_query():
    f = vq.lib().vq_fp8_panel_bytes
    # records of 128 features x 1024 k of E4M3 codes (128 KiB)
    assert f(17408, 5120) == 136 * 5 * 131072 == 17408 * 5120
    assert f(128, 1024) == 131072
    assert f(129, 1152) == 2 * 2 * 131072    # ragged M and K round up to whole records
    assert f(1, 128) == 131072
    assert f(0, 1024) == 0 and f(128, 1000) == 0 and f(128, 96) == 0 and f(128, (1 << 24) + 128) == 0
    assert vq.fp8_panel_bytes(5120, 17408) == 40 * 17 * 131072


def _fk(w=A, m=128, k=1024, p=C, pb=1 << 20):
    return vq.lib().vq_fp8_to_panel(w, m, k, p, pb, None)


def _fg(w=A, s=B, x=C, xd=vq.DTYPE_BF16, o=D, od=vq.DTYPE_BF16, n=16, m=256, k=1024, groups=0, ws=F,
        wsb=1 << 30):
    return vq.lib().vq_gemm_fp8_blk128_panel_ex(w, s, x, xd, o, od, n, m, k, groups, ws, wsb, None)


def test_fp8_panel_argument_errors():
    assert _fk(w=None) == vq.VQ_ERR_NULL_POINTER
    assert _fk(p=None) == vq.VQ_ERR_NULL_POINTER
    assert _fk(k=1000) == vq.VQ_ERR_BAD_SHAPE
    assert _fk(pb=131072 - 16) == vq.VQ_ERR_BAD_SHAPE          # (128, 1024) needs one whole record
    assert _fk(m=129, pb=2 * 131072 - 16) == vq.VQ_ERR_BAD_SHAPE
    assert _fk(w=A + 8) == vq.VQ_ERR_MISALIGNED
    assert _fk(p=C + 8) == vq.VQ_ERR_MISALIGNED
    assert _fg(w=None) == vq.VQ_ERR_NULL_POINTER
    assert _fg(s=None) == vq.VQ_ERR_NULL_POINTER
    assert _fg(xd=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert _fg(od=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert _fg(k=1000) == vq.VQ_ERR_BAD_SHAPE
    assert _fg(n=0) == vq.VQ_ERR_BAD_SHAPE
    assert _fg(x=C + 8) == vq.VQ_ERR_MISALIGNED
    assert _fg(groups=-1) == vq.VQ_ERR_BAD_CONFIG
    assert _fg(ws=None) == vq.VQ_ERR_WORKSPACE                # panels always walk
    assert _fg(wsb=64) == vq.VQ_ERR_WORKSPACE
    assert _fg(ws=F + 4) == vq.VQ_ERR_MISALIGNED
    g = vq.lib().vq_gemm_fp8_blk128_panel
    assert g(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 16, 256, 1024, None, 0, None) == vq.VQ_ERR_WORKSPACE
    h = vq.lib().vq_gemm_fp8_blk128_panel_grouped
    t = _table([(A, B, C, D, 256, 1024)])
    assert h(t, 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, None, 0, None) == vq.VQ_ERR_WORKSPACE
    assert h(_table([(A, B, C, D, 256, 1000)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, F, 1 << 30,
             None) == vq.VQ_ERR_BAD_SHAPE
    assert h(_table([(A, None, C, D, 256, 1024)]), 1, vq.DTYPE_BF16, vq.DTYPE_BF16, 16, F, 1 << 30,
             None) == vq.VQ_ERR_NULL_POINTER


def test_fp8_panel_workspace_and_shape_queries():
    # any K % 128 == 0 walks; one 128-feature panel of 8 one-tile waves per
    # workgroup, chunks of 8 steps (one record)
    for m, k in ((128, 1024), (17408, 5120), (1, 128), (129, 1152), (5120, 17408)):
        t, w, walk, used = vq.default_launch_shape("fp8_panel", m, k)
        assert (t, w, walk) == (1, 8, 1)
        assert used == vq.workspace_bytes("fp8_panel", m, k) == _walk_need(m, k, 1, 8, chunk_steps=8)
    f = vq.lib().vq_workspace_bytes_grouped
    layer = [(A, B, C, D, m, k) for m, k in ((8192, 5120), (5120, 8192), (17408, 5120), (17408, 5120),
                                             (5120, 17408))]
    # 2 x 680 + 320 + 320 + 680 = 2680 chunks, capped at 1024 workgroups
    assert f(vq.KIND_FP8_PANEL, _table(layer), 5) == 65536 + 1024 * 2 * 8 * 1024


def test_greedy_argument_errors_and_workspace_query():
    f = vq.lib().vq_greedy_verify
    ws = vq.lib().vq_greedy_workspace_bytes
    # one 8-byte key per row and segment of at most 4096 entries (up to 128 segments)
    assert ws(16, 151936) == 16 * 38 * 8
    assert ws(1, 1) == 8 and ws(4096, 1 << 24) == 4096 * 128 * 8
    assert ws(0, 10) == 0 and ws(4097, 10) == 0 and ws(4, 0) == 0
    big = 1 << 30

    def call(lg=A, dt=vq.DTYPE_F32, n=16, v=1000, d=B, t=C, c=D, w=F, wb=big):
        return f(lg, dt, n, v, d, t, c, w, wb, None)
    assert call(lg=None) == vq.VQ_ERR_NULL_POINTER
    assert call(d=None) == vq.VQ_ERR_NULL_POINTER
    assert call(c=None) == vq.VQ_ERR_NULL_POINTER
    assert call(dt=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert call(n=0) == vq.VQ_ERR_BAD_SHAPE
    assert call(n=4097) == vq.VQ_ERR_BAD_SHAPE
    assert call(v=0) == vq.VQ_ERR_BAD_SHAPE
    assert call(t=C + 4) == vq.VQ_ERR_MISALIGNED
    assert call(w=None) == vq.VQ_ERR_WORKSPACE
    assert call(wb=16 * 8 - 8) == vq.VQ_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert call(n=1, d=None) == vq.VQ_ERR_DEVICE   # a one-row block needs no draft


def test_rotate_argument_errors():
    f = vq.lib().vq_q4_0_rotate_h32
    assert f(None, B, 256, 512, C, D, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, B, 256, 512, C, None, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, B, 256, 500, C, D, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B, 0, 512, C, D, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B + 2, 256, 512, C, D, None) == vq.VQ_ERR_MISALIGNED
    if not torch.cuda.is_available():
        assert f(A, B, 256, 512, C, D, None) == vq.VQ_ERR_DEVICE


def test_fp8_prefill_argument_errors():
    f = vq.lib().vq_gemm_fp8_blk128_prefill
    assert f(None, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 512, 256, 512, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, B, C, vq.DTYPE_I8, D, vq.DTYPE_BF16, 512, 256, 512, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_I8, 512, 256, 512, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 512, 256, 480, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 0, 256, 512, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B, C + 2, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 512, 256, 512, None) == vq.VQ_ERR_MISALIGNED


def test_hbm_probe_argument_errors():
    L = vq.lib()

    def probe(buf=A, nbytes=1 << 20, mode=vq.PROBE_BLOCKS, groups=0, waves=8, depth=8, nt=0, sink=B):
        return L.vq_hbm_read_probe(buf, nbytes, mode, groups, waves, depth, nt, sink, None)
    assert probe(buf=None) == vq.VQ_ERR_NULL_POINTER
    assert probe(sink=None) == vq.VQ_ERR_NULL_POINTER
    assert probe(buf=A + 8) == vq.VQ_ERR_MISALIGNED
    assert probe(nbytes=65536 + 1024) == vq.VQ_ERR_BAD_SHAPE
    assert probe(nbytes=0) == vq.VQ_ERR_BAD_SHAPE
    assert probe(nbytes=(1 << 31) + 65536) == vq.VQ_ERR_BAD_SHAPE
    assert probe(mode=5) == vq.VQ_ERR_BAD_CONFIG
    assert probe(mode=vq.PROBE_LDS, groups=0) == vq.VQ_ERR_BAD_CONFIG
    assert probe(mode=vq.PROBE_LDS, groups=16, nt=1) == vq.VQ_ERR_BAD_CONFIG  # LDS reads have no cache policy
    assert probe(mode=vq.PROBE_REREAD, groups=0) == vq.VQ_ERR_BAD_CONFIG
    assert probe(mode=vq.PROBE_REREAD, groups=3) == vq.VQ_ERR_BAD_SHAPE  # 1 MiB is not 3 equal shares
    assert probe(nbytes=3 << 20, mode=vq.PROBE_REREAD, groups=1) == vq.VQ_ERR_BAD_SHAPE  # 384 pieces per wave
    assert probe(waves=2) == vq.VQ_ERR_BAD_CONFIG
    assert probe(depth=5) == vq.VQ_ERR_BAD_CONFIG
    assert probe(nt=2) == vq.VQ_ERR_BAD_CONFIG
    assert probe(groups=4) == vq.VQ_ERR_BAD_CONFIG                     # blocks: no group count
    assert probe(mode=vq.PROBE_SHARES, groups=0) == vq.VQ_ERR_BAD_CONFIG
    assert probe(mode=vq.PROBE_SHARES, groups=3) == vq.VQ_ERR_BAD_SHAPE  # shares must divide evenly
    assert probe(mode=vq.PROBE_WINDOW, groups=70000) == vq.VQ_ERR_BAD_CONFIG
    # valid arguments get as far as the device check (no GPU here)
    if not torch.cuda.is_available():
        assert probe(mode=vq.PROBE_SHARES, groups=16) == vq.VQ_ERR_DEVICE
        assert probe(nbytes=3 << 20, mode=vq.PROBE_REREAD, groups=3) == vq.VQ_ERR_DEVICE  # 128 pieces per wave
        assert probe(mode=vq.PROBE_LDS, groups=3) == vq.VQ_ERR_DEVICE


def test_noalloc_argument_errors():
    L = vq.lib()

    def na(w=A, s=B, x=C, xd=vq.DTYPE_BF16, xs=None, o=D, od=vq.DTYPE_BF16, n=16, m=256, k=512):
        return L.vq_gemm_q4_0_noalloc(w, s, x, xd, xs, o, od, n, m, k, 1.0, None)
    assert na(w=None) == vq.VQ_ERR_NULL_POINTER
    assert na(o=None) == vq.VQ_ERR_NULL_POINTER
    assert na(xd=vq.DTYPE_F32) == vq.VQ_ERR_BAD_DTYPE
    assert na(xs=E) == vq.VQ_ERR_BAD_DTYPE
    assert na(od=vq.DTYPE_I8) == vq.VQ_ERR_BAD_DTYPE
    assert na(k=500) == vq.VQ_ERR_BAD_SHAPE
    assert na(n=0) == vq.VQ_ERR_BAD_SHAPE
    assert na(x=C + 8) == vq.VQ_ERR_MISALIGNED
    assert na(xd=vq.DTYPE_I8, xs=None) == vq.VQ_ERR_NULL_POINTER
    if not torch.cuda.is_available():
        assert na() == vq.VQ_ERR_DEVICE
