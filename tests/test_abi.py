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
    assert vq.lib().vq_version() == 100
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert vq.status_string(st) and vq.status_string(st) != "unknown status"
    assert vq.status_string(-99) == "unknown status"


A = 0x10000   # fake, 16-byte-aligned addresses: never dereferenced, validation fails first
B = 0x20000
C = 0x30000
D = 0x40000
E = 0x50000


def _q4(w=A, s=B, x=C, xd=vq.DTYPE_BF16, xs=None, o=D, od=vq.DTYPE_BF16, n=16, m=256, k=512, alpha=1.0):
    return vq.lib().vq_gemm_q4_0(w, s, x, xd, xs, o, od, n, m, k, alpha, None)


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


def test_fp8_argument_errors():
    f = vq.lib().vq_gemm_fp8_blk128
    assert f(None, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 512, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, B, C, vq.DTYPE_I8, D, vq.DTYPE_BF16, 4, 256, 512, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 480, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, B + 4, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 4, 256, 512, None) == vq.VQ_ERR_MISALIGNED


def test_quant_argument_errors():
    f = vq.lib().vq_hadamard32_quant_int8
    assert f(None, vq.DTYPE_BF16, B, C, 4, 64, None) == vq.VQ_ERR_NULL_POINTER
    assert f(A, vq.DTYPE_F32, B, C, 4, 64, None) == vq.VQ_ERR_BAD_DTYPE
    assert f(A, vq.DTYPE_BF16, B, C, 4, 48, None) == vq.VQ_ERR_BAD_SHAPE
    assert f(A, vq.DTYPE_BF16, B + 2, C, 4, 64, None) == vq.VQ_ERR_MISALIGNED


def test_explicit_launch_shape_errors():
    f = vq.lib().vq_gemm_q4_0_ex
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 16, 256, 512, 1.0, 3, 4, None) == vq.VQ_ERR_BAD_CONFIG
    assert f(A, B, C, vq.DTYPE_BF16, D, vq.DTYPE_BF16, 16, 256, 512, 1.0, 1, 32, None) == vq.VQ_ERR_BAD_CONFIG


def test_default_launch_shape_ignores_rows():
    # the shape is a function of (M, K) only, which is what keeps rows N-invariant
    for m, k in ((256, 512), (17408, 5120), (5120, 17408), (8192, 5120), (5120, 8192)):
        t, w = vq.default_launch_shape("q4_0", m, k)
        assert t in (1, 2, 4) and w in (1, 2, 4, 8, 16)
        t, w = vq.default_launch_shape("fp8", m, k)
        assert t in (1, 2, 4) and w in (1, 2, 4, 8, 16)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_arguments_without_device_report_device_error():
    assert _q4() == vq.VQ_ERR_DEVICE
