"""CPU oracle for the block-quantized verify GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``block_quantized_gemm_amd``) never imports it, and it never imports
the product library: the two share no code.

The arithmetic lives in ``vq_oracle.c`` (plain scalar C, fp64 accumulation,
fp32 step-by-step emulation of the H32 int8 quantizer); this module only
marshals numpy arrays into it.  Citations of the pages are in the C file's
header and on each function there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libvq_oracle.so")

F16 = 1
BF16 = 2
F32 = 3

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile vq_oracle.c with gcc into oracle/libvq_oracle.so."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.vqo_f16_to_f64.restype = ctypes.c_double
        lib.vqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.vqo_bf16_to_f64.restype = ctypes.c_double
        lib.vqo_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.vqo_e4m3_to_f64.restype = ctypes.c_double
        lib.vqo_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.vqo_q4_0_code.restype = ctypes.c_int
        lib.vqo_q4_0_code.argtypes = [P, I64, I64, I64]
        lib.vqo_q4_0_dequant.restype = None
        lib.vqo_q4_0_dequant.argtypes = [P, P, I64, I64, P, I64, P]
        lib.vqo_fp8_dequant.restype = None
        lib.vqo_fp8_dequant.argtypes = [P, P, I64, I64, P, I64, P]
        lib.vqo_gemm_q4_0.restype = None
        lib.vqo_gemm_q4_0.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, P, I64,
                                      ctypes.c_double, P]
        lib.vqo_gemm_fp8_blk128.restype = None
        lib.vqo_gemm_fp8_blk128.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, P, I64, P]
        lib.vqo_w4a8_block_dot.restype = ctypes.c_int64
        lib.vqo_w4a8_block_dot.argtypes = [P, P, I64, I64, I64, I64]
        lib.vqo_gemm_w4a8.restype = None
        lib.vqo_gemm_w4a8.argtypes = [P, P, P, P, I64, I64, I64, P, I64, ctypes.c_double, P]
        lib.vqo_f32_to_f16_rne.restype = ctypes.c_uint16
        lib.vqo_f32_to_f16_rne.argtypes = [ctypes.c_float]
        lib.vqo_fwht32_f32.restype = None
        lib.vqo_fwht32_f32.argtypes = [P]
        lib.vqo_h32_matrix.restype = None
        lib.vqo_h32_matrix.argtypes = [P]
        lib.vqo_h32_quant_int8.restype = ctypes.c_int
        lib.vqo_h32_quant_int8.argtypes = [P, ctypes.c_int, I64, I64, P, P]
        lib.vqo_h32_quant_int4.restype = ctypes.c_int
        lib.vqo_h32_quant_int4.argtypes = [P, ctypes.c_int, I64, I64, P, P]
        lib.vqo_block_quant.restype = ctypes.c_int
        lib.vqo_block_quant.argtypes = [P, ctypes.c_int, I64, I64, ctypes.c_int, ctypes.c_int, P, P]
        lib.vqo_q4_0_rotate_h32.restype = None
        lib.vqo_q4_0_rotate_h32.argtypes = [P, P, I64, I64, P, P]
        lib.vqo_greedy_verify.restype = I64
        lib.vqo_greedy_verify.argtypes = [P, ctypes.c_int, I64, I64, P, P]
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _cols(cols, M):
    if cols is None:
        return np.arange(M, dtype=np.int64)
    return _c(cols, np.int64)


# ---------------------------------------------------------------- decoders

def f16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.vqo_f16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.vqo_bf16_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def e4m3_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint8)
    return np.array([lib.vqo_e4m3_to_f64(int(v)) for v in b.ravel()]).reshape(b.shape)


def f32_to_f16_bits(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib.vqo_f32_to_f16_rne(float(x)) for x in v.ravel()],
                    dtype=np.uint16).reshape(v.shape)


def q4_0_code(codes: np.ndarray, K: int, m: int, k: int) -> int:
    codes = _c(codes, np.uint8)
    return int(_load().vqo_q4_0_code(_ptr(codes), K, m, k))


def q4_0_dequant(codes, scales, M, K, rows=None) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    rows = _cols(rows, M)
    out = np.empty((rows.size, K), dtype=np.float64)
    _load().vqo_q4_0_dequant(_ptr(codes), _ptr(scales), M, K, _ptr(rows), rows.size, _ptr(out))
    return out


def fp8_dequant(w, tscales, M, K, rows=None) -> np.ndarray:
    w = _c(w, np.uint8)
    tscales = _c(tscales, np.float32)
    rows = _cols(rows, M)
    out = np.empty((rows.size, K), dtype=np.float64)
    _load().vqo_fp8_dequant(_ptr(w), _ptr(tscales), M, K, _ptr(rows), rows.size, _ptr(out))
    return out


# ---------------------------------------------------------------- GEMMs

def gemm_q4_0(codes, scales, act_bits, act_dtype, N, M, K, cols=None, alpha=1.0) -> np.ndarray:
    """fp64 Y[n][c] = alpha * sum_k x[n][k] * w[cols[c]][k] for the listed features."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    act = _c(act_bits, np.uint16)
    cols = _cols(cols, M)
    out = np.empty((N, cols.size), dtype=np.float64)
    _load().vqo_gemm_q4_0(_ptr(codes), _ptr(scales), _ptr(act), int(act_dtype), N, M, K,
                          _ptr(cols), cols.size, float(alpha), _ptr(out))
    return out


def gemm_fp8_blk128(w, tscales, act_bits, act_dtype, N, M, K, cols=None) -> np.ndarray:
    w = _c(w, np.uint8)
    tscales = _c(tscales, np.float32)
    act = _c(act_bits, np.uint16)
    cols = _cols(cols, M)
    out = np.empty((N, cols.size), dtype=np.float64)
    _load().vqo_gemm_fp8_blk128(_ptr(w), _ptr(tscales), _ptr(act), int(act_dtype), N, M, K,
                                _ptr(cols), cols.size, _ptr(out))
    return out


def w4a8_block_dot(codes, qx, K, n, m, b) -> int:
    codes = _c(codes, np.uint8)
    qx = _c(qx, np.int8)
    return int(_load().vqo_w4a8_block_dot(_ptr(codes), _ptr(qx), K, n, m, b))


def gemm_w4a8(codes, wscales, qx, xscales, N, M, K, cols=None, alpha=1.0) -> np.ndarray:
    codes = _c(codes, np.uint8)
    wscales = _c(wscales, np.uint16)
    qx = _c(qx, np.int8)
    xscales = _c(xscales, np.uint16)
    cols = _cols(cols, M)
    out = np.empty((N, cols.size), dtype=np.float64)
    _load().vqo_gemm_w4a8(_ptr(codes), _ptr(wscales), _ptr(qx), _ptr(xscales), N, M, K,
                          _ptr(cols), cols.size, float(alpha), _ptr(out))
    return out


# ---------------------------------------------------------------- H32 quantizer

def fwht32_f32(x) -> np.ndarray:
    v = np.array(x, dtype=np.float32).reshape(32).copy()
    _load().vqo_fwht32_f32(_ptr(v))
    return v


def h32_matrix() -> np.ndarray:
    h = np.empty((32, 32), dtype=np.int8)
    _load().vqo_h32_matrix(_ptr(h))
    return h


def h32_quant_int8(x_bits, x_dtype, N, K):
    """Returns (q int8 [N][K], d fp16-bits uint16 [N][K/32], status)."""
    x = _c(x_bits, np.uint16)
    q = np.empty((N, K), dtype=np.int8)
    d = np.empty((N, K // 32), dtype=np.uint16)
    st = _load().vqo_h32_quant_int8(_ptr(x), int(x_dtype), N, K, _ptr(q), _ptr(d))
    return q, d, int(st)


def h32_quant_int4(x_bits, x_dtype, N, K):
    """The 4-bit quantizer: returns (q int8 [N][K] holding codes in [-7, 7],
    d fp16-bits uint16 [N][K/32], status)."""
    x = _c(x_bits, np.uint16)
    q = np.empty((N, K), dtype=np.int8)
    d = np.empty((N, K // 32), dtype=np.uint16)
    st = _load().vqo_h32_quant_int4(_ptr(x), int(x_dtype), N, K, _ptr(q), _ptr(d))
    return q, d, int(st)


def block_quant(x_bits, x_dtype, N, K, qmax, rotate):
    """Either quantizer rule with any symmetric bound, with or without the
    H32 rotation (rotate = False quantizes the plain blocks); see
    vqo_block_quant."""
    x = _c(x_bits, np.uint16)
    q = np.empty((N, K), dtype=np.int8)
    d = np.empty((N, K // 32), dtype=np.uint16)
    st = _load().vqo_block_quant(_ptr(x), int(x_dtype), N, K, int(qmax), int(bool(rotate)), _ptr(q), _ptr(d))
    return q, d, int(st)


# ---------------------------------------------------------------- greedy verification

def greedy_verify(logits, dtype, draft):
    """(target choice per row, number of committed tokens) for logits [n][V]
    (float32 values for F32, uint16 bit patterns for F16 / BF16) and drafted
    tokens [n - 1]; see vqo_greedy_verify."""
    lib = _load()
    lg = _c(logits, np.float32 if dtype == F32 else np.uint16)
    n, v = lg.shape
    d = _c(np.asarray(draft, dtype=np.int32).reshape(-1), np.int32)
    if d.size != n - 1:
        raise ValueError("draft must hold n_rows - 1 tokens")
    target = np.zeros(n, dtype=np.int32)
    count = lib.vqo_greedy_verify(_ptr(lg), dtype, n, v, _ptr(d) if d.size else None, _ptr(target))
    return target, int(count)


# ---------------------------------------------------------------- offline H32 rotation of Q4_0 weights

def q4_0_rotate_h32(codes, scales, M, K):
    """(codes, scales) of the H32-rotated, requantized Q4_0 matrix; see
    vqo_q4_0_rotate_h32."""
    lib = _load()
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint16)
    co = np.zeros((M, K // 2), dtype=np.uint8)
    so = np.zeros((M, K // 32), dtype=np.uint16)
    lib.vqo_q4_0_rotate_h32(_ptr(c), _ptr(s), M, K, _ptr(co), _ptr(so))
    return co, so
