"""Block-quantized verify GEMM for MI355X (gfx950): thin Python binding of libvq.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvq.so`` (built in-tree by ``block_quantized_gemm_amd.build``).
There is no fallback: if the library is missing, every call raises.

The C ABI is declared and documented in ``include/vq.h``.  The functions here
take torch tensors on the current ROCm device, check their dtypes, shapes and
contiguity, and pass raw pointers plus the current torch stream to the library.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvq.so")

VQ_OK = 0
VQ_ERR_NULL_POINTER = -1
VQ_ERR_BAD_SHAPE = -2
VQ_ERR_MISALIGNED = -3
VQ_ERR_BAD_DTYPE = -4
VQ_ERR_DEVICE = -5
VQ_ERR_LAUNCH = -6
VQ_ERR_BAD_CONFIG = -7
VQ_ERR_WORKSPACE = -8
VQ_ERR_SCRATCH = -9

KIND_Q4_0 = 0
KIND_FP8_BLK128 = 1
KIND_Q4_0_PANEL = 2
KIND_FP8_PANEL = 3
_KINDS = {"q4_0": KIND_Q4_0, "fp8": KIND_FP8_BLK128, "q4_0_panel": KIND_Q4_0_PANEL, "fp8_panel": KIND_FP8_PANEL}

PROBE_BLOCKS = 0
PROBE_SHARES = 1
PROBE_WINDOW = 2
PROBE_REREAD = 3
PROBE_LDS = 4
PROBE_REREAD_PASSES = 16
_PROBES = {"blocks": PROBE_BLOCKS, "shares": PROBE_SHARES, "window": PROBE_WINDOW, "reread": PROBE_REREAD,
           "lds": PROBE_LDS}

DTYPE_F16 = 1
DTYPE_BF16 = 2
DTYPE_F32 = 3
DTYPE_I8 = 4

# Every symbol include/vq.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "vq_gemm_q4_0": (_I, [_P, _P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _F, _P, _SZ, _P]),
    "vq_gemm_q4_0_noalloc": (_I, [_P, _P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _F, _P]),
    "vq_gemm_fp8_blk128": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "vq_hadamard32_quant_int8": (_I, [_P, _I, _P, _P, _I64, _I64, _P]),
    "vq_hadamard32_quant_int4": (_I, [_P, _I, _P, _P, _I64, _I64, _P]),
    "vq_gemm_fp8_blk128_prefill": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _P]),
    "vq_workspace_bytes": (_SZ, [_I, _I64, _I64]),
    "vq_gemm_q4_0_ex": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _F, _I, _I, _I, _P, _SZ, _P]),
    "vq_gemm_fp8_blk128_ex": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _I, _I, _I, _P, _SZ, _P]),
    "vq_default_launch_shape": (_I, [_I, _I64, _I64, _SZ, ctypes.POINTER(_I), ctypes.POINTER(_I),
                                     ctypes.POINTER(_I), ctypes.POINTER(_SZ)]),
    "vq_gemm_q4_0_grouped": (_I, [_P, _I, _I, _I, _I64, _F, _P, _SZ, _P]),
    "vq_gemm_fp8_blk128_grouped": (_I, [_P, _I, _I, _I, _I64, _P, _SZ, _P]),
    "vq_workspace_bytes_grouped": (_SZ, [_I, _P, _I]),
    "vq_q4_0_panel_bytes": (_SZ, [_I64, _I64]),
    "vq_q4_0_to_panel": (_I, [_P, _P, _I64, _I64, _P, _SZ, _P]),
    "vq_gemm_q4_0_panel": (_I, [_P, _P, _I, _P, _I, _I64, _I64, _I64, _F, _P, _SZ, _P]),
    "vq_gemm_q4_0_panel_ex": (_I, [_P, _P, _I, _P, _I, _I64, _I64, _I64, _F, _I, _P, _SZ, _P]),
    "vq_gemm_q4_0_panel_grouped": (_I, [_P, _I, _I, _I, _I64, _F, _P, _SZ, _P]),
    "vq_fp8_panel_bytes": (_SZ, [_I64, _I64]),
    "vq_fp8_to_panel": (_I, [_P, _I64, _I64, _P, _SZ, _P]),
    "vq_gemm_fp8_blk128_panel": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _P, _SZ, _P]),
    "vq_gemm_fp8_blk128_panel_ex": (_I, [_P, _P, _P, _I, _P, _I, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "vq_gemm_fp8_blk128_panel_grouped": (_I, [_P, _I, _I, _I, _I64, _P, _SZ, _P]),
    "vq_greedy_verify": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "vq_q4_0_rotate_h32": (_I, [_P, _P, _I64, _I64, _P, _P, _P]),
    "vq_greedy_workspace_bytes": (_SZ, [_I64, _I64]),
    "vq_hbm_read_probe": (_I, [_P, _SZ, _I, _I, _I, _I, _I, _P, _P]),
    "vq_status_string": (ctypes.c_char_p, [_I]),
    "vq_version": (_I, []),
}

_lock = threading.Lock()
_lib = None


class VerifyProblem(ctypes.Structure):
    """Mirror of vq_verify_problem."""
    _fields_ = [("w", _P), ("scales", _P), ("act", _P), ("out", _P), ("m", _I64), ("k", _I64)]


class VqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def lib() -> ctypes.CDLL:
    """The loaded libvq.so.  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libvq.so is not built (run python -m block_quantized_gemm_amd.build); "
                                   "there is no fallback path")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def status_string(status: int) -> str:
    return lib().vq_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != VQ_OK:
        raise VqError(status, where)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32,
         torch.int8: DTYPE_I8}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _dev_ptr(t, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return _torch().cuda.current_stream().cuda_stream


def _check_2d(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class Workspace:
    """A zero-filled device buffer for the walk form of the verify GEMMs:
    arrival counters and the partial sums of tile groups cut between two
    workgroups.

    The library leaves the counters at zero after every call, so it is zeroed
    once.  The zero fill runs on torch's current stream and is waited for here,
    so the buffer is ready for a call on any stream.  Calls sharing one
    workspace must be ordered (one stream, or streams the caller orders)."""

    def __init__(self, nbytes: int, device=None):
        torch = _torch()
        dev = torch.device(device if device is not None else "cuda")
        alloc = torch.cuda.current_stream(dev)
        self.tensor = torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=dev)
        if not torch.cuda.is_current_stream_capturing():
            alloc.synchronize()
        self._streams = {alloc.cuda_stream}

    @property
    def nbytes(self) -> int:
        return self.tensor.numel()

    def ptr(self) -> int:
        return self.tensor.data_ptr()

    def used_on(self, stream_handle: int):
        """Tell torch's caching allocator that kernels on this stream use the
        buffer, so that once the Workspace is dropped the memory is not handed
        out again before that stream's work is done."""
        if stream_handle not in self._streams:
            torch = _torch()
            self.tensor.record_stream(torch.cuda.ExternalStream(stream_handle, device=self.tensor.device))
            self._streams.add(stream_handle)


_auto_ws = {}
_auto_lock = threading.Lock()


def _workspace_args(workspace, kind: int, m: int, k: int, device, stream_handle: int):
    """(pointer, bytes) for a call: a Workspace, None (one-shot form), or "auto" = a
    workspace cached per (device, stream), grown to what the default shape uses."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, Workspace):
        workspace.used_on(stream_handle)
        return workspace.ptr(), workspace.nbytes
    if workspace != "auto":
        raise TypeError("workspace must be a Workspace, None or 'auto'")
    need = int(lib().vq_workspace_bytes(kind, m, k))
    if need == 0:
        return None, 0
    key = (str(device), stream_handle)
    with _auto_lock:
        ws = _auto_ws.get(key)
        if ws is None or ws.nbytes < need:
            ws = Workspace(need, device)
            _auto_ws[key] = ws
        ws.used_on(stream_handle)
    return ws.ptr(), ws.nbytes


def _kind(kind: str) -> int:
    if kind not in _KINDS:
        raise ValueError("kind must be one of %s" % sorted(_KINDS))
    return _KINDS[kind]


def workspace_bytes(kind: str, m: int, k: int) -> int:
    """Workspace bytes the default launch shape of an (M, K) verify GEMM uses
    (kind "q4_0", "fp8", "q4_0_panel" or "fp8_panel")."""
    return int(lib().vq_workspace_bytes(_kind(kind), m, k))


def gemm_q4_0(codes, scales, x, out, *, x_scales=None, alpha: float = 1.0, workspace="auto", stream=None,
              tiles_per_wave: int = 0, waves_per_group: int = 0, max_groups: int = 0):
    """out[N][M] = alpha * x[N][K] @ dequant(codes, scales)[M][K]^T.

    codes: uint8 [M][K/2]; scales: float16 [M][K/32]; x: float16 / bfloat16 [N][K]
    or int8 [N][K] with x_scales float16 [N][K/32]; out: float16 / bfloat16 /
    float32 [N][M].  workspace: "auto" (a cached per-stream Workspace), a
    Workspace, or None (the one-shot form).  tiles_per_wave / waves_per_group
    / max_groups select an explicit launch shape, the walk form when a
    workspace is given (float activations only; 0 = library default)."""
    N, K = x.shape
    M = codes.shape[0]
    _check_2d(codes, "codes", (M, K // 2))
    _check_2d(scales, "scales", (M, K // 32))
    _check_2d(out, "out", (N, M))
    act_dtype = _dtype_code(x)
    L = lib()
    sh = _stream(stream)
    if act_dtype == DTYPE_I8:
        if x_scales is None:
            raise ValueError("int8 activations need x_scales")
        _check_2d(x_scales, "x_scales", (N, K // 32))
        st = L.vq_gemm_q4_0(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), _dev_ptr(x, "x"),
                            act_dtype, _dev_ptr(x_scales, "x_scales"), _dev_ptr(out, "out"),
                            _dtype_code(out), N, M, K, float(alpha), None, 0, sh)
        _check(st, "vq_gemm_q4_0")
        return out
    if x_scales is not None:
        raise ValueError("x_scales only go with int8 activations")
    wp, wn = _workspace_args(workspace, KIND_Q4_0, M, K, codes.device, sh)
    if tiles_per_wave or waves_per_group or max_groups:
        st = L.vq_gemm_q4_0_ex(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), _dev_ptr(x, "x"),
                               act_dtype, _dev_ptr(out, "out"), _dtype_code(out), N, M, K,
                               float(alpha), int(tiles_per_wave), int(waves_per_group), int(max_groups),
                               wp, wn, sh)
        _check(st, "vq_gemm_q4_0_ex")
    else:
        st = L.vq_gemm_q4_0(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), _dev_ptr(x, "x"),
                            act_dtype, None, _dev_ptr(out, "out"), _dtype_code(out), N, M, K,
                            float(alpha), wp, wn, sh)
        _check(st, "vq_gemm_q4_0")
    return out


def gemm_q4_0_noalloc(codes, scales, x, out, *, x_scales=None, alpha: float = 1.0, stream=None):
    """gemm_q4_0 through the allocation-free entry point: no workspace, the
    library's fixed per-GPU scratch array instead (calls on one GPU must not
    overlap in time).  Same arguments and results as gemm_q4_0."""
    N, K = x.shape
    M = codes.shape[0]
    _check_2d(codes, "codes", (M, K // 2))
    _check_2d(scales, "scales", (M, K // 32))
    _check_2d(out, "out", (N, M))
    xs = None
    if _dtype_code(x) == DTYPE_I8:
        if x_scales is None:
            raise ValueError("int8 activations need x_scales")
        _check_2d(x_scales, "x_scales", (N, K // 32))
        xs = _dev_ptr(x_scales, "x_scales")
    elif x_scales is not None:
        raise ValueError("x_scales only go with int8 activations")
    st = lib().vq_gemm_q4_0_noalloc(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), _dev_ptr(x, "x"),
                                    _dtype_code(x), xs, _dev_ptr(out, "out"), _dtype_code(out), N, M, K,
                                    float(alpha), _stream(stream))
    _check(st, "vq_gemm_q4_0_noalloc")
    return out


def gemm_fp8_blk128(w, tile_scales, x, out, *, workspace="auto", stream=None, tiles_per_wave: int = 0,
                    waves_per_group: int = 0, max_groups: int = 0):
    """out[N][M] = x[N][K] @ (e4m3(w) * tile_scales[m/128][k/128])^T.

    w: uint8 [M][K] (E4M3FN bits); tile_scales: float32 [ceil(M/128)][K/128];
    x: float16 / bfloat16 [N][K]; out: float16 / bfloat16 / float32 [N][M]."""
    N, K = x.shape
    M = w.shape[0]
    _check_2d(w, "w", (M, K))
    _check_2d(tile_scales, "tile_scales", ((M + 127) // 128, K // 128))
    _check_2d(out, "out", (N, M))
    L = lib()
    sh = _stream(stream)
    wp, wn = _workspace_args(workspace, KIND_FP8_BLK128, M, K, w.device, sh)
    if tiles_per_wave or waves_per_group or max_groups:
        st = L.vq_gemm_fp8_blk128_ex(_dev_ptr(w, "w"), _dev_ptr(tile_scales, "tile_scales"), _dev_ptr(x, "x"),
                                     _dtype_code(x), _dev_ptr(out, "out"), _dtype_code(out), N, M, K,
                                     int(tiles_per_wave), int(waves_per_group), int(max_groups), wp, wn, sh)
        _check(st, "vq_gemm_fp8_blk128_ex")
    else:
        st = L.vq_gemm_fp8_blk128(_dev_ptr(w, "w"), _dev_ptr(tile_scales, "tile_scales"), _dev_ptr(x, "x"),
                                  _dtype_code(x), _dev_ptr(out, "out"), _dtype_code(out), N, M, K, wp, wn, sh)
        _check(st, "vq_gemm_fp8_blk128")
    return out


def q4_0_panel_bytes(m: int, k: int) -> int:
    """Bytes of the panel form of an M x K Q4_0 matrix (0 for invalid sizes)."""
    return int(lib().vq_q4_0_panel_bytes(m, k))


def q4_0_to_panel(codes, scales, panel=None, *, stream=None):
    """The panel form of Q4_0 weights (codes uint8 [M][K/2], scales float16
    [M][K/32]) as a uint8 device tensor of q4_0_panel_bytes(M, K) bytes
    (written into `panel` when given)."""
    torch = _torch()
    M, K = codes.shape[0], codes.shape[1] * 2
    _check_2d(scales, "scales", (M, K // 32))
    nbytes = q4_0_panel_bytes(M, K)
    if nbytes == 0:
        raise ValueError("invalid Q4_0 shape %s" % ((M, K),))
    if panel is None:
        panel = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    if panel.dtype != torch.uint8 or panel.numel() < nbytes:
        raise ValueError("panel must be a uint8 tensor of at least %d bytes" % nbytes)
    st = lib().vq_q4_0_to_panel(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), M, K,
                                _dev_ptr(panel, "panel"), panel.numel(), _stream(stream))
    _check(st, "vq_q4_0_to_panel")
    return panel


def gemm_q4_0_panel(panel, m: int, k: int, x, out, *, alpha: float = 1.0, workspace="auto", stream=None,
                    max_groups: int = 0):
    """gemm_q4_0 on panel weights (q4_0_to_panel) with float16 / bfloat16 x
    [N][K]; the walk form always (workspace "auto" or a Workspace)."""
    N, K = x.shape
    if K != k:
        raise ValueError("x has K = %d, the panel %d" % (K, k))
    _check_2d(out, "out", (N, m))
    if panel.numel() < q4_0_panel_bytes(m, k):
        raise ValueError("panel tensor is smaller than the panel form of (%d, %d)" % (m, k))
    L = lib()
    sh = _stream(stream)
    if workspace is None:
        raise ValueError("panel weights need a workspace")
    wp, wn = _workspace_args(workspace, KIND_Q4_0_PANEL, m, k, x.device, sh)
    if max_groups:
        st = L.vq_gemm_q4_0_panel_ex(_dev_ptr(panel, "panel"), _dev_ptr(x, "x"), _dtype_code(x),
                                     _dev_ptr(out, "out"), _dtype_code(out), N, m, k, float(alpha),
                                     int(max_groups), wp, wn, sh)
        _check(st, "vq_gemm_q4_0_panel_ex")
    else:
        st = L.vq_gemm_q4_0_panel(_dev_ptr(panel, "panel"), _dev_ptr(x, "x"), _dtype_code(x),
                                  _dev_ptr(out, "out"), _dtype_code(out), N, m, k, float(alpha), wp, wn, sh)
        _check(st, "vq_gemm_q4_0_panel")
    return out


def fp8_panel_bytes(m: int, k: int) -> int:
    """Bytes of the panel form of an M x K E4M3 matrix (0 for invalid sizes)."""
    return int(lib().vq_fp8_panel_bytes(m, k))


def fp8_to_panel(w, panel=None, *, stream=None):
    """The panel form of E4M3 weights (w uint8 [M][K]) as a uint8 device
    tensor of fp8_panel_bytes(M, K) bytes (written into `panel` when given).
    The tile scales are used as they are."""
    torch = _torch()
    M, K = w.shape
    _check_2d(w, "w", (M, K))
    nbytes = fp8_panel_bytes(M, K)
    if nbytes == 0:
        raise ValueError("invalid FP8 shape %s" % ((M, K),))
    if panel is None:
        panel = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if panel.dtype != torch.uint8 or panel.numel() < nbytes:
        raise ValueError("panel must be a uint8 tensor of at least %d bytes" % nbytes)
    st = lib().vq_fp8_to_panel(_dev_ptr(w, "w"), M, K, _dev_ptr(panel, "panel"), panel.numel(), _stream(stream))
    _check(st, "vq_fp8_to_panel")
    return panel


def gemm_fp8_blk128_panel(panel, tile_scales, x, out, *, workspace="auto", stream=None, max_groups: int = 0):
    """gemm_fp8_blk128 on panel weights (fp8_to_panel): tile_scales float32
    [ceil(M/128)][K/128], x float16 / bfloat16 [N][K], out [N][M]; the walk
    form always (workspace "auto" or a Workspace)."""
    N, K = x.shape
    M = out.shape[1]
    _check_2d(out, "out", (N, M))
    _check_2d(tile_scales, "tile_scales", ((M + 127) // 128, K // 128))
    if panel.numel() < fp8_panel_bytes(M, K):
        raise ValueError("panel tensor is smaller than the panel form of (%d, %d)" % (M, K))
    if workspace is None:
        raise ValueError("panel weights need a workspace")
    L = lib()
    sh = _stream(stream)
    wp, wn = _workspace_args(workspace, KIND_FP8_PANEL, M, K, x.device, sh)
    if max_groups:
        st = L.vq_gemm_fp8_blk128_panel_ex(_dev_ptr(panel, "panel"), _dev_ptr(tile_scales, "tile_scales"),
                                           _dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(out, "out"),
                                           _dtype_code(out), N, M, K, int(max_groups), wp, wn, sh)
        _check(st, "vq_gemm_fp8_blk128_panel_ex")
    else:
        st = L.vq_gemm_fp8_blk128_panel(_dev_ptr(panel, "panel"), _dev_ptr(tile_scales, "tile_scales"),
                                        _dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(out, "out"), _dtype_code(out),
                                        N, M, K, wp, wn, sh)
        _check(st, "vq_gemm_fp8_blk128_panel")
    return out


def gemm_fp8_blk128_prefill(w, tile_scales, x, out, *, stream=None):
    """gemm_fp8_blk128 for prompt-sized row counts (the MFMA-tiled kernel):
    w uint8 [M][K] (E4M3FN), tile_scales float32 [ceil(M/128)][K/128], x
    float16 / bfloat16 [N][K], out float16 / bfloat16 / float32 [N][M]."""
    N, K = x.shape
    M = w.shape[0]
    _check_2d(w, "w", (M, K))
    _check_2d(tile_scales, "tile_scales", ((M + 127) // 128, K // 128))
    _check_2d(out, "out", (N, M))
    st = lib().vq_gemm_fp8_blk128_prefill(_dev_ptr(w, "w"), _dev_ptr(tile_scales, "tile_scales"), _dev_ptr(x, "x"),
                                          _dtype_code(x), _dev_ptr(out, "out"), _dtype_code(out), N, M, K,
                                          _stream(stream))
    _check(st, "vq_gemm_fp8_blk128_prefill")
    return out


class GroupedCall:
    """A prepared grouped verify GEMM: the problem table is built once, so a
    repeated call (a decode step) costs one C call.

    problems: list of (w, scales, x, out) device tensors, all with the same
    x dtype, out dtype and row count; kind "q4_0" (w uint8 [M][K/2], scales
    float16 [M][K/32]), "fp8" (w uint8 [M][K], scales float32
    [ceil(M/128)][K/128]), "q4_0_panel" (w the panel form, scales the
    integer M) or "fp8_panel" (w the FP8 panel form, scales the tile scales;
    M is out's width).  workspace: a Workspace (grown here to what the group needs),
    "auto" (a new one of that size) or None (one-shot form; not for panels)."""

    def __init__(self, kind: str, problems, *, alpha: float = 1.0, workspace="auto"):
        self.kind = _kind(kind)
        if not problems:
            raise ValueError("empty group")
        self.alpha = float(alpha)
        x0, o0 = problems[0][2], problems[0][3]
        self.n_rows = x0.shape[0]
        self.act_dtype, self.out_dtype = _dtype_code(x0), _dtype_code(o0)
        self.table = (VerifyProblem * len(problems))()
        self._keep = []
        for i, (w, sc, x, out) in enumerate(problems):
            N, K = x.shape
            M = int(sc) if self.kind == KIND_Q4_0_PANEL else out.shape[1] if self.kind == KIND_FP8_PANEL \
                else w.shape[0]
            if N != self.n_rows or _dtype_code(x) != self.act_dtype or _dtype_code(out) != self.out_dtype:
                raise ValueError("problem %d: row count and dtypes must match the first problem" % i)
            if self.kind == KIND_Q4_0_PANEL:
                if w.numel() < q4_0_panel_bytes(M, K):
                    raise ValueError("problem %d: panel tensor too small" % i)
                _check_2d(out, "out", (N, M))
                self.table[i] = VerifyProblem(_dev_ptr(w, "w"), None, _dev_ptr(x, "x"), _dev_ptr(out, "out"),
                                              M, K)
                self._keep.append((w, x, out))
                continue
            if self.kind == KIND_Q4_0:
                _check_2d(w, "w", (M, K // 2))
                _check_2d(sc, "scales", (M, K // 32))
            elif self.kind == KIND_FP8_PANEL:
                if w.numel() < fp8_panel_bytes(M, K):
                    raise ValueError("problem %d: panel tensor too small" % i)
                _check_2d(sc, "scales", ((M + 127) // 128, K // 128))
            else:
                _check_2d(w, "w", (M, K))
                _check_2d(sc, "scales", ((M + 127) // 128, K // 128))
            _check_2d(out, "out", (N, M))
            self.table[i] = VerifyProblem(_dev_ptr(w, "w"), _dev_ptr(sc, "scales"), _dev_ptr(x, "x"),
                                          _dev_ptr(out, "out"), M, K)
            self._keep.append((w, sc, x, out))
        self.count = len(problems)
        need = int(lib().vq_workspace_bytes_grouped(self.kind, self.table, self.count))
        if workspace is None:
            if self.kind in (KIND_Q4_0_PANEL, KIND_FP8_PANEL):
                raise ValueError("panel weights need a workspace")
            self.ws = None
        elif isinstance(workspace, Workspace):
            self.ws = workspace if workspace.nbytes >= need else Workspace(need, x0.device)
        elif workspace == "auto":
            self.ws = Workspace(need, x0.device) if need else None
        else:
            raise TypeError("workspace must be a Workspace, None or 'auto'")
        self.workspace_bytes = need

    def __call__(self, stream=None):
        L = lib()
        sh = _stream(stream)
        if self.ws is not None:
            self.ws.used_on(sh)
        wp, wn = (self.ws.ptr(), self.ws.nbytes) if self.ws is not None else (None, 0)
        if self.kind == KIND_Q4_0:
            st = L.vq_gemm_q4_0_grouped(self.table, self.count, self.act_dtype, self.out_dtype, self.n_rows,
                                        self.alpha, wp, wn, sh)
            _check(st, "vq_gemm_q4_0_grouped")
        elif self.kind == KIND_Q4_0_PANEL:
            st = L.vq_gemm_q4_0_panel_grouped(self.table, self.count, self.act_dtype, self.out_dtype,
                                              self.n_rows, self.alpha, wp, wn, sh)
            _check(st, "vq_gemm_q4_0_panel_grouped")
        elif self.kind == KIND_FP8_PANEL:
            st = L.vq_gemm_fp8_blk128_panel_grouped(self.table, self.count, self.act_dtype, self.out_dtype,
                                                    self.n_rows, wp, wn, sh)
            _check(st, "vq_gemm_fp8_blk128_panel_grouped")
        else:
            st = L.vq_gemm_fp8_blk128_grouped(self.table, self.count, self.act_dtype, self.out_dtype,
                                              self.n_rows, wp, wn, sh)
            _check(st, "vq_gemm_fp8_blk128_grouped")


def gemm_q4_0_grouped(problems, *, alpha: float = 1.0, workspace="auto", stream=None):
    """Grouped Q4_0 verify GEMMs: problems = [(codes, scales, x, out), ...]."""
    GroupedCall("q4_0", problems, alpha=alpha, workspace=workspace)(stream)


def gemm_fp8_blk128_grouped(problems, *, workspace="auto", stream=None):
    """Grouped FP8 verify GEMMs: problems = [(w, tile_scales, x, out), ...]."""
    GroupedCall("fp8", problems, workspace=workspace)(stream)


def hadamard32_quant_int8(x, q_out, scales_out, *, stream=None):
    """Per 32-block: u = H32 x (fp32), d = fp16(amax/127), q = clamp(rint(u/d), +-127).

    x: float16 / bfloat16 [N][K]; q_out: int8 [N][K]; scales_out: float16 [N][K/32]."""
    N, K = x.shape
    _check_2d(q_out, "q_out", (N, K))
    _check_2d(scales_out, "scales_out", (N, K // 32))
    st = lib().vq_hadamard32_quant_int8(_dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(q_out, "q_out"),
                                        _dev_ptr(scales_out, "scales_out"), N, K, _stream(stream))
    _check(st, "vq_hadamard32_quant_int8")
    return q_out, scales_out


def hadamard32_quant_int4(x, q_out, scales_out, *, stream=None):
    """The 4-bit quantizer: per 32-block u = H32 x (fp32), d = fp16(amax/7),
    q = clamp(rint(u/d), +-7), codes one per byte (gemm_q4_0 reads them as int8).

    x: float16 / bfloat16 [N][K]; q_out: int8 [N][K]; scales_out: float16 [N][K/32]."""
    N, K = x.shape
    _check_2d(q_out, "q_out", (N, K))
    _check_2d(scales_out, "scales_out", (N, K // 32))
    st = lib().vq_hadamard32_quant_int4(_dev_ptr(x, "x"), _dtype_code(x), _dev_ptr(q_out, "q_out"),
                                        _dev_ptr(scales_out, "scales_out"), N, K, _stream(stream))
    _check(st, "vq_hadamard32_quant_int4")
    return q_out, scales_out


def q4_0_rotate_h32(codes, scales, codes_out=None, scales_out=None, *, stream=None):
    """The offline H32 rotation of Q4_0 weights for the W4A8 path: returns the
    rotated, requantized (codes uint8 [M][K/2], scales float16 [M][K/32])."""
    torch = _torch()
    M, K = codes.shape[0], codes.shape[1] * 2
    _check_2d(scales, "scales", (M, K // 32))
    if codes_out is None:
        codes_out = torch.empty_like(codes)
    if scales_out is None:
        scales_out = torch.empty_like(scales)
    _check_2d(codes_out, "codes_out", (M, K // 2))
    _check_2d(scales_out, "scales_out", (M, K // 32))
    st = lib().vq_q4_0_rotate_h32(_dev_ptr(codes, "codes"), _dev_ptr(scales, "scales"), M, K,
                                  _dev_ptr(codes_out, "codes_out"), _dev_ptr(scales_out, "scales_out"),
                                  _stream(stream))
    _check(st, "vq_q4_0_rotate_h32")
    return codes_out, scales_out


def greedy_workspace_bytes(n_rows: int, vocab: int) -> int:
    """Workspace bytes of greedy_verify for a block of n_rows over vocab (0 if invalid)."""
    return int(lib().vq_greedy_workspace_bytes(n_rows, vocab))


def greedy_verify(logits, draft, tokens_out=None, count_out=None, *, workspace="auto", stream=None):
    """Greedy acceptance of a draft block: logits float32 / float16 / bfloat16
    [n][V], draft int32 [n - 1].  Returns (tokens_out int32 [n], count_out
    int32 [1]) on the device: the target's choice per row and the number of
    committed tokens (tokens_out[:count] are committed).  workspace: "auto"
    (a cached one per device and stream) or a Workspace."""
    torch = _torch()
    n, v = logits.shape
    if draft is None:
        if n != 1:
            raise ValueError("draft must hold n_rows - 1 tokens")
    elif draft.dtype != torch.int32 or draft.numel() != n - 1:
        raise ValueError("draft must be int32 with n_rows - 1 tokens")
    if tokens_out is None:
        tokens_out = torch.empty(n, dtype=torch.int32, device=logits.device)
    if count_out is None:
        count_out = torch.empty(1, dtype=torch.int32, device=logits.device)
    need = greedy_workspace_bytes(n, v)
    sh = _stream(stream)
    if isinstance(workspace, Workspace):
        ws = workspace
    elif workspace == "auto":
        key = ("greedy", str(logits.device), sh)
        with _auto_lock:
            ws = _auto_ws.get(key)
            if ws is None or ws.nbytes < need:
                ws = Workspace(need, logits.device)
                _auto_ws[key] = ws
    else:
        raise TypeError("workspace must be a Workspace or 'auto'")
    ws.used_on(sh)
    dptr = _dev_ptr(draft, "draft") if (draft is not None and draft.numel()) else None
    st = lib().vq_greedy_verify(_dev_ptr(logits, "logits"), _dtype_code(logits), n, v, dptr,
                                _dev_ptr(tokens_out, "tokens_out"), _dev_ptr(count_out, "count_out"),
                                ws.ptr(), ws.nbytes, sh)
    _check(st, "vq_greedy_verify")
    return tokens_out, count_out


def default_launch_shape(kind: str, m: int, k: int, workspace_bytes=None):
    """(tiles_per_wave, waves_per_group, walk, workspace_used) the library
    picks for an (M, K) verify GEMM given workspace_bytes (None = unlimited);
    walk is 1 for the walk form, 0 for one-shot."""
    t, w, s = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    used = ctypes.c_size_t(0)
    cap = (1 << 64) - 1 if workspace_bytes is None else int(workspace_bytes)
    _check(lib().vq_default_launch_shape(_kind(kind), m, k, cap,
                                         ctypes.byref(t), ctypes.byref(w), ctypes.byref(s), ctypes.byref(used)),
           "vq_default_launch_shape")
    return t.value, w.value, s.value, used.value


def hbm_read_probe(buf, sink, *, mode: str = "blocks", groups: int = 0, waves_per_group: int = 8, depth: int = 8,
                   nontemporal: bool = False, stream=None):
    """One plain read of the device tensor `buf` (its bytes, a multiple of
    64 KiB up to 2 GiB) by the probe kernel; sink: a device tensor of >= 4
    bytes.  mode "blocks" (one workgroup per 64 KiB; groups 0), "shares"
    (`groups` persistent workgroups, contiguous shares), "window" (`groups`
    persistent workgroups sweeping 64 KiB blocks) or "reread" (as "shares",
    each share read PROBE_REREAD_PASSES times within the launch: the rate of
    L2 hits once a share fits in L2) or "lds" (`groups` workgroups each copy
    the first 64 KiB into LDS and read the buffer's byte count from LDS: the
    LDS read rate per CU; nontemporal False); nontemporal: the loads' cache
    policy."""
    if mode not in _PROBES:
        raise ValueError("mode must be one of %s" % sorted(_PROBES))
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold 4 bytes")
    st = lib().vq_hbm_read_probe(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(), _PROBES[mode],
                                 int(groups), int(waves_per_group), int(depth), int(bool(nontemporal)),
                                 _dev_ptr(sink, "sink"),
                                 _stream(stream))
    _check(st, "vq_hbm_read_probe")
