"""Shared test utilities: parity metrics and numpy-bits -> torch-device marshalling."""
from __future__ import annotations

import numpy as np

# Parity bar for floating-point outputs (per the verify-GEMM contract):
#   relative Frobenius error <= 2e-3, and every element within 1e-2 * ||oracle row||_2.
REL_FROB = 2e-3
ROW_REL = 1e-2


# Below this many elements a Frobenius ratio measures single roundings, not the
# kernel: a lone bf16 output already carries up to 2^-8 relative error.
FROB_MIN_ELEMS = 256

_ULP_BITS = {"bf16": 8, "f16": 11, "f32": 24}   # significand bits incl. the implicit one
_MIN_NORMAL = {"bf16": 2.0 ** -126, "f16": 2.0 ** -14, "f32": 2.0 ** -126}


def ulp(values, out_dtype):
    """Spacing of the output type's values at |values| (subnormal spacing below)."""
    v = np.maximum(np.abs(np.asarray(values, dtype=np.float64)), _MIN_NORMAL[out_dtype])
    return np.exp2(np.floor(np.log2(v)) - (_ULP_BITS[out_dtype] - 1))


def accumulation_slack(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-element bound on fp32 accumulation error for Y = x @ w.T: the dot's
    absolute sum is at most ||x_n|| ||w_m|| (Cauchy-Schwarz), and a length-K fp32
    sum in any tree order errs by about sqrt(K) roundings of 2^-24 of it; the
    factor 4 leaves margin.  x [N][K], w [M][K] as float64."""
    K = x.shape[1]
    return 4.0 * np.sqrt(K) * 2.0 ** -24 * np.outer(np.linalg.norm(x, axis=1), np.linalg.norm(w, axis=1))


def parity(y_gpu: np.ndarray, y_ref: np.ndarray, out_dtype=None, rel_frob=REL_FROB, row_rel=ROW_REL,
           slack=None):
    """GPU output vs the exact (fp64, unrounded) oracle.

    Bar: relative Frobenius error <= 2e-3 (outputs with >= 256 elements) and
    every element within 1e-2 * ||oracle row||_2.  With out_dtype given, also
    every element within one output ulp of the oracle value plus 1e-4 of the
    row's RMS plus `slack` (an optional per-element accumulation bound, see
    accumulation_slack: needed where a near-zero output comes from cancelling
    terms, e.g. rows of very few elements in fp32).
    Returns (rel_frob, worst_row_ratio, worst_ulps)."""
    y = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    fro = np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-300)
    rown = np.linalg.norm(r, axis=1, keepdims=True)
    err = np.abs(y - r)
    worst = np.max(err / np.maximum(rown, 1e-300))
    if y.size >= FROB_MIN_ELEMS:
        assert fro <= rel_frob, "relative Frobenius error %.3e > %.1e" % (fro, rel_frob)
    assert worst <= row_rel, "per-element error %.3e of row norm > %.1e" % (worst, row_rel)
    worst_ulps = float("nan")
    if out_dtype is not None:
        rms = rown / np.sqrt(r.shape[1])
        u = ulp(r, out_dtype)
        worst_ulps = float(np.max(err / u))
        bad = err > u + 1e-4 * rms + (0.0 if slack is None else slack)
        assert not bad.any(), "%d elements beyond 1 ulp + 1e-4 rms (worst %.2f ulp)" % (bad.sum(), worst_ulps)
    return fro, worst, worst_ulps


def to_dev(a: np.ndarray, dtype=None, device="cuda"):
    """numpy array of raw bits -> torch device tensor, reinterpreted as `dtype`."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16).copy())
    else:
        t = torch.from_numpy(a.copy())
    t = t.to(device)
    if dtype is not None and dtype != t.dtype:
        t = t.view(dtype)
    return t


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits_u16(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)
