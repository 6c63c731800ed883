"""Greedy verification on the GPU, through the C ABI, against the CPU oracle:
the target's choice per row and the committed count are exact integers, so
they must match bit for bit."""
import numpy as np
import pytest
import torch

import block_quantized_gemm_amd as vq
import oracle
import workloads as W
from helpers import to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16), "f16": (torch.float16, oracle.F16)}


def _logits(n, v, g, kind="normal"):
    x = g.standard_normal((n, v)).astype(np.float32)
    if kind == "ties":       # few distinct values: many equal maxima
        x = np.round(x * 2) / 2
    return x


def _as(x, dt):
    if dt == "f32":
        return x.astype(np.float32)
    return W.f32_to_bf16_bits(x) if dt == "bf16" else W.f32_to_f16_bits(x)


def _run(bits, dt, draft):
    tdt, _ = DT[dt]
    lg = to_dev(bits, tdt) if dt != "f32" else torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    d = torch.from_numpy(np.asarray(draft, dtype=np.int32)).cuda()
    tokens, count = vq.greedy_verify(lg, d)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), int(count.cpu().item())


def _drafts(target, g):
    """Draft blocks that agree with the target's choices for 0, 1, ..., all
    leading positions (and disagree right after)."""
    n = len(target)
    out = []
    for a in sorted({0, 1, n // 2, n - 2, n - 1}):
        if a < 0 or a > n - 1:
            continue
        d = target[:n - 1].copy()
        if a < n - 1:
            d[a] = target[a] + 1
            d[a + 1:] = g.integers(0, 1 << 20, size=n - 1 - a - 1) if n - 1 - a - 1 > 0 else d[a + 1:]
        out.append((a, d.astype(np.int32)))
    return out


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n,v,kind", [(1, 1, "normal"), (2, 5, "ties"), (8, 4096, "normal"), (16, 4097, "ties"),
                                      (16, 151936, "normal"), (17, 30000, "ties"), (100, 1000, "ties")])
def test_choices_and_count_match_oracle(dt, n, v, kind):
    g = np.random.Generator(np.random.PCG64(601 + n + v))
    bits = _as(_logits(n, v, g, kind), dt)
    target, _ = oracle.greedy_verify(bits, DT[dt][1], np.zeros(n - 1, np.int32))
    for a, draft in _drafts(target, g):
        t, c = _run(bits, dt, draft)
        assert np.array_equal(t, target)
        ref_t, ref_c = oracle.greedy_verify(bits, DT[dt][1], draft)
        assert c == ref_c == a + 1


def test_special_values():
    """NaN wins (its first position), -0 equals +0, infinities order normally,
    equal maxima resolve to the first index, in every segment position."""
    g = np.random.Generator(np.random.PCG64(610))
    n, v = 8, 20000
    x = g.standard_normal((n, v)).astype(np.float32)
    x[0, [9000, 15000]] = np.nan
    x[0, 3] = np.inf
    x[1] = -np.inf
    x[1, [19999, 12345]] = [0.0, -0.0]
    x[2, [4095, 4096, 19999]] = 50.0
    x[3, v - 1] = 1e30
    x[4] = 0.0
    x[5, 0] = np.inf
    x[5, 7] = np.inf
    x[6, :] = -1e30
    x[7, 12288] = np.nan
    t, c = _run(x, "f32", np.zeros(n - 1, np.int32))
    ref, ref_c = oracle.greedy_verify(x, oracle.F32, np.zeros(n - 1, np.int32))
    assert np.array_equal(t, ref) and c == ref_c
    assert list(t) == [9000, 12345, 4095, v - 1, 0, 0, 0, 12288]


def test_one_row_block_commits_the_target_token():
    g = np.random.Generator(np.random.PCG64(611))
    x = g.standard_normal((1, 777)).astype(np.float32)
    lg = torch.from_numpy(x).cuda()
    tokens, count = vq.greedy_verify(lg, None)
    torch.cuda.synchronize()
    assert int(count.item()) == 1 and int(tokens.item()) == int(np.argmax(x[0]))


def test_workspace_reused_with_any_contents():
    g = np.random.Generator(np.random.PCG64(612))
    ws = vq.Workspace(vq.greedy_workspace_bytes(16, 151936))
    ws.tensor.fill_(0xFF)
    for v in (151936, 5000, 64):
        x = g.standard_normal((16, v)).astype(np.float32)
        lg = torch.from_numpy(x).cuda()
        target, _ = oracle.greedy_verify(x, oracle.F32, np.zeros(15, np.int32))
        d = torch.from_numpy(target[:15].copy()).cuda()
        tokens, count = vq.greedy_verify(lg, d, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(tokens.cpu().numpy(), target) and int(count.item()) == 16
