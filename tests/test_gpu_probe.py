"""The HBM read probe on the GPU: every pattern runs and writes nothing (a
buffer of zeros folds to an XOR of zero, never the probe's constant); the
LDS form likewise, also on a buffer whose words do not fold to zero."""
import pytest
import torch

import block_quantized_gemm_amd as vq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,groups", [("blocks", 0), ("shares", 16), ("window", 7), ("window", 300),
                                         ("reread", 16), ("reread", 256)])
@pytest.mark.parametrize("waves,depth", [(4, 16), (8, 8), (16, 4)])
@pytest.mark.parametrize("nt", [False, True])
def test_probe_patterns_run_and_write_nothing(mode, groups, waves, depth, nt):
    buf = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 0x55, dtype=torch.uint8, device="cuda")
    vq.hbm_read_probe(buf, sink, mode=mode, groups=groups, waves_per_group=waves, depth=depth, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.all(sink == 0x55)


@pytest.mark.parametrize("groups", [1, 256, 600])
@pytest.mark.parametrize("waves,depth", [(4, 16), (8, 8), (16, 4)])
@pytest.mark.parametrize("nbytes", [64 << 10, 1 << 20])
def test_lds_probe_runs_and_writes_nothing(groups, waves, depth, nbytes):
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda").view(torch.uint8)
    sink = torch.full((4,), 0x55, dtype=torch.uint8, device="cuda")
    vq.hbm_read_probe(buf, sink, mode="lds", groups=groups, waves_per_group=waves, depth=depth)
    torch.cuda.synchronize()
    assert torch.all(sink == 0x55)
