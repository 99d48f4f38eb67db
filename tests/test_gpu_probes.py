"""The two measurement probes launch and finish on the device.  Each writes its
sink only when its folded value equals one fixed marker word: over zero bytes
the read probe folds to 0, so its sink stays 0; the matrix-core probe's sink
holds either 0 or the marker."""
from __future__ import annotations

import pytest

from gpu_common import announce, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import quantized_gemv_gemm_amd as m
    m.lib()
    return m


def test_read_probe_runs(tl):
    import torch
    d = dev()
    announce("read_probe 1 MiB of zeros")
    src = torch.zeros((1 << 20,), dtype=torch.uint8, device=d)
    sink = torch.zeros((4,), dtype=torch.int32, device=d)
    tl.read_probe(src, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0      # the xor of zero words is 0, never the marker word


@pytest.mark.parametrize("random_operands", [False, True])
def test_mfma_probe_runs(tl, random_operands):
    import torch
    d = dev()
    announce(f"mfma_probe random={random_operands} iters=4")
    sink = torch.zeros((4,), dtype=torch.int32, device=d)
    tl.mfma_probe(random_operands, 4, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) in (0, 0x2545F491)
