"""The layer's calls captured in a HIP graph and replayed: a decode step (fused
rotation + limb prep, then the GEMV) and a prefill step (fused rotation +
int8 quantisation, then the K-split int8 GEMM, whose counters every call must
leave at zero for the next replay).  Every replay, with eager work and a
synchronisation in between, must reproduce the eager result bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_common import announce, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import quantized_gemv_gemm_amd as m
    m.lib()
    return m


def test_graph_replay_decode_and_prefill(tl):
    import torch
    d = dev()
    K, N = 2048, 1000
    rng = np.random.default_rng(99)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    sd = to_dev(scales, d)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), sd)
    Td, Tp = 4, 200
    assert tl.linear_path(Td, K, N) == tl.PATH_GEMV and tl.linear_path(Tp, K, N) == tl.PATH_INT8
    assert tl.gemm_workspace_size(Tp, K, N) > 0        # the prefill GEMM is split along K
    xd = bf16_dev(synth.activations(0, 1, 21, Td, K), d)
    xp = bf16_dev(synth.activations(0, 3, 21, Tp, K), d)
    # workspaces and outputs allocated (and the workspaces zero-filled) before capture
    wsd = torch.zeros((tl.linear_workspace_size(Td, K, N),), dtype=torch.uint8, device=d)
    wsp = torch.zeros((tl.linear_workspace_size(Tp, K, N),), dtype=torch.uint8, device=d)
    yd = torch.empty((Td, N), dtype=torch.float32, device=d)
    yp = torch.empty((Tp, N), dtype=torch.bfloat16, device=d)

    def step():
        tl.linear_apply(xd, packed, sd, q, rs, out=yd, workspace=wsd)
        tl.linear_apply(xp, packed, sd, q, rs, out=yp, workspace=wsp)

    step()
    torch.cuda.synchronize()
    ref_d, ref_p = yd.clone(), yp.clone()
    announce(f"graph capture: decode T={Td} ({tl.last_kernel_name()} last), prefill T={Tp}, K={K} N={N}")
    side = torch.cuda.Stream(d)
    side.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(side):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream(d).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for r in range(4):
        yd.fill_(float("nan"))      # eager work between replays
        yp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        announce(f"  replay {r}")
        assert torch.equal(yd, ref_d) and torch.equal(yp.view(torch.int16), ref_p.view(torch.int16))
        assert int(wsp[:1024].count_nonzero()) == 0    # split-K counters back at zero
