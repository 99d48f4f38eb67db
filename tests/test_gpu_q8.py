"""Decode GEMV against the per-token int8 activations of the prefill path
(tl_gemv_ternary_q8) checked against the oracle of the same computation, on the
layer shapes, ragged shapes and an odd group count, for both the LDS-staged and
the register variant; the error against the exact layer is reported beside it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, announce, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import quantized_gemv_gemm_amd as m
    m.lib()
    return m


CASES = [(1024, 256, 1), (5120, 10240, 1), (5120, 10240, 4), (5120, 10240, 8), (5120, 10240, 16),
         (17408, 5120, 1), (17408, 5120, 16), (5120, 34816, 16), (3072, 77, 5), (384, 40, 3), (1024, 300, 13)]


@pytest.mark.parametrize("K,N,b", CASES)
def test_gemv_q8_matches_oracle(tl, K, N, b):
    import torch
    d = dev()
    announce(f"gemv_ternary_q8 K={K} N={N} b={b}")
    rng = np.random.default_rng(7 * K + N + b)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    packed, _, _ = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    s_d = to_dev(scales, d)
    if K % 1024 == 0:
        xbits = synth.activations(0, 1, 13, b, K)
        xr = oracle.rotate_f32(synth.bf16_bits_to_f32(xbits))
        xq_d, sx_d = tl.quant_act_int8_x(bf16_dev(xbits, d))
    else:  # no whole rotation blocks: quantise a synthetic rotated row directly
        xr = rng.standard_normal((b, K)).astype(np.float32)
        xq_d, sx_d = tl.quant_act_int8(to_dev(xr, d))
    xq_ref, sx_ref = oracle.quant_act_int8(xr)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq_d.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(sx_d.cpu().numpy(), sx_ref)
    y = torch.full((b, N), float("nan"), dtype=torch.float32, device=d)
    tl.gemv_ternary_q8(xq_d, sx_d, packed, s_d, out=y)
    name = tl.last_kernel_name()
    yb = tl.gemv_ternary_q8(xq_d, sx_d, packed, s_d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.gemv_ternary_q8(xq_ref, sx_ref, codes, scales)
    e = oracle.rel_fro(y.cpu().numpy(), ref)
    assert e <= REL_TOL, (name, e)
    eb = oracle.rel_fro(yb.float().cpu().numpy(), oracle.bf16_round(ref))
    assert eb <= REL_TOL, (name, eb)
    exact = oracle.gemv_ternary(xr.astype(np.float64), codes, scales)
    print(f"[gpu-case] {name}: vs same-path oracle {e:.2e}, vs exact layer {oracle.rel_fro(y.cpu().numpy(), exact):.2e}",
          flush=True)
    assert name.startswith("gemv_q8_")


def test_gemv_q8_zero_token(tl):
    """A token whose activations are all zero (sx = 0) gives y = 0, not NaN."""
    import torch
    d = dev()
    K, N = 1024, 64
    x = torch.zeros((2, K), dtype=torch.bfloat16, device=d)
    x[0, 3] = 2.0
    xq, sx = tl.quant_act_int8_x(x)
    codes = torch.ones((N, K), dtype=torch.int8, device=d)
    scales = torch.ones((N, K // 128), dtype=torch.float16, device=d)
    packed, _, _ = tl.pack_weights(codes, scales)
    y = tl.gemv_ternary_q8(xq, sx, packed, scales, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and float(y[1].abs().max()) == 0.0
