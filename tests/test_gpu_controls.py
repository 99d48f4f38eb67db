"""Negative controls of the parity checks.  Each GPU result is compared twice:
with the oracle, where it must pass, and with the oracle fed one planted mistake
of a kind a kernel could make, where the same comparison must fail by a wide
margin.  The planted mistakes are
  * the sign vector not applied (rotation of x instead of d * x);
  * the two 512-wide halves of a Hadamard block swapped;
  * a transposed weight layout (a square layer read as W^T);
  * the group scales (GEMV) or the int8 scale factors q (GEMM) taken one group off;
  * two tokens' rows exchanged.
They live on the CPU side only: the GPU path runs exactly as in the other tests.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, announce, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu

K, N, T = 2048, 2048, 3   # square, so that a transposed layout has the same shape


@pytest.fixture(scope="module")
def case():
    import torch
    import quantized_gemv_gemm_amd as tl
    d = dev()
    rng = np.random.default_rng(2024)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    signs = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    xbits = synth.activations(0, 1, 21, T, K)
    x = bf16_dev(xbits, d)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    sd = to_dev(scales, d)
    announce(f"negative controls K={K} N={N} T={T}")
    y = tl.gemv_ternary_x(x, packed, sd, signs=to_dev(signs, d), out_dtype=torch.float32)
    xq, sx = tl.quant_act_int8_x(x, to_dev(signs, d))
    _, acc = tl.gemm_int8_rescale(xq, sx, packed, q, rs, out_dtype=torch.float32, want_acc=True)
    torch.cuda.synchronize()
    return dict(codes=codes, scales=scales, signs=signs, xf=synth.bf16_bits_to_f32(xbits),
                y=y.cpu().numpy(), acc=acc.cpu().numpy().astype(np.int64), xq=xq.cpu().numpy())


def _swap_halves(xr):
    """Each 1024-block's two 512-wide halves exchanged."""
    out = xr.copy()
    for j in range(0, xr.shape[1], 1024):
        out[:, j:j + 512], out[:, j + 512:j + 1024] = xr[:, j + 512:j + 1024], xr[:, j:j + 512]
    return out


def _shift_groups(a):
    """Per-row group values taken one group off (group g reads group g + 1, cyclically)."""
    return np.roll(a, -1, axis=1)


def _gemv_mutants(c):
    xr = oracle.rotate_exact(c["xf"], c["signs"])
    yield "no signs", oracle.gemv_ternary(oracle.rotate_exact(c["xf"]), c["codes"], c["scales"])
    yield "halves swapped", oracle.gemv_ternary(_swap_halves(xr), c["codes"], c["scales"])
    yield "transposed W", oracle.gemv_ternary(xr, np.ascontiguousarray(c["codes"].T),
                                              c["scales"])
    yield "scales one group off", oracle.gemv_ternary(xr, c["codes"], _shift_groups(c["scales"]))
    yield "tokens exchanged", oracle.gemv_ternary(xr[[1, 0, 2]], c["codes"], c["scales"])


def test_gemv_controls(case):
    c = case
    xr = oracle.rotate_exact(c["xf"], c["signs"])
    e = oracle.rel_fro(c["y"], oracle.gemv_ternary(xr, c["codes"], c["scales"]))
    assert e <= REL_TOL, e
    for label, ref in _gemv_mutants(c):
        em = oracle.rel_fro(c["y"], ref)
        announce(f"  GEMV vs oracle with {label}: rel_fro {em:.3f} (vs the oracle itself {e:.1e})")
        assert em > 100 * REL_TOL, (label, em)


def test_gemm_controls(case):
    c = case
    q, _, _ = oracle.decompose_scales(c["scales"])
    xq_ref, _ = oracle.quant_act_int8(oracle.rotate_f32(c["xf"], c["signs"]))
    np.testing.assert_array_equal(c["xq"], xq_ref)
    acc_ref = oracle.gemm_int8_acc(xq_ref, c["codes"], q)
    np.testing.assert_array_equal(c["acc"], acc_ref)
    xq_nosign, _ = oracle.quant_act_int8(oracle.rotate_f32(c["xf"]))
    mutants = {
        "no signs": oracle.gemm_int8_acc(xq_nosign, c["codes"], q),
        "transposed W": oracle.gemm_int8_acc(xq_ref, np.ascontiguousarray(c["codes"].T), q),
        "q one group off": oracle.gemm_int8_acc(xq_ref, c["codes"], _shift_groups(q)),
        "tokens exchanged": acc_ref[[1, 0, 2]],
    }
    for label, ref in mutants.items():
        differ = float(np.mean(c["acc"] != ref))
        announce(f"  GEMM int32 vs oracle with {label}: {differ:.3f} of the accumulators differ")
        assert differ > 0.5, (label, differ)
