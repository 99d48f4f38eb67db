"""Fused layer inputs: rotation -> GEMV limbs and rotation -> int8, checked bit-exactly
against the unfused sequence (rotation kernel, then prep or quantisation) and
against the oracle, with and without a sign table."""
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


def _signs(K, seed):
    return np.where(np.random.default_rng(seed).random(K) < 0.5, -1, 1).astype(np.int8)


def _limb_region(b, K):
    return 32 * K * ((b + 15) // 16) if b > 8 else 2 * b * (K + 16)


def _limbs(ws, b, K):
    """hi and lo limb rows [b, K] and the limb scales [b, K/1024] from a GEMV workspace: rows
    K + 16 bytes apart for b <= 8; for b > 8 the matrix-core operand order (chunks
    of 16 tokens 32 K bytes apart; in a chunk, per 128-group, 64-k half and limb:
    64 lanes x 16 bytes, lane = row + 16 (k%128)//32, row = 4 (t % 4) + (t % 16) // 4)."""
    a = ws.cpu().numpy()
    if b <= 8:
        Kp = K + 16
        hi = np.stack([a[t * Kp:t * Kp + K] for t in range(b)])
        lo = np.stack([a[(b + t) * Kp:(b + t) * Kp + K] for t in range(b)])
    else:
        k = np.arange(K)
        g, kk = k // 128, k % 128
        hi, lo = np.empty((b, K), np.uint8), np.empty((b, K), np.uint8)
        for t in range(b):
            row = 4 * (t % 4) + (t % 16) // 4
            base = 32 * K * (t // 16) + \
                (((g * 2 + (kk // 16) % 2) * 2) * 64 + row + 16 * (kk // 32)) * 16 + kk % 16
            hi[t] = a[base]
            lo[t] = a[base + 64 * 16]
    off = (_limb_region(b, K) + 255) // 256 * 256
    nbk = (K + 1023) // 1024
    return hi, lo, a[off:off + 4 * b * nbk].view(np.float32).reshape(b, nbk)


def _expected_limbs(xr):
    """The limb split of f32 rows xr [b, K] (K % 1024 == 0), per token and 1024-block:
    sigma = |x|max / 32639 and q = clamp(RNE(fl32(x * fl32(32639 / |x|max))), +-32639),
    every step in binary32 as the kernels take it (q decides integers)."""
    b, K = xr.shape
    blk = xr.reshape(b, K // 1024, 1024)
    amax = np.abs(blk).max(axis=2)
    sigma = (amax / np.float32(32639.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(32639.0) / np.where(amax > 0, amax, np.float32(1)), 0).astype(np.float32)
    q = np.rint((blk * inv[..., None]).astype(np.float32)).clip(-32639, 32639).astype(np.int32)
    return sigma, q.reshape(b, K)


@pytest.mark.parametrize("K,b,signed", [(1024, 1, False), (5120, 4, True), (5120, 16, False),
                                        (17408, 1, True), (17408, 3, False), (33792, 2, True),
                                        (2048, 17, True), (5120, 40, False), (1024, 64, False)])
def test_gemv_prepare_fused_bitexact(tl, K, b, signed):
    import torch
    d = dev()
    announce(f"gemv_prepare_x K={K} b={b} signed={signed}")
    xbits = synth.activations(0, 1, 7, b, K)
    x = bf16_dev(xbits, d)
    signs = to_dev(_signs(K, K + b), d) if signed else None
    need = tl.gemv_workspace_size(b, K, 256)
    w_ref = torch.zeros((need,), dtype=torch.uint8, device=d)
    w_fus = torch.full((need,), 0x5A, dtype=torch.uint8, device=d)
    tl.gemv_prepare(tl.hadamard_blk(x, signs), w_ref)
    tl.gemv_prepare_x(x, w_fus, signs)
    torch.cuda.synchronize()
    h0, l0, s0 = _limbs(w_ref, b, K)
    h1, l1, s1 = _limbs(w_fus, b, K)
    np.testing.assert_array_equal(h1, h0)
    np.testing.assert_array_equal(l1, l0)
    np.testing.assert_array_equal(s1, s0)
    # the limbs are the fixed-point split of the oracle's f32 rotation, per 1024-block
    xr = oracle.rotate_f32(synth.bf16_bits_to_f32(xbits), _signs(K, K + b) if signed else None)
    sigma, q = _expected_limbs(xr)
    np.testing.assert_array_equal(s0, sigma)
    v = h0.astype(np.int8).astype(np.int32) * 256 + l0.astype(np.int8).astype(np.int32)
    np.testing.assert_array_equal(v, q)
    assert np.abs(v).max() <= 32639


@pytest.mark.parametrize("K,N,b", [(5120, 1000, 1), (5120, 10240, 8), (17408, 512, 2),
                                   (5120, 1000, 33), (3072, 300, 64), (2048, 1000, 2), (5120, 3000, 2)])
def test_gemv_ternary_fused_matches(tl, K, N, b):
    import torch
    d = dev()
    announce(f"gemv_ternary_x K={K} N={N} b={b}")
    rng = np.random.default_rng(K + N + b)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    packed, _, _ = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    xbits = synth.activations(0, 1, 9, b, K)
    x = bf16_dev(xbits, d)
    s_d = to_dev(scales, d)
    y_ref = tl.gemv_ternary(tl.hadamard_blk(x), packed, s_d, out_dtype=torch.float32)
    y_fus = tl.gemv_ternary_x(x, packed, s_d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_fused_vs_sequence(tl, y_fus.cpu().numpy(), y_ref.cpu().numpy())
    ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(xbits)), codes, scales)
    assert oracle.rel_fro(y_fus.cpu().numpy(), ref) <= REL_TOL


def _check_fused_vs_sequence(tl, y_fus, y_seq):
    """The prep + GEMV pair is bit-identical to the rotation kernel + GEMV; the
    one-launch kernel (one or two tokens) has the same limbs but adds the groups'
    results in another order, so it differs from them by float rounding alone:
    both lie within about 3e-5 of the exact layer."""
    kname = tl.last_kernel_name()
    if kname.startswith("gemv_rot"):
        e = oracle.rel_fro(y_fus, y_seq)
        announce(f"  one launch ({kname}): rel_fro vs rotation + GEMV = {e:.3e}")
        assert e <= 2e-4
    else:
        np.testing.assert_array_equal(y_fus, y_seq)


@pytest.mark.parametrize("T,K,signed", [(1, 1024, False), (7, 5120, True), (64, 17408, False),
                                        (33, 17408, True), (300, 5120, False)])
def test_quant_fused_bitexact(tl, T, K, signed):
    import torch
    d = dev()
    announce(f"quant_act_int8_x T={T} K={K} signed={signed}")
    xbits = synth.activations(0, 3, 5, T, K)
    x = bf16_dev(xbits, d)
    sg = _signs(K, T + K) if signed else None
    signs = to_dev(sg, d) if signed else None
    xq0, sx0 = tl.quant_act_int8(tl.hadamard_blk(x, signs))
    xq1, sx1 = tl.quant_act_int8_x(x, signs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xq1.cpu().numpy(), xq0.cpu().numpy())
    np.testing.assert_array_equal(sx1.cpu().numpy(), sx0.cpu().numpy())
    xq_ref, sx_ref = oracle.quant_act_int8(oracle.rotate_f32(synth.bf16_bits_to_f32(xbits), sg))
    np.testing.assert_array_equal(xq1.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(sx1.cpu().numpy(), sx_ref)


def test_quant_fused_zero_token(tl):
    """A token of zeros: sx = 0 and xq = 0 (no division by zero)."""
    import torch
    d = dev()
    x = torch.zeros((3, 2048), dtype=torch.bfloat16, device=d)
    x[1, 5] = 1.0
    xq, sx = tl.quant_act_int8_x(x)
    torch.cuda.synchronize()
    assert float(sx[0]) == 0.0 and float(sx[2]) == 0.0 and float(sx[1]) > 0.0
    assert int(xq[0].abs().sum()) == 0 and int(xq[2].abs().sum()) == 0


@pytest.mark.parametrize("K,N,b,signed", [(5120, 10240, 1, False), (5120, 10240, 2, True),
                                          (17408, 5120, 1, True), (17408, 5120, 2, False),
                                          (5120, 34816, 1, False), (5120, 5120, 2, False),
                                          (1024, 300, 1, True), (3072, 77, 2, False),
                                          (33792, 1024, 1, False), (6144, 4100, 1, True),
                                          (6144, 12288, 1, False), (2048, 6144, 2, True),
                                          (5120, 12289, 1, False), (7168, 1000, 1, False)])
def test_gemv_ternary_fused_signed_shapes(tl, K, N, b, signed):
    """Decode at b <= 2 from the raw input, with and without signs, on the layer
    shapes and ragged ones (the one-launch kernel with 16 and 32 rows per
    workgroup, one to six blocks, and just past its limits in N and K): within the
    relative bound of the oracle, and bit-identical to the rotation kernel + GEMV
    sequence where the prep + GEMV pair runs."""
    import torch
    d = dev()
    announce(f"gemv_ternary_x signed-shapes K={K} N={N} b={b} signed={signed}")
    rng = np.random.default_rng(3 * K + N + b)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    packed, _, _ = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    xbits = synth.activations(0, 1, 11, b, K)
    x = bf16_dev(xbits, d)
    sg = _signs(K, K + N) if signed else None
    signs = to_dev(sg, d) if signed else None
    s_d = to_dev(scales, d)
    y_ref = tl.gemv_ternary(tl.hadamard_blk(x, signs), packed, s_d, out_dtype=torch.float32)
    y_fus = torch.full((b, N), float("nan"), dtype=torch.float32, device=d)
    tl.gemv_ternary_x(x, packed, s_d, signs=signs, out=y_fus)
    torch.cuda.synchronize()
    _check_fused_vs_sequence(tl, y_fus.cpu().numpy(), y_ref.cpu().numpy())
    xr = oracle.rotate_exact(synth.bf16_bits_to_f32(xbits), sg)
    ref = oracle.gemv_ternary(xr, codes, scales)
    e = oracle.rel_fro(y_fus.cpu().numpy(), ref)
    announce(f"  kernel={tl.last_kernel_name()} rel_fro vs exact layer = {e:.3e}")
    assert e <= REL_TOL
