"""Split-block rotation for a K-shard boundary inside a 1024-block ([P1] "1. TP=2
への移植"), emulated on one GPU: each rank's half stage, the exchange (both
results are on the same device), the sum/difference join -- bit-identical to the
unsplit rotation -- and the down_proj layer at its TP=2 shard shape (K = 8704 per
rank) with the partial outputs added as the all-reduce would."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, announce, bf16_dev, dev, poison_, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import quantized_gemv_gemm_amd as m
    m.lib()
    return m


def _signs(K, seed):
    return np.where(np.random.default_rng(seed).random(K) < 0.5, -1, 1).astype(np.int8)


@pytest.mark.parametrize("T,signed", [(1, False), (5, True), (300, False)])
def test_half_join_bitexact(tl, T, signed):
    import torch
    d = dev()
    announce(f"tl_hadamard_half/join T={T} signed={signed}")
    xbits = synth.activations(0, 2, 1, T, 1024)
    x = bf16_dev(xbits, d)
    xf = synth.bf16_bits_to_f32(xbits)
    sg = _signs(1024, T) if signed else None
    s_lo = to_dev(sg[:512], d) if signed else None
    s_hi = to_dev(sg[512:], d) if signed else None
    u_lo = tl.hadamard_half(x[:, :512], s_lo)
    u_hi = tl.hadamard_half(x[:, 512:], s_hi)
    xr = poison_(torch.empty((T, 1024), dtype=torch.float32, device=d))
    tl.hadamard_join(u_lo, u_hi, 0, out=xr[:, :512])
    tl.hadamard_join(u_lo, u_hi, 1, out=xr[:, 512:])
    full = tl.hadamard_blk(x, to_dev(sg, d) if signed else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u_lo.cpu().numpy(), oracle.half_block_stage(xf[:, :512], None if sg is None else sg[:512]))
    np.testing.assert_array_equal(u_hi.cpu().numpy(), oracle.half_block_stage(xf[:, 512:], None if sg is None else sg[512:]))
    np.testing.assert_array_equal(xr.cpu().numpy(), oracle.rotate_f32(xf, sg))
    np.testing.assert_array_equal(xr.cpu().numpy(), full.cpu().numpy())


def _pack(tl, d, codes, scales):
    sd = to_dev(np.ascontiguousarray(scales), d)
    packed, q, rs = tl.pack_weights(to_dev(np.ascontiguousarray(codes), d), sd)
    return packed, sd, q, rs


@pytest.mark.parametrize("T", [4, 16])
def test_tp2_down_proj_emulation(tl, T):
    """down_proj (17408 -> 5120) split over two ranks at 8704 = 8.5 blocks."""
    import torch
    d = dev()
    K, N, cut = 17408, 5120, 8704
    announce(f"TP=2 emulation down_proj T={T}")
    L = synth.LayerInputs(0, 2, 1, K, N)
    codes, scales = L.codes(), L.scales()
    xbits = synth.activations(0, 2, 1, T, K)
    x = bf16_dev(xbits, d)
    sg = _signs(K, 17)
    sd_all = to_dev(sg, d)
    # rank 0: blocks 0..7 whole, first half of block 8; rank 1: second half, blocks 9..16
    xr0 = poison_(torch.empty((T, cut), dtype=torch.float32, device=d))
    xr1 = poison_(torch.empty((T, K - cut), dtype=torch.float32, device=d))
    xr0[:, :8192] = tl.hadamard_blk(x[:, :8192].contiguous(), sd_all[:8192].contiguous())
    u0 = tl.hadamard_half(x[:, 8192:8704], sd_all[8192:8704].contiguous())
    u1 = tl.hadamard_half(x[:, 8704:9216], sd_all[8704:9216].contiguous())
    xr1[:, 512:] = tl.hadamard_blk(x[:, 9216:].contiguous(), sd_all[9216:].contiguous())
    # exchange, then each rank joins its own half
    tl.hadamard_join(u0, u1, 0, out=xr0[:, 8192:])
    tl.hadamard_join(u0, u1, 1, out=xr1[:, :512])
    full = tl.hadamard_blk(x, sd_all)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(torch.cat([xr0, xr1], 1).cpu().numpy(), full.cpu().numpy())
    # each rank's GEMV on its K-shard (the shard shape K = 8704 = 68 groups), then the all-reduce sum
    p0, s0, _, _ = _pack(tl, d, codes[:, :cut], scales[:, :cut // 128])
    p1, s1, _, _ = _pack(tl, d, codes[:, cut:], scales[:, cut // 128:])
    y0 = tl.gemv_ternary(xr0, p0, s0, out_dtype=torch.float32)
    k0 = tl.last_kernel_name()
    y1 = tl.gemv_ternary(xr1, p1, s1, out_dtype=torch.float32)
    y = (y0 + y1).cpu().numpy()
    ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(xbits), sg), codes, scales)
    e = oracle.rel_fro(y, ref)
    announce(f"  shard kernel={k0} rel_fro(sum of shards vs exact layer)={e:.3e}")
    assert e <= REL_TOL


@pytest.mark.parametrize("name,K,N,k0,k1", [("down shard", 17408, 5120, 0, 8704),
                                            ("gate_up shard", 5120, 17408, 0, 5120)])
def test_shard_shape_gemm(tl, name, K, N, k0, k1):
    """The int8 GEMM at a TP=2 shard shape (down: K = 8704; gate_up: N = 17408), accumulators exact."""
    import torch
    d = dev()
    M = 128
    L = synth.LayerInputs(0, 2, 1 if K == 17408 else 0, K, 2 * N if name.startswith("gate") else N)
    codes, scales = L.codes()[:N, k0:k1], L.scales()[:N, k0 // 128:k1 // 128]
    announce(f"GEMM {name} M={M} K={k1 - k0} N={N}")
    packed, _, q, rs = _pack(tl, d, codes, scales)
    xq = np.random.default_rng(3).integers(-127, 128, (M, k1 - k0)).astype(np.int8)
    sx = np.full(M, 0.01, np.float32)
    y, acc = tl.gemm_int8_rescale(to_dev(xq, d), to_dev(sx, d), packed, q, rs, out_dtype=torch.float32,
                                  want_acc=True)
    torch.cuda.synchronize()
    q_ref, rs_ref, _ = oracle.decompose_scales(scales)
    acc_ref = oracle.gemm_int8_acc(xq, codes, q_ref)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    assert oracle.rel_fro(y.cpu().numpy(), oracle.rescale(acc_ref, rs_ref, sx)) <= REL_TOL


def test_tp2_rank_swap_control(tl):
    """[P1] §1 swaps the ranks on purpose and sees a relative error of 1.44: a
    one-block layer split in the middle, with the sum and the difference given to
    the wrong ranks, is off by 2 |b| / sqrt(|a|^2 + |b|^2) (a, b the two input
    halves; the error is W0 - W1 applied to the second half's transform) -- about
    sqrt(2) for halves of equal norm, as here (Gaussian inputs without outlier
    channels); the right assignment is within the bar."""
    import torch
    d = dev()
    K, N, T = 1024, 2048, 4
    rng = np.random.default_rng(8)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xbits = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    x = bf16_dev(xbits, d)
    u0, u1 = tl.hadamard_half(x[:, :512]), tl.hadamard_half(x[:, 512:])
    ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(xbits)), codes, scales)
    errs = {}
    for label, (h0, h1) in (("right", (0, 1)), ("swapped", (1, 0))):
        y = 0.0
        for r, h in ((0, h0), (1, h1)):
            xr = tl.hadamard_join(u0, u1, h)
            p, s, _, _ = _pack(tl, d, codes[:, 512 * r:512 * (r + 1)], scales[:, 4 * r:4 * (r + 1)])
            y = y + tl.gemv_ternary(xr, p, s, out_dtype=torch.float32).cpu().numpy()
        errs[label] = oracle.rel_fro(y, ref)
    announce(f"  rank assignment right={errs['right']:.3e} swapped={errs['swapped']:.3f}")
    assert errs["right"] <= REL_TOL
    assert 1.3 < errs["swapped"] < 1.53
