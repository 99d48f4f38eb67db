"""The whole layer from the raw input (tl_linear_apply): the path chosen by the
token count, bit-identical to calling that path's kernels directly, and within the
bound of the oracle of the same path (two-limb GEMV against the exact layer; int8
path against the oracle's int8 computation)."""
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


def _layer(tl, d, K, N, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    sd = to_dev(scales, d)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), sd)
    return codes, scales, sd, packed, q, rs


@pytest.mark.parametrize("T,K,N,signed", [(1, 5120, 1000, True), (2, 3072, 5000, False),
                                          (5, 1024, 300, False), (40, 2048, 1000, True), (64, 1024, 77, False),
                                          (80, 1024, 300, True), (17, 1024, 20544, False), (200, 3072, 129, False),
                                          (2, 5120, 1000, False), (1, 6144, 10000, True), (2, 4096, 6144, True)])
def test_linear_apply(tl, T, K, N, signed):
    import torch
    d = dev()
    path = tl.linear_path(T, K, N)
    announce(f"tl_linear_apply T={T} K={K} N={N} signed={signed} path={path}")
    codes, scales, sd, packed, q, rs = _layer(tl, d, K, N, T + K + N)
    xbits = synth.activations(0, 1, 11, T, K)
    x = bf16_dev(xbits, d)
    sg = np.where(np.random.default_rng(K).random(K) < 0.5, -1, 1).astype(np.int8) if signed else None
    signs = to_dev(sg, d) if signed else None
    y = poison_(torch.empty((T, N), dtype=torch.float32, device=d))
    tl.linear_apply(x, packed, sd, q, rs, signs=signs, out=y)
    kname = tl.last_kernel_name()
    if path == tl.PATH_GEMV:
        assert kname.startswith("gemv_"), kname
        y_dir = tl.gemv_ternary_x(x, packed, sd, signs=signs, out_dtype=torch.float32)
        ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(xbits), sg), codes, scales)
    else:
        assert kname.startswith("gemm_i8"), kname
        xq, sx = tl.quant_act_int8_x(x, signs)
        y_dir = tl.gemm_int8_rescale(xq, sx, packed, q, rs, out_dtype=torch.float32)
        xq_ref, sx_ref = oracle.quant_act_int8(oracle.rotate_f32(synth.bf16_bits_to_f32(xbits), sg))
        q_ref, rs_ref, _ = oracle.decompose_scales(scales)
        ref = oracle.rescale(oracle.gemm_int8_acc(xq_ref, codes, q_ref), rs_ref, sx_ref)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    np.testing.assert_array_equal(got, y_dir.cpu().numpy())
    e = oracle.rel_fro(got, ref)
    announce(f"  path={path} kernel={kname} rel_fro={e:.3e}")
    assert e <= REL_TOL


def test_linear_workspace_shared_across_paths(tl):
    """One workspace serves calls on both paths in turn: the GEMV path never
    touches the int8 GEMM's counters, which every call leaves at zero."""
    import torch
    d = dev()
    K, N = 17408, 6000        # T = 17 takes the int8 path (split-K counters in use), T = 9 the GEMV
    codes, scales, sd, packed, q, rs = _layer(tl, d, K, N, 5)
    ws = torch.zeros((max(tl.linear_workspace_size(17, K, N), tl.linear_workspace_size(9, K, N)),),
                     dtype=torch.uint8, device=d)
    xs = {T: bf16_dev(synth.activations(0, 1, 12, T, K), d) for T in (17, 9)}
    first = {}
    for T in (17, 9, 17, 9):
        y = tl.linear_apply(xs[T], packed, sd, q, rs, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        if T in first:
            np.testing.assert_array_equal(y.cpu().numpy(), first[T])
        else:
            first[T] = y.cpu().numpy()
    assert int(ws[:1024].count_nonzero()) == 0


@pytest.mark.parametrize("T,K,N,one_launch", [(1, 5120, 10240, True), (1, 6144, 8192, True), (1, 6144, 12288, False),
                                               (1, 5120, 12289, False), (2, 4096, 6144, True), (2, 5120, 1000, False),
                                               (2, 2048, 6145, False), (3, 1024, 256, False)])
def test_one_launch_rule(tl, T, K, N, one_launch):
    """The decode layer runs as one launch (rotation in every workgroup) exactly
    where the measured rule says it is ahead of the fused prep + GEMV pair: one
    token up to N = 12288 (8192 at K = 6144), two tokens up to N = 6144 while
    K <= 4096."""
    import torch
    d = dev()
    codes, scales, sd, packed, q, rs = _layer(tl, d, K, N, T * 7 + K + N)
    x = bf16_dev(synth.activations(0, 1, 13, T, K), d)
    announce(f"one-launch rule T={T} K={K} N={N}")
    y = tl.linear_apply(x, packed, sd, q, rs, out_dtype=torch.float32)
    kname = tl.last_kernel_name()
    torch.cuda.synchronize()
    assert kname.startswith("gemv_rot") == one_launch, kname
    ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(synth.activations(0, 1, 13, T, K))),
                              codes, scales)
    assert oracle.rel_fro(y.cpu().numpy(), ref) <= REL_TOL
