"""tl_linear_apply_noalloc: the layer entry point that allocates nothing (its
workspace is the library's static per-GPU scratch array) must give what
tl_linear_apply gives, bit for bit, call after call, including a second call
with a smaller input, and must reject a request larger than the array before
touching the GPU."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, announce, bf16_dev, dev, poison_, to_dev

import quantized_gemv_gemm_amd as tl_mod

FAKE = ctypes.c_void_p(0x10000)


@pytest.mark.skipif(not os.path.exists(tl_mod.LIB_PATH), reason="libtl.so not built")
def test_noalloc_rejects_oversize_on_host():
    L = tl_mod.lib()
    cap = L.tl_noalloc_scratch_bytes()
    assert cap == 64 << 20
    # int8 path at 8192 tokens of K = 16384: 128 MiB of int8 activations alone
    T, K, N = 8192, 16384, 4096
    assert L.tl_linear_workspace_size(T, K, N) > cap
    assert L.tl_linear_apply_noalloc(FAKE, T, K, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 9
    assert "static" in tl_mod.status_string(9)
    # the other argument errors come first, with tl_linear_apply's codes
    assert L.tl_linear_apply_noalloc(FAKE, 4, 1536, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 2
    assert L.tl_linear_apply_noalloc(None, 4, 1024, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 1
    assert L.tl_linear_apply_noalloc(FAKE, 4, 1024, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, 7, None) == 4
    assert L.tl_linear_apply_noalloc(FAKE, 0, 1024, N, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == 0


def _layer(tl, d, K, N, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    sd = to_dev(scales, d)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), sd)
    return codes, scales, sd, packed, q, rs


@pytest.mark.gpu
def test_noalloc_matches_linear_apply():
    import torch
    tl = tl_mod
    d = dev()
    K, N = 3072, 2304
    codes, scales, sd, packed, q, rs = _layer(tl, d, K, N, 77)
    # int8 path (K-split GEMM counters in use), then a smaller GEMV-path call,
    # then the large one again: the shared array keeps the last call's contents
    for T in (200, 5, 200, 1):
        path = tl.linear_path(T, K, N)
        announce(f"tl_linear_apply_noalloc T={T} K={K} N={N} path={path}")
        xbits = synth.activations(0, 1, 12 + T, T, K)
        x = bf16_dev(xbits, d)
        y_ref = poison_(torch.empty((T, N), dtype=torch.float32, device=d))
        tl.linear_apply(x, packed, sd, q, rs, out=y_ref)
        k_ref = tl.last_kernel_name()
        y = poison_(torch.empty((T, N), dtype=torch.float32, device=d))
        tl.linear_apply_noalloc(x, packed, sd, q, rs, out=y)
        assert tl.last_kernel_name() == k_ref
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"T={T}: differs from tl_linear_apply"
        xf = synth.bf16_bits_to_f32(xbits)
        if path == tl.PATH_GEMV:
            ref = oracle.gemv_ternary(oracle.rotate_exact(xf), codes, scales)
        else:
            xq_ref, sx_ref = oracle.quant_act_int8(oracle.rotate_f32(xf))
            q_ref, rs_ref, _ = oracle.decompose_scales(scales)
            ref = oracle.rescale(oracle.gemm_int8_acc(xq_ref, codes, q_ref), rs_ref, sx_ref)
        e = oracle.rel_fro(y.cpu().numpy(), ref)
        assert e <= REL_TOL, (T, e)
