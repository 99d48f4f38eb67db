"""HIP path vs the CPU oracle, element by element, on seeded synthetic layers.

Bars: bit-exact for packed words, q, row_scale, the rotation's f32 output (the
rotation is exact before its single rounding), int8 activations, token scales
and int32 accumulators; relative Frobenius error <= 1e-3 for floating-point
outputs (f32 against the binary64 oracle, bf16 against the oracle rounded to
bf16).  Every output is poisoned before the call.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_common import REL_TOL, Layer, announce, bf16_dev, dev, poison_, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tl():
    import quantized_gemv_gemm_amd as tl
    tl.lib()   # raises if the library is missing: no silent fallback
    return tl


# (random stream of the workload, layer index, K, N) of every layer shape in the workloads
SHAPES = {
    "tiny": (synth.WORKLOADS["tiny"]["stream"], 0, 1024, 256),
    "qkv": (synth.WORKLOADS["decode_qkv"]["stream"], 0, 5120, 10240),
    "gate_up": (synth.WORKLOADS["decode_mlp"]["stream"], 0, 5120, 34816),
    "down": (synth.WORKLOADS["decode_mlp"]["stream"], 1, 17408, 5120),
}

_layers = {}


def layer(name, tl):
    if name not in _layers:
        c, li, K, N = SHAPES[name]
        announce(f"build layer {name} K={K} N={N}")
        _layers[name] = Layer(0, c, li, K, N, dev()).pack()
    return _layers[name]


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "qkv", "gate_up", "down"])
def test_pack_bit_exact(tl, name):
    import torch
    d = dev()
    c, li, K, N = SHAPES[name]
    L = Layer(0, c, li, K, N, d)
    packed = poison_(torch.empty((tl.packed_words(N, K),), dtype=torch.int32, device=d))
    q = poison_(torch.empty((N, K // 128), dtype=torch.int8, device=d))
    rs = poison_(torch.empty((N,), dtype=torch.float32, device=d))
    bad = torch.zeros((1,), dtype=torch.int32, device=d)
    announce(f"tl_pack_weights {name} N={N} K={K}")
    tl.pack_weights(L.codes_d, L.scales_d, packed, q, rs, invalid_count=bad)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), oracle.pack_codes(L.codes))
    q_ref, rs_ref, _ = oracle.decompose_scales(L.scales)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(rs.cpu().numpy().view(np.uint32), rs_ref.view(np.uint32))
    assert int(bad.item()) == 0
    assert tl.last_kernel_name() == "pack_tiles+scale_rows"


@pytest.mark.parametrize("N,K", [(7, 1024), (33, 384), (300, 128)])
def test_pack_ragged_tiles(tl, N, K):
    """Partial row blocks and an odd number of groups: padding words are zero."""
    import torch
    d = dev()
    rng = np.random.default_rng(N + K)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    packed = poison_(torch.empty((tl.packed_words(N, K),), dtype=torch.int32, device=d))
    announce(f"tl_pack_weights ragged N={N} K={K}")
    tl.pack_weights(to_dev(codes, d), to_dev(scales, d), packed=packed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), oracle.pack_codes(codes))


def test_pack_edge_rows_and_bad_codes(tl):
    import torch
    d = dev()
    rng = np.random.default_rng(12)
    K, N = 256, 5
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, 2))).astype(np.float16)
    scales[1] = 0.0                                   # zero row -> q = 0, row_scale = 0
    scales[2] = [np.float16(0.25), np.float16(0.5)]   # exact tie 63.5 -> 64
    scales[3] = [np.float16(-0.75), np.float16(0.5)]  # negative maximum magnitude
    scales[4] = [np.float16(0.48828125), np.float16(0.9921875)]  # tie 62.5 -> 62
    announce("tl_pack_weights edge rows")
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    q_ref, rs_ref, _ = oracle.decompose_scales(scales)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(rs.cpu().numpy(), rs_ref)
    assert q.cpu().numpy()[2, 0] == 64 and q.cpu().numpy()[4, 0] == 62
    # invalid codes are counted
    bad_codes = codes.copy()
    bad_codes[0, 3], bad_codes[4, 100], bad_codes[2, 7] = 2, -2, 5
    cnt = torch.zeros((1,), dtype=torch.int32, device=d)
    tl.pack_weights(to_dev(bad_codes, d), to_dev(scales, d), invalid_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 3


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,K,with_signs", [(1, 1024, False), (16, 5120, False), (3, 17408, True),
                                            (512, 17408, False), (7, 2048, True)])
def test_hadamard_bit_exact(tl, T, K, with_signs):
    import torch
    d = dev()
    xbits = synth.activations(0, 9, K, T, K)
    signs = None
    if with_signs:
        signs = np.where(np.random.default_rng(K).random(K) < 0.5, -1, 1).astype(np.int8)
    out = poison_(torch.empty((T, K), dtype=torch.float32, device=d))
    announce(f"tl_hadamard_blk T={T} K={K} signs={with_signs}")
    tl.hadamard_blk(bf16_dev(xbits, d), None if signs is None else to_dev(signs, d), out=out)
    ref = oracle.rotate_f32(synth.bf16_bits_to_f32(xbits), signs)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_hadamard_closed_form(tl):
    """x = H e_m / 32 (entries +-1/32, exact in bf16) rotates to e_m."""
    d = dev()
    H = oracle.sylvester_hadamard(1024)
    x = np.zeros((4, 2048), dtype=np.float32)
    ms = [0, 5, 1023, 511]
    for t, m in enumerate(ms):
        x[t, 1024 * (t % 2):1024 * (t % 2) + 1024] = H[:, m] / 32.0
    xr = tl.hadamard_blk(bf16_dev(synth.f32_to_bf16_bits(x), d)).cpu().numpy()
    want = np.zeros_like(x)
    for t, m in enumerate(ms):
        want[t, 1024 * (t % 2) + m] = 1.0
    np.testing.assert_array_equal(xr, want)


# ---------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,K", [(1, 1024), (512, 5120), (512, 17408), (5, 256)])
def test_quant_bit_exact(tl, T, K):
    import torch
    d = dev()
    rng = np.random.default_rng(T * 7 + K)
    xr = (rng.standard_normal((T, K)) * np.exp(rng.standard_normal((T, 1)))).astype(np.float32)
    if T > 2:
        xr[1] = 0.0            # zero token
        xr[2, 3] = 1e4         # one dominant value
    xq = poison_(torch.empty((T, K), dtype=torch.int8, device=d))
    sx = poison_(torch.empty((T,), dtype=torch.float32, device=d))
    announce(f"tl_quant_act_int8 T={T} K={K}")
    tl.quant_act_int8(to_dev(xr, d), xq, sx)
    xq_ref, sx_ref = oracle.quant_act_int8(xr)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)


def test_quant_near_ties(tl):
    """Rows whose values sit where x/sx and x*(127/amax) round apart."""
    d = dev()
    near = [(-0.74002606, 3.68562), (-1.5955694, 3.5241272), (0.5879848, 3.3188474), (1.9004934, 3.5235422)]
    xr = np.zeros((4, 128), dtype=np.float32)
    for r, (v, amax) in enumerate(near):
        xr[r, 0], xr[r, 3] = np.float32(amax), np.float32(v)
    xq, sx = tl.quant_act_int8(to_dev(xr, d))
    xq_ref, sx_ref = oracle.quant_act_int8(xr)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), sx_ref)


# ---------------------------------------------------------------------------
# decode GEMV
# ---------------------------------------------------------------------------
def _gemv_case(tl, L, b, x_layer_cfg):
    import torch
    d = L.d
    xbits = synth.activations(0, x_layer_cfg[0], x_layer_cfg[1], b, L.K)
    x = bf16_dev(xbits, d)
    xr = tl.hadamard_blk(x)
    announce(f"tl_gemv_ternary b={b} K={L.K} N={L.N}")
    y32 = poison_(torch.empty((b, L.N), dtype=torch.float32, device=d))
    tl.gemv_ternary(xr, L.packed, L.scales_d, out=y32)
    kname = tl.last_kernel_name()
    y16 = poison_(torch.empty((b, L.N), dtype=torch.bfloat16, device=d))
    tl.gemv_ternary(xr, L.packed, L.scales_d, out=y16)
    torch.cuda.synchronize()
    ref = oracle.gemv_ternary(oracle.rotate_exact(synth.bf16_bits_to_f32(xbits)), L.codes, L.scales)
    e32 = oracle.rel_fro(y32.cpu().numpy(), ref)
    e16 = oracle.rel_fro(y16.float().cpu().numpy(), oracle.bf16_round(ref))
    announce(f"  rel_fro f32={e32:.3e} bf16={e16:.3e} kernel={kname}")
    assert e32 <= REL_TOL and e16 <= REL_TOL, (e32, e16)
    assert kname.startswith("gemv_")
    return e32


@pytest.mark.parametrize("name,b", [("tiny", 1), ("qkv", 1), ("qkv", 4), ("qkv", 8), ("qkv", 16),
                                    ("gate_up", 1), ("gate_up", 16), ("down", 1), ("down", 16),
                                    ("qkv", 32), ("qkv", 64), ("down", 48)])
def test_gemv_parity(tl, name, b):
    L = layer(name, tl)
    c, li, _, _ = SHAPES[name]
    _gemv_case(tl, L, b, (c, li))


@pytest.mark.parametrize("K,N,b", [(128, 300, 3), (256, 17, 16), (1024, 1000, 5), (3072, 64, 2),
                                   (384, 33, 8), (17408, 48, 1), (5120, 100, 12), (13440, 40, 1),
                                   (17024, 70, 2),
                                   (256, 17, 17), (1024, 1000, 31), (384, 33, 50), (17408, 48, 64)])
def test_gemv_ragged(tl, K, N, b):
    """N not a multiple of the row tile, K smaller than the wave count, odd b."""
    import torch
    d = dev()
    rng = np.random.default_rng(K + N + b)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    scales[N // 2] = 0
    xr = rng.standard_normal((b, K)).astype(np.float32)
    xr[b - 1, :] *= 1e-3
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    y = poison_(torch.empty((b, N), dtype=torch.float32, device=d))
    announce(f"tl_gemv_ternary ragged K={K} N={N} b={b}")
    tl.gemv_ternary(to_dev(xr, d), packed, to_dev(scales, d), out=y)
    got = y.cpu().numpy()
    ref = oracle.gemv_ternary(xr, codes, scales)
    assert oracle.rel_fro(got, ref) <= REL_TOL
    assert np.all(got[:, N // 2] == 0)
    # each token row on its own (a tiny row must not drown in the others)
    for t in range(b):
        assert oracle.rel_fro(got[t], ref[t]) <= REL_TOL


@pytest.mark.parametrize("K,N,b", [(5120, 300, 4), (5120, 300, 16), (2304, 1000, 16), (17408, 200, 1),
                                   (17024, 70, 2), (13440, 40, 1),
                                   (17408, 200, 16), (3200, 64, 8)])
def test_gemv_block_scales(tl, K, N, b):
    """Activations whose 1024-blocks differ wildly in size: a block of zeros
    (first, middle, last), a block 1e-6 times and one 1e3 times the rest.  The
    limbs are scaled per block, and a wave whose pairs span two blocks changes the
    units of its sums once (in every kernel shape: limbs in LDS or registers, or
    the long-K ring)."""
    import torch
    d = dev()
    rng = np.random.default_rng(K * 7 + b)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xr = rng.standard_normal((b, K)).astype(np.float32)
    nbk = (K + 1023) // 1024
    for t in range(b):
        j = t % nbk
        kind = t % 4
        sl = slice(1024 * j, min(K, 1024 * (j + 1)))
        if kind == 0:
            xr[t, sl] = 0
        elif kind == 1:
            xr[t, sl] *= 1e-6
        elif kind == 2:
            xr[t, sl] *= 1e3
    packed, _, _ = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    y = poison_(torch.empty((b, N), dtype=torch.float32, device=d))
    announce(f"tl_gemv_ternary block scales K={K} N={N} b={b}")
    tl.gemv_ternary(to_dev(xr, d), packed, to_dev(scales, d), out=y)
    announce(f"  kernel={tl.last_kernel_name()}")
    got = y.cpu().numpy()
    ref = oracle.gemv_ternary(xr, codes, scales)
    for t in range(b):
        assert oracle.rel_fro(got[t], ref[t]) <= REL_TOL, t


def test_gemv_zero_token(tl):
    d = dev()
    L = layer("tiny", tl)
    xr = np.zeros((2, L.K), dtype=np.float32)
    xr[1] = np.random.default_rng(13).standard_normal(L.K)
    y = tl.gemv_ternary(to_dev(xr, d), L.packed, L.scales_d, out_dtype=__import__("torch").float32)
    got = y.cpu().numpy()
    assert np.all(got[0] == 0)
    assert oracle.rel_fro(got[1], oracle.gemv_ternary(xr[1:], L.codes, L.scales)[0]) <= REL_TOL


# ---------------------------------------------------------------------------
# prefill int8 GEMM + rescale
# ---------------------------------------------------------------------------
def _gemm_check(tl, codes, scales, packed, q, rs, xq_np, sx_np, label):
    import torch
    d = packed.device
    M, N = xq_np.shape[0], codes.shape[0]
    y32 = poison_(torch.empty((M, N), dtype=torch.float32, device=d))
    acc = poison_(torch.empty((M, N), dtype=torch.int32, device=d))
    announce(f"tl_gemm_int8_rescale {label} M={M} K={codes.shape[1]} N={N}")
    tl.gemm_int8_rescale(to_dev(xq_np, d), to_dev(sx_np, d), packed, q, rs, out=y32, acc_out=acc)
    kname = tl.last_kernel_name()
    y16 = poison_(torch.empty((M, N), dtype=torch.bfloat16, device=d))
    tl.gemm_int8_rescale(to_dev(xq_np, d), to_dev(sx_np, d), packed, q, rs, out=y16)
    torch.cuda.synchronize()
    q_ref, rs_ref, _ = oracle.decompose_scales(scales)
    acc_ref = oracle.gemm_int8_acc(xq_np, codes, q_ref)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    ref = oracle.rescale(acc_ref, rs_ref, sx_np)
    e32 = oracle.rel_fro(y32.cpu().numpy(), ref)
    e16 = oracle.rel_fro(y16.float().cpu().numpy(), oracle.bf16_round(ref))
    announce(f"  acc bit-exact; rel_fro f32={e32:.3e} bf16={e16:.3e} kernel={kname}")
    assert e32 <= REL_TOL and e16 <= REL_TOL
    return acc


@pytest.mark.parametrize("name,M", [("tiny", 1), ("tiny", 64), ("gate_up", 512), ("down", 512)])
def test_prefill_path_parity(tl, name, M):
    """rotation -> per-token int8 -> int8 GEMM + rescale, each stage checked."""
    import torch
    L = layer(name, tl)
    c, li, K, N = SHAPES[name]
    d = L.d
    xbits = synth.activations(0, 3 if name != "tiny" else 0, li, M, K)
    announce(f"prefill {name} M={M}: rotation + quant")
    xr = tl.hadamard_blk(bf16_dev(xbits, d))
    xq, sx = tl.quant_act_int8(xr)
    torch.cuda.synchronize()
    xr_ref = oracle.rotate_f32(synth.bf16_bits_to_f32(xbits))
    np.testing.assert_array_equal(xr.cpu().numpy(), xr_ref)
    xq_ref, sx_ref = oracle.quant_act_int8(xr_ref)
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    np.testing.assert_array_equal(sx.cpu().numpy(), sx_ref)
    _gemm_check(tl, L.codes, L.scales, L.packed, L.q, L.rs, xq_ref, sx_ref, name)


@pytest.mark.parametrize("M,K,N", [(77, 256, 300), (1, 128, 33), (130, 1024, 257), (129, 2048, 512),
                                   (64, 384, 96), (200, 640, 40)])
def test_gemm_ragged(tl, M, K, N):
    d = dev()
    rng = np.random.default_rng(M * 31 + K + N)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.exp(rng.standard_normal(M)).astype(np.float32)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    _gemm_check(tl, codes, scales, packed, q, rs, xq, sx, "ragged")


@pytest.mark.parametrize("M,K,N", [(500, 256, 33500), (130, 384, 65700)])
def test_gemm_narrow_tail(tl, M, K, N):
    """A short last round (524 or 514 tiles of 128 x 256) cut into 32 x 128
    sub-tiles, some of them partly or wholly past M and N (500 rows = 3 whole
    M-blocks + 116 rows; 130 = 1 + 2 rows; ragged last strips)."""
    d = dev()
    rng = np.random.default_rng(M + K + N)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.exp(rng.standard_normal(M)).astype(np.float32)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    _gemm_check(tl, codes, scales, packed, q, rs, xq, sx, "narrow tail")
    assert tl.last_kernel_name().endswith("narrowtail")


@pytest.mark.parametrize("M,K,N", [(2000, 384, 8200), (1100, 1280, 30000)])
def test_gemm_two_per_cu_ragged(tl, M, K, N):
    """At least two tiles per compute unit: the two-workgroups-per-CU pipeline,
    with ragged last M-block and N-strip, an odd group count (K = 384) and a
    left-over round (cut into sub-tiles, or split along K)."""
    d = dev()
    rng = np.random.default_rng(M + K + N)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.exp(rng.standard_normal(M)).astype(np.float32)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    _gemm_check(tl, codes, scales, packed, q, rs, xq, sx, "two per CU")
    assert "_lds2" in tl.last_kernel_name()


@pytest.mark.parametrize("M,K,N", [(512, 17408, 5120), (130, 2048, 1000), (33, 384, 4000), (200, 640, 40),
                                   (64, 128, 700), (1500, 640, 6000), (300, 256, 22940)])
def test_gemm_mid_tiles(tl, M, K, N):
    """Fewer than 512 tiles of 128 x 256: 128 x 128 tiles on the two-per-CU
    pipeline (down at 512 tokens: 160 tiles x 3 pieces; 16 tiles x 2; ragged M and
    N; an odd group count; N narrower than a tile; one pair of groups; a whole
    round of 512 and 52 left-over tiles x 2 pieces; 540 tiles, no split)."""
    d = dev()
    rng = np.random.default_rng(M + K + N + 7)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.exp(rng.standard_normal(M)).astype(np.float32)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    _gemm_check(tl, codes, scales, packed, q, rs, xq, sx, "mid tiles")
    assert tl.last_kernel_name().startswith("gemm_i8_mfma32_128x128_lds2")


def test_gemm_workspace_reused_across_shapes(tl):
    """One workspace, K-split GEMMs of different shapes in turn (64 and 128 split
    tiles): the counters of one shape never overlap the partials of another, and
    every call leaves them at zero."""
    import torch
    d = dev()
    rng = np.random.default_rng(2048)
    K, M = 5120, 2048
    shapes = [5120, 10240, 5120]
    layers = {}
    for N in sorted(set(shapes)):
        codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
        scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
        packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
        layers[N] = (codes, scales, packed, q, rs)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = np.exp(rng.standard_normal(M)).astype(np.float32)
    xq_d, sx_d = to_dev(xq, d), to_dev(sx, d)
    need = max(tl.gemm_workspace_size(M, K, N) for N in shapes)
    assert all(tl.gemm_workspace_size(M, K, N) > 0 for N in shapes)
    ws = torch.zeros((need,), dtype=torch.uint8, device=d)
    toks = np.sort(rng.choice(M, 48, replace=False))
    for N in shapes:
        announce(f"gemm workspace reuse M={M} K={K} N={N}")
        codes, scales, packed, q, rs = layers[N]
        acc = poison_(torch.empty((M, N), dtype=torch.int32, device=d))
        tl.gemm_int8_rescale(xq_d, sx_d, packed, q, rs, out_dtype=torch.float32, acc_out=acc, workspace=ws)
        torch.cuda.synchronize()
        rows = np.sort(rng.choice(N, 96, replace=False))
        q_ref, _, _ = oracle.decompose_scales(scales[rows])
        acc_ref = oracle.gemm_int8_acc(xq[toks], codes[rows], q_ref)
        got = acc[torch.from_numpy(toks).to(d)][:, torch.from_numpy(rows).to(d)].cpu().numpy()
        np.testing.assert_array_equal(got.astype(np.int64), acc_ref)
        assert int(ws[:1024].view(torch.int32).abs().sum()) == 0   # counters back at zero


def test_gemm_extreme_accumulator(tl):
    """All +-127 inputs and weights: |acc| = K * 127^2 at K = 17408 stays exact."""
    d = dev()
    K, N, M = 17408, 64, 4
    codes = np.ones((N, K), dtype=np.int8)
    codes[1::2] = -1
    scales = np.ones((N, K // 128), dtype=np.float16)
    xq = np.full((M, K), 127, dtype=np.int8)
    xq[1] = -127
    sx = np.ones(M, dtype=np.float32)
    packed, q, rs = tl.pack_weights(to_dev(codes, d), to_dev(scales, d))
    acc = _gemm_check(tl, codes, scales, packed, q, rs, xq, sx, "extreme")
    assert int(acc[0, 0]) == K * 127 * 127 and int(acc[1, 0]) == -K * 127 * 127


def test_int_outputs_deterministic(tl):
    import torch
    L = layer("qkv", tl)
    d = L.d
    rng = np.random.default_rng(14)
    xq = to_dev(rng.integers(-127, 128, (40, L.K)).astype(np.int8), d)
    sx = to_dev(np.ones(40, dtype=np.float32), d)
    _, a1 = tl.gemm_int8_rescale(xq, sx, L.packed, L.q, L.rs, want_acc=True)
    _, a2 = tl.gemm_int8_rescale(xq, sx, L.packed, L.q, L.rs, want_acc=True)
    p2, q2, r2 = tl.pack_weights(L.codes_d, L.scales_d)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(p2, L.packed) and torch.equal(q2, L.q)
