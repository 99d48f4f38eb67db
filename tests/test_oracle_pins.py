"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``check_*`` takes the implementation under test, so the same check runs on
the oracle (must pass) and on deliberately broken copies of it (must fail): a
plausible mistake -- dropped term, wrong sign or index, transposed operand,
wrong tie rule -- is caught by at least one pin.

Sources of the pinned facts:
  [P1] qiita.com/nakanokensetsu/items/ecc183fae033565af7cb
       "前提" (format), "1. TP=2 への移植" (Sylvester blocks, rank-swap control),
       "4. 効いた高速化" (q = round(127 s/smax), exact int8 weight, per-token int8)
  textbook identities (H H^T = n I, Parseval, involution), exact rational
  arithmetic (fractions.Fraction) and brute-force loops on tiny shapes.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ternary as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# fixtures from tests/golden
# ---------------------------------------------------------------------------
def _golden_h8():
    rows = []
    for line in open(os.path.join(GOLD, "sylvester_h8.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append([float(v) for v in line.split()])
    return np.array(rows)


def _golden_pack():
    cases = []
    for line in open(os.path.join(GOLD, "pack_words.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            codes, word = line.split("|")
            cases.append(([int(v) for v in codes.split()], int(word, 16)))
    return cases


def _golden_scales():
    cases = []
    for line in open(os.path.join(GOLD, "scale_decomposition.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            s, smax, q = line.split()
            cases.append((float(s), float(smax), int(q)))
    return cases


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------
def check_hadamard(had):
    np.testing.assert_array_equal(had(8), _golden_h8())
    for n in (2, 16, 128, 1024):
        H = had(n)
        np.testing.assert_array_equal(H @ H.T, n * np.eye(n))
    # Sylvester identity of [P1] §1, bit-equal in binary64
    rng = np.random.default_rng(1)
    a = rng.integers(-100, 100, 512) / 64.0
    b = rng.integers(-100, 100, 512) / 64.0
    H1024, H512 = had(1024), had(512)
    lhs = H1024 @ np.concatenate([a, b])
    rhs = np.concatenate([H512 @ a + H512 @ b, H512 @ a - H512 @ b])
    np.testing.assert_array_equal(lhs, rhs)


def check_rotation(rot):
    rng = np.random.default_rng(2)
    K = 2048
    x = rng.integers(-512, 512, (3, K)) / 256.0           # exact small dyadics
    xr = rot(x)
    # involution: the orthonormal symmetric block transform is its own inverse
    np.testing.assert_array_equal(rot(xr), x)
    # Parseval per block
    for j in range(K // 1024):
        blk = slice(1024 * j, 1024 * (j + 1))
        np.testing.assert_allclose(np.linalg.norm(xr[:, blk], axis=1),
                                   np.linalg.norm(x[:, blk], axis=1), rtol=1e-12)
    # closed form: x = H e_m / 32 in block 1 rotates to e_m (entries +-1/32, exact in bf16)
    H = oracle.sylvester_hadamard(1024)
    for m in (0, 1, 37, 1023):
        x = np.zeros((1, K))
        x[0, 1024:] = H[:, m] / 32.0
        e = np.zeros((1, K))
        e[0, 1024 + m] = 1.0
        np.testing.assert_array_equal(rot(x), e)
    # signs multiply the input before H
    d = np.where(rng.random(K) < 0.5, -1.0, 1.0)
    np.testing.assert_array_equal(rot(x, d), rot(x * d))


def test_hadamard_pins():
    check_hadamard(oracle.sylvester_hadamard)


def test_rotation_pins():
    check_rotation(oracle.rotate_exact)


def test_rotation_exact_on_generator_range():
    """Extreme values of the generator's range still rotate exactly.

    Inputs are bf16 values of magnitude in [2**-24, 255]; the exact rotation of
    a block is an integer multiple of 2**-36 below 2**13.  Rotating back must
    return the input bit for bit, which a rounded intermediate would break.
    """
    rng = np.random.default_rng(3)
    mant = rng.integers(128, 256, (2, 1024))
    expo = rng.integers(-31, 1, (2, 1024))
    x = np.ldexp(mant.astype(np.float64), expo) * np.where(rng.random((2, 1024)) < .5, -1, 1)
    x[0, :8] = 255.0
    xr = oracle.rotate_exact(x)
    assert np.all(np.abs(xr) < 2.0 ** 13)
    assert np.all(np.ldexp(xr, 36) == np.rint(np.ldexp(xr, 36)))


def test_rotation_rank_swap_control():
    """[P1] §1 checks its TP split by swapping ranks on purpose (error 1.44).

    Swapping sum and difference of the two H512 halves gives, for halves of
    equal norm, a relative error of exactly sqrt(2) against the true rotation;
    the correct split reproduces the rotation bit for bit.
    """
    rng = np.random.default_rng(4)
    a = rng.integers(-64, 64, 512) / 8.0
    b = rng.permutation(a)                       # equal norms
    x = np.concatenate([a, b])[None, :]
    ref = oracle.rotate_exact(x)[0]
    H512 = oracle.sylvester_hadamard(512)
    ha, hb = H512 @ a, H512 @ b
    good = np.concatenate([ha + hb, ha - hb]) / 32.0
    swapped = np.concatenate([ha - hb, ha + hb]) / 32.0
    np.testing.assert_array_equal(good, ref)
    assert abs(oracle.rel_fro(swapped, ref) - np.sqrt(2.0)) < 1e-12


def check_half_block(stage, join):
    """The split-block stages reproduce the unsplit rotation bit for bit."""
    rng = np.random.default_rng(5)
    T = 3
    mant = rng.integers(128, 256, (T, 1024))
    expo = rng.integers(-24, 1, (T, 1024))
    x = np.ldexp(mant.astype(np.float64), expo) * np.where(rng.random((T, 1024)) < .5, -1, 1)
    d = np.where(rng.random(1024) < 0.5, -1.0, 1.0)
    for signs in (None, d):
        lo = stage(x[:, :512], None if signs is None else signs[:512])
        hi = stage(x[:, 512:], None if signs is None else signs[512:])
        got = np.concatenate([join(lo, hi, 0), join(lo, hi, 1)], axis=1)
        np.testing.assert_array_equal(got, oracle.rotate_f32(x, signs))
    # closed form of the stage: a unit vector e_m gives (-1)^popcount(i & m), no 1/32
    for m in (0, 1, 300, 511):
        e = np.zeros((1, 512))
        e[0, m] = 1.0
        want = np.array([(-1.0) ** bin(i & m).count("1") for i in range(512)])
        np.testing.assert_array_equal(stage(e)[0], want)


def test_half_block_pins():
    check_half_block(oracle.half_block_stage, oracle.half_block_join)


def _join_swapped(u_lo, u_hi, half):
    """Mutant: the ranks' sum and difference exchanged ([P1] §1's deliberate swap)."""
    return oracle.half_block_join(u_lo, u_hi, 1 - half)


def _stage_scaled(x_half, signs_half=None):
    """Mutant: the 1/32 applied in the stage as well."""
    return oracle.half_block_stage(x_half, signs_half) / 32.0


@pytest.mark.parametrize("stage,join", [(oracle.half_block_stage, _join_swapped),
                                        (_stage_scaled, oracle.half_block_join)])
def test_half_block_mutants_fail(stage, join):
    with pytest.raises(AssertionError):
        check_half_block(stage, join)


def test_sharded_layer_matches_unsplit():
    """Two K-shards split inside a block ([P1] §1's TP=2 layout at K = 2048,
    boundary 1536): each rank rotates its full blocks and its half block, the
    halves are joined, and the partial outputs add up to the unsplit layer."""
    rng = np.random.default_rng(6)
    T, K, N, cut = 2, 2048, 40, 1536
    x = rng.integers(-512, 512, (T, K)) / 256.0
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    scales = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    xr0 = np.empty((T, cut), np.float32)
    xr0[:, :1024] = oracle.rotate_f32(x[:, :1024])
    u_lo = oracle.half_block_stage(x[:, 1024:1536])
    u_hi = oracle.half_block_stage(x[:, 1536:2048])
    xr0[:, 1024:] = oracle.half_block_join(u_lo, u_hi, 0)
    xr1 = oracle.half_block_join(u_lo, u_hi, 1)
    np.testing.assert_array_equal(np.concatenate([xr0, xr1], axis=1), oracle.rotate_f32(x))
    y = (oracle.gemv_ternary(xr0, codes[:, :cut], scales[:, :cut // 128]) +
         oracle.gemv_ternary(xr1, codes[:, cut:], scales[:, cut // 128:]))
    ref = oracle.gemv_ternary(oracle.rotate_f32(x), codes, scales)
    assert oracle.rel_fro(y, ref) < 1e-13


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
def _decode_word_independently(w: int):
    """Decode one word with plain Python ints, from the layout text alone."""
    out = [0] * 16
    for byte in range(4):
        for pair in range(4):
            f = (w >> (8 * byte + 2 * pair)) & 3
            out[4 * pair + byte] = {0: 0, 1: 1, 3: -1, 2: None}[f]
    return out


def _golden_tiles():
    cases = []
    for line in open(os.path.join(GOLD, "pack_tiles.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            lhs, rhs = line.split("|")
            N, K, n, k, code = (int(v) for v in lhs.split())
            total, index, value = rhs.split()
            cases.append((N, K, n, k, code, int(total), int(index), int(value, 16)))
    return cases


def check_words(encode, decode):
    for codes, word in _golden_pack():
        got = encode(np.array([codes], dtype=np.int8))
        assert got.shape == (1, 1) and int(got[0, 0]) == word, (codes, hex(int(got[0, 0])), hex(word))
    # all 3**8 patterns on j = 0..7 with a fixed upper half, then decoded twice
    pats = np.array(np.meshgrid(*[[-1, 0, 1]] * 8, indexing="ij")).reshape(8, -1).T
    upper = np.array([1, -1, 0, 0, 1, 1, -1, 0])
    codes = np.concatenate([pats, np.broadcast_to(upper, pats.shape)], axis=1).astype(np.int8)
    words = encode(codes.reshape(-1, 16))[:, 0]
    for i in range(0, len(words), 97):
        assert _decode_word_independently(int(words[i])) == codes[i].tolist()
    np.testing.assert_array_equal(decode(words[:, None]), codes)


def check_pack(pack, unpack):
    for N, K, n, k, code, total, index, value in _golden_tiles():
        c = np.zeros((N, K), dtype=np.int8)
        c[n, k] = code
        got = pack(c)
        assert got.shape == (total,), (N, K, got.shape, total)
        nz = np.nonzero(got)[0]
        assert nz.tolist() == [index] and int(got[index]) == value, (N, K, n, k, nz, hex(int(got[nz[0]])))
    # round trip with ragged N and an odd number of groups; every word decodes by hand
    rng = np.random.default_rng(5)
    for N, K in ((7, 1024), (33, 384), (16, 256)):
        c = rng.integers(-1, 2, (N, K)).astype(np.int8)
        p = pack(c)
        np.testing.assert_array_equal(unpack(p, N, K), c)
        # spot-check words against the index formula with the independent decoder
        GP = -(-K // 256)
        for n, w in ((0, 0), (N - 1, K // 16 - 1), (N // 2, 5)):
            g, wi = w // 8, w % 8
            idx = 256 * ((n // 16) * GP + g // 2) + 4 * (16 * (wi // 2) + n % 16) + 2 * (g % 2) + wi % 2
            assert _decode_word_independently(int(p[idx])) == c[n, 16 * w:16 * w + 16].tolist()


def test_word_pins():
    check_words(oracle.encode_words, oracle.decode_words)


def test_pack_pins():
    check_pack(oracle.pack_codes, oracle.unpack_codes)


# ---------------------------------------------------------------------------
# scale decomposition
# ---------------------------------------------------------------------------
def _fp16_values_upto(smax: float):
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    return v[v <= smax]


def check_scales(decomp):
    for s, smax, q in _golden_scales():
        row = np.array([[s, smax]], dtype=np.float16)
        qq, rs, sm = decomp(row)
        assert int(qq[0, 0]) == q, (s, smax, int(qq[0, 0]), q)
        assert int(qq[0, 1]) == 127
    # exhaustive over fp16 s <= smax against exact rational rounding (ties even)
    for smax in (0.9921875, 0.5, 0.0999755859375, 6.103515625e-05 * 127, 1.0):
        smax16 = float(np.float16(smax))
        s = _fp16_values_upto(smax16)
        row = np.concatenate([s, [smax16]]).astype(np.float16)[None, :]
        qq, rs, sm = decomp(row)
        exact = [round(Fraction(127) * Fraction(float(v)) / Fraction(smax16)) for v in row[0].astype(np.float64)]
        np.testing.assert_array_equal(qq[0].astype(np.int64), np.array(exact))
        assert float(rs[0]) == float(np.float32(np.float32(smax16) / np.float32(127)))
    # random rows: bounds, exact int8 weights, +-127 at the arg-max, monotone
    rng = np.random.default_rng(6)
    sc = np.exp(-4 + 0.5 * rng.standard_normal((64, 40))).astype(np.float16)
    sc[3] = 0
    sc[5, 7] = -sc[5].astype(np.float32).max() * 2
    qq, rs, sm = decomp(sc)
    assert np.all(np.abs(qq.astype(int)) <= 127)
    assert np.all(qq[3] == 0) and rs[3] == 0
    for n in (0, 9, 63):
        g = int(np.argmax(np.abs(sc[n].astype(np.float32))))
        assert abs(int(qq[n, g])) == 127
        order = np.argsort(sc[n].astype(np.float32), kind="stable")
        assert np.all(np.diff(qq[n, order].astype(int)) >= 0)
    assert int(qq[5, 7]) == -127


def test_scale_pins():
    check_scales(oracle.decompose_scales)


def test_int8_weight_exact():
    rng = np.random.default_rng(7)
    codes = rng.integers(-1, 2, (5, 256)).astype(np.int8)
    q = rng.integers(-127, 128, (5, 2)).astype(np.int8)
    W = oracle.int8_weight(codes, q)
    for n in range(5):
        for k in range(0, 256, 13):
            assert int(W[n, k]) == int(codes[n, k]) * int(q[n, k // 128])


# ---------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------
def _round_half_even(fr: Fraction) -> int:
    return round(fr)


def check_quant(quant):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((6, 1024)) * np.exp(rng.standard_normal((6, 1)))).astype(np.float32)
    x[2] = 0.0
    x[4, 5] = -np.abs(x[4]).max() * 3
    xq, sx = quant(x)
    assert xq.dtype == np.int8 and np.all(np.abs(xq.astype(int)) <= 127)
    assert sx[2] == 0 and np.all(xq[2] == 0)
    assert int(xq[4, 5]) == -127
    for t in (0, 1, 3, 5):
        amax = np.float32(np.abs(x[t]).max())
        # scale: the correctly rounded float32 quotient amax/127, derived from Fraction
        want_sx = np.float32(float(Fraction(float(amax)) / 127))
        assert sx[t] == want_sx
        k = int(np.argmax(np.abs(x[t])))
        assert abs(int(xq[t, k])) == 127
        for i in range(0, 1024, 7):
            fq = np.float32(float(Fraction(float(x[t, i])) / Fraction(float(sx[t]))))
            want = max(-127, min(127, _round_half_even(Fraction(float(fq)))))
            assert int(xq[t, i]) == want
        assert np.all(np.sign(xq[t]) * np.sign(x[t]) >= 0)
    # near-tie rows: the quotient x/sx rounds differently from x*(127/amax) here
    near = [(-0.74002606, 3.68562), (-1.5955694, 3.5241272), (0.5879848, 3.3188474), (1.9004934, 3.5235422)]
    xt = np.zeros((len(near), 8), dtype=np.float32)
    for r, (v, amax) in enumerate(near):
        xt[r, 0], xt[r, 3] = np.float32(amax), np.float32(v)
    xqt, sxt = quant(xt)
    for r in range(len(near)):
        fq = np.float32(float(Fraction(float(xt[r, 3])) / Fraction(float(sxt[r]))))
        assert int(xqt[r, 3]) == _round_half_even(Fraction(float(fq))), r
    # scale invariance under powers of two
    xq2, sx2 = quant(x * np.float32(2.0 ** 7))
    np.testing.assert_array_equal(xq2, xq)
    np.testing.assert_array_equal(sx2, sx * np.float32(2.0 ** 7))


def test_quant_pins():
    check_quant(oracle.quant_act_int8)


# ---------------------------------------------------------------------------
# decode GEMV
# ---------------------------------------------------------------------------
def check_gemv(gemv):
    rng = np.random.default_rng(9)
    K, N, b = 256, 3, 2
    xr = rng.standard_normal((b, K))
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    sc = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    y = gemv(xr, codes, sc)
    # brute force without group factoring
    ref = np.zeros((b, N))
    for t in range(b):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(codes[n, k]) * float(sc[n, k // 128]) * xr[t, k]
            ref[t, n] = acc
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    # closed form: xr = e_m picks code[n, m] * s[n, m//128] exactly
    for m in (0, 127, 128, 255):
        e = np.zeros((1, K))
        e[0, m] = 1.0
        np.testing.assert_array_equal(gemv(e, codes, sc)[0],
                                      codes[:, m].astype(np.float64) * sc[:, m // 128].astype(np.float64))
    # linearity
    x2 = rng.standard_normal((b, K))
    np.testing.assert_allclose(gemv(xr + 2 * x2, codes, sc), y + 2 * gemv(x2, codes, sc), rtol=1e-12, atol=1e-12)


def test_gemv_pins():
    check_gemv(oracle.gemv_ternary)


def check_gemv_q8(gemv_q8):
    """int8-activation decode: brute force with integer group sums, a closed form,
    and the scale of each token."""
    rng = np.random.default_rng(21)
    b, K, N = 3, 384, 5
    xq = rng.integers(-127, 128, (b, K)).astype(np.int8)
    sx = rng.random(b).astype(np.float32) + np.float32(0.5)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    sc = np.exp(-4 + 0.5 * rng.standard_normal((N, K // 128))).astype(np.float16)
    y = gemv_q8(xq, sx, codes, sc)
    ref = np.zeros((b, N))
    for t in range(b):
        for n in range(N):
            acc = 0.0
            for g in range(K // 128):
                isum = sum(int(codes[n, k]) * int(xq[t, k]) for k in range(128 * g, 128 * g + 128))
                acc += float(sc[n, g]) * isum
            ref[t, n] = float(sx[t]) * acc
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    # closed form: a single activation 1 at m with sx = 1 picks code[n, m] * s[n, m//128]
    for m in (0, 129, 383):
        e = np.zeros((1, K), dtype=np.int8)
        e[0, m] = 1
        np.testing.assert_array_equal(gemv_q8(e, np.ones(1, np.float32), codes, sc)[0],
                                      codes[:, m].astype(np.float64) * sc[:, m // 128].astype(np.float64))


def test_gemv_q8_pins():
    check_gemv_q8(oracle.gemv_ternary_q8)
    # against the exact layer it differs by the activation rounding
    # only: with xq from the oracle's own quantisation the error is that of [P1] §4
    rng = np.random.default_rng(22)
    xr = rng.standard_normal((4, 1024))
    codes = rng.integers(-1, 2, (64, 1024)).astype(np.int8)
    sc = np.exp(-4 + 0.5 * rng.standard_normal((64, 8))).astype(np.float16)
    xq, sx = oracle.quant_act_int8(xr.astype(np.float32))
    e = oracle.rel_fro(oracle.gemv_ternary_q8(xq, sx, codes, sc), oracle.gemv_ternary(xr, codes, sc))
    assert 1e-3 < e < 2e-2, e


# ---------------------------------------------------------------------------
# int8 GEMM and rescale
# ---------------------------------------------------------------------------
def check_gemm(gemm):
    rng = np.random.default_rng(10)
    M, K, N = 3, 256, 4
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    codes = rng.integers(-1, 2, (N, K)).astype(np.int8)
    q = rng.integers(-127, 128, (N, K // 128)).astype(np.int8)
    acc = gemm(xq, codes, q)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(xq[m, k]) * int(codes[n, k]) * int(q[n, k // 128])
            assert int(acc[m, n]) == s
    e = np.zeros((1, K), dtype=np.int8)
    e[0, 200] = 1
    np.testing.assert_array_equal(gemm(e, codes, q)[0], codes[:, 200].astype(np.int64) * q[:, 1])
    ones = np.ones((1, K), dtype=np.int8)
    want = [sum(int(q[n, g]) * int(codes[n, g * 128:(g + 1) * 128].astype(int).sum()) for g in range(2))
            for n in range(N)]
    np.testing.assert_array_equal(gemm(ones, codes, q)[0], want)
    # extreme magnitude: K * 127**2 still exact and within int32
    K2 = 17408
    big = np.full((1, K2), 127, dtype=np.int8)
    c = np.ones((2, K2), dtype=np.int8)
    c[1] = -1
    qq = np.full((2, K2 // 128), 127, dtype=np.int8)
    got = gemm(big, c, qq)
    assert got[0, 0] == K2 * 127 * 127 and got[0, 1] == -K2 * 127 * 127 and K2 * 127 * 127 < 2 ** 31


def test_gemm_pins():
    check_gemm(oracle.gemm_int8_acc)


def test_rescale_pin():
    acc = np.array([[1, -3], [7, 0]], dtype=np.int64)
    rs = np.array([0.5, 0.25], dtype=np.float32)
    sx = np.array([2.0, 3.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.rescale(acc, rs, sx), [[1.0, -1.5], [10.5, 0.0]])


def test_rel_fro_and_bf16_round():
    assert oracle.rel_fro(np.array([np.nan, 1.0]), np.array([1.0, 1.0])) == float("inf")
    assert oracle.rel_fro(np.array([3.0, 4.0]), np.array([3.0, 4.0])) == 0.0
    # bf16 rounding from binary64 agrees with the generator's float32 -> bf16 path
    # on values that float32 holds exactly
    import synth
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(4096) * 10).astype(np.float32)
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v)).astype(np.float64)
    np.testing.assert_array_equal(oracle.bf16_round(v.astype(np.float64)), want)
    # ties go to even: 1 + 2**-8 is halfway between 1 and 1 + 2**-7
    assert oracle.bf16_round(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.bf16_round(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------
def _had_or(n):                                   # popcount(i | m) instead of (i & m)
    i = np.arange(n)
    par = np.array([[bin(a | b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 1, -1.0, 1.0)


def _rot_no_norm(x, signs=None):                  # forgets the 1/32
    return oracle.rotate_exact(x, signs) * 32.0


def _rot_signs_after(x, signs=None):              # applies the signs after H
    y = oracle.rotate_exact(x)
    return y if signs is None else y * signs


def _pack_natural(codes):                         # natural bit order 2j
    codes = np.asarray(codes)
    N, K = codes.shape
    f = (codes.astype(np.int64) & 3).astype(np.uint64).reshape(N, K // 16, 16)
    w = np.zeros((N, K // 16), dtype=np.uint64)
    for j in range(16):
        w |= f[:, :, j] << np.uint64(2 * j)
    return w.astype(np.uint32)


def _pack_rowmajor(codes):                        # right words, row-major instead of tiles
    codes = np.asarray(codes)
    N, K = codes.shape
    NB, GP = -(-N // 16), -(-K // 256)
    padded = np.zeros((NB * 16, GP * 256), dtype=np.int8)
    padded[:N, :K] = codes
    return oracle.encode_words(padded).reshape(-1)


def _decomp_half_up(scales):                      # round half away from zero
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    smax = np.max(np.abs(s), axis=1)
    quo = np.float32(127.0) * s / smax[:, None]
    q = (np.sign(quo) * np.floor(np.abs(quo) + 0.5)).astype(np.int8)
    return q, (smax / np.float32(127)).astype(np.float32), smax


def _quant_mul_recip(x):                          # x * (127/amax) instead of x / (amax/127)
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    sx = (amax / np.float32(127.0)).astype(np.float32)
    inv = np.where(amax > 0, np.float32(127.0) / amax, 0).astype(np.float32)
    return np.clip(np.rint(x * inv[:, None]), -127, 127).astype(np.int8), sx


def _gemv_wrong_group(xr, codes, scales):         # scale index off by one group
    return oracle.gemv_ternary(xr, codes, np.roll(np.asarray(scales), 1, axis=1))


def _gemv_q8_no_token_scale(xq, sx, codes, scales):  # the per-token scale left out
    return oracle.gemv_ternary(np.asarray(xq, dtype=np.float64), codes, scales)


def _gemm_transposed_q(xq, codes, q):             # q indexed by k % G instead of k // 128
    G = q.shape[1]
    W = np.asarray(codes, dtype=np.int64) * np.asarray(q, dtype=np.int64)[:, np.arange(codes.shape[1]) % G]
    return np.asarray(xq, dtype=np.int64) @ W.T


@pytest.mark.parametrize("mutant,check", [
    (lambda: check_hadamard(_had_or), "hadamard"),
    (lambda: check_rotation(_rot_no_norm), "rotation-norm"),
    (lambda: check_rotation(_rot_signs_after), "rotation-signs"),
    (lambda: check_words(_pack_natural, oracle.decode_words), "word-bit-order"),
    (lambda: check_pack(_pack_rowmajor, lambda p, N, K: oracle.decode_words(p.reshape(N, K // 16))), "pack-tile-order"),
    (lambda: check_scales(_decomp_half_up), "scale-ties"),
    (lambda: check_quant(_quant_mul_recip), "quant-formula"),
    (lambda: check_gemv(_gemv_wrong_group), "gemv-group"),
    (lambda: check_gemv_q8(_gemv_q8_no_token_scale), "gemv-q8-token-scale"),
    (lambda: check_gemm(_gemm_transposed_q), "gemm-q-index"),
])
def test_planted_mistakes_are_caught(mutant, check):
    with pytest.raises(AssertionError):
        mutant()
