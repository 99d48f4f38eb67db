"""Plain CPU definitions of the ternary linear layer (test infrastructure only).

[P1] = qiita.com/nakanokensetsu/items/ecc183fae033565af7cb (ternary 27B model on
2x RTX 5070 with vLLM TP=2).  Sections cited by their headings:
  "前提"                       model format: 2-bit {-1,0,+1} codes, one scale per
                               128 weights, block Hadamard rotation on the input
  "1. TP=2 への移植"            1024-wide Sylvester blocks, sign table, and the
                               recursion H1024[a;b] = [H512 a + H512 b; H512 a - H512 b]
  "4. 効いた高速化" (int8 prefill)  q = round(127 s / smax), W_int8 = code * q,
                               per-token int8 activations after the rotation,
                               one int8 GEMM, per-row and per-token rescale

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use this.
"""
from __future__ import annotations

import numpy as np

GROUP = 128      # [P1] "前提": one scale per 128 weights along K
HBLOCK = 1024    # [P1] §1: Hadamard blocks are 1024 wide


# ---------------------------------------------------------------------------
# rotation  ([P1] "前提", §1)
# ---------------------------------------------------------------------------
def sylvester_hadamard(n: int) -> np.ndarray:
    """Dense Sylvester-order Hadamard matrix, H[i, m] = (-1)^popcount(i & m).

    This is the closed form of the Sylvester recursion H_2n = [[H, H], [H, -H]]
    that [P1] §1 uses in the form H1024 [a; b] = [H512 a + H512 b; H512 a - H512 b].
    Entries are exact +-1 in binary64.
    """
    if n <= 0 or n & (n - 1):
        raise ValueError("n must be a power of two")
    i = np.arange(n, dtype=np.int64)
    anded = i[:, None] & i[None, :]
    parity = np.zeros_like(anded)
    while np.any(anded):
        parity ^= anded & 1
        anded >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def rotate_exact(x: np.ndarray, signs: np.ndarray | None = None) -> np.ndarray:
    """Block rotation xr = (1/32) H1024 (d * x) on every 1024-block of each row.

    x     : [T, K] real values (the bf16 inputs, already widened), K % 1024 == 0
    signs : [K] of +-1 or None (all +1).  READING: [P1] §1 speaks of a sign table
            keyed by the layer width but gives no values; the signs multiply the
            input before H.
    READING: [P1] calls it a rotation, so the block transform is orthonormal,
            H/sqrt(1024) = H/32 (an exact power of two).  Blocks are contiguous
            from k = 0 ([P1] §1: 17408/2 = 8704 splits a block in the middle).

    Computed densely in binary64: with inputs that are multiples of 2**-31 below
    2**8 in magnitude (the generator's range) every partial sum is an exact
    binary64 number, so this returns the exact rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    T, K = x.shape
    if K % HBLOCK:
        raise ValueError("K must be a multiple of 1024")
    d = np.ones(K) if signs is None else np.asarray(signs, dtype=np.float64)
    H = sylvester_hadamard(HBLOCK)
    out = np.empty_like(x)
    for j in range(K // HBLOCK):
        blk = slice(j * HBLOCK, (j + 1) * HBLOCK)
        out[:, blk] = ((x[:, blk] * d[blk]) @ H.T) / 32.0
    return out


def rotate_f32(x: np.ndarray, signs: np.ndarray | None = None) -> np.ndarray:
    """The exact rotation rounded once to float32 (nearest, ties to even)."""
    return rotate_exact(x, signs).astype(np.float32)


def half_block_stage(x_half: np.ndarray, signs_half: np.ndarray | None = None) -> np.ndarray:
    """First stage of a 1024-block split in the middle by a K-shard boundary:
    u = H512 (d * x_half) for the 512 columns one rank holds, without the 1/32.

    [P1] §1: down_proj's 17408 inputs split over two GPUs at 8704, the middle of a
    block; by H1024 [a; b] = [H512 a + H512 b; H512 a - H512 b] each rank
    transforms only its own half and the halves are exchanged.
    x_half: [T, 512]; signs_half: [512] of +-1 or None.  Dense, binary64 (exact for
    the generator's inputs, as in rotate_exact).
    """
    x = np.asarray(x_half, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != HBLOCK // 2:
        raise ValueError("x_half must be [T, 512]")
    d = np.ones(HBLOCK // 2) if signs_half is None else np.asarray(signs_half, dtype=np.float64)
    return (x * d) @ sylvester_hadamard(HBLOCK // 2).T


def half_block_join(u_lo: np.ndarray, u_hi: np.ndarray, half: int) -> np.ndarray:
    """Second stage: the rotated values of one half of the split block from both
    halves' stage results, rounded once to float32.

    [P1] §1: the rank holding the first half keeps the sum, the other the
    difference.  half 0: (u_lo + u_hi)/32, half 1: (u_lo - u_hi)/32, where u_lo
    and u_hi are the stages of the block's first and second 512 columns.
    """
    if half not in (0, 1):
        raise ValueError("half must be 0 or 1")
    u_lo = np.asarray(u_lo, dtype=np.float64)
    u_hi = np.asarray(u_hi, dtype=np.float64)
    v = u_lo + u_hi if half == 0 else u_lo - u_hi
    return (v / 32.0).astype(np.float32)


# ---------------------------------------------------------------------------
# packed 2-bit codes  ([P1] "前提": 2-bit representation of {-1, 0, +1})
# ---------------------------------------------------------------------------
# The page does not give the bit layout; this one is ours (include/tl.h, ABI 2).
# Word encoding: a uint32 holds 16 codes k = 16w + j; code j sits in byte
# (j mod 4), bit pair (j div 4) of that byte, i.e. at bits 8*(j mod 4) + 2*(j div 4)
# .. +1; field = two's complement low 2 bits: 0 -> 00, +1 -> 01, -1 -> 11.
# Tile order: rows in blocks of 16, K in pairs of 128-groups (zero padded);
# tile (rb, p) = 256 words at 256*(rb*GP + p); its word 4*l + 2*gi + m holds
# codes 128*(2p+gi) + 16*(2*(l//16) + m) + j of row 16*rb + l%16.
def _bitpos(j: np.ndarray) -> np.ndarray:
    return 8 * (j % 4) + 2 * (j // 4)


def encode_words(codes: np.ndarray) -> np.ndarray:
    """codes int8 [N, K] in {-1,0,1} -> row-major words uint32 [N, K/16] (word encoding only)."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    fields = (codes.astype(np.int64) & 3).astype(np.uint64).reshape(N, K // 16, 16)
    shifts = _bitpos(np.arange(16)).astype(np.uint64)
    words = np.zeros((N, K // 16), dtype=np.uint64)
    for j in range(16):
        words |= fields[:, :, j] << shifts[j]
    return words.astype(np.uint32)


def decode_words(words: np.ndarray) -> np.ndarray:
    """Inverse of :func:`encode_words` (field 10 decodes to -2, flagging a bad word)."""
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    N, nw = w.shape
    out = np.empty((N, nw, 16), dtype=np.int8)
    for j in range(16):
        f = (w >> int(_bitpos(np.array(j)))) & 3
        out[:, :, j] = np.where(f >= 2, f - 4, f)
    return out.reshape(N, nw * 16)


def packed_size_words(N: int, K: int) -> int:
    NB, GP = -(-N // 16), -(-K // 256)
    return NB * GP * 256


def _tile_index(N: int, K: int):
    """For every (padded row, padded word column) its index in the tiled array."""
    NB, GP = -(-N // 16), -(-K // 256)
    n = np.arange(NB * 16)[:, None]
    wc = np.arange(GP * 16)[None, :]          # word column: 16 words per group pair
    rb, nl = n // 16, n % 16
    g, w = wc // 8, wc % 8                     # group, word within group
    p, gi = g // 2, g % 2
    q, m = w // 2, w % 2
    lane = 16 * q + nl
    return 256 * (rb * GP + p) + 4 * lane + 2 * gi + m


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes int8 [N, K] -> the tiled packed array, uint32 [packed_size_words(N, K)]."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    NB, GP = -(-N // 16), -(-K // 256)
    padded = np.zeros((NB * 16, GP * 256), dtype=np.int8)
    padded[:N, :K] = codes
    words = encode_words(padded)
    out = np.zeros(packed_size_words(N, K), dtype=np.uint32)
    out[_tile_index(N, K)] = words
    return out


def unpack_codes(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`: codes [N, K] (field 10 decodes to -2)."""
    words = np.asarray(packed, dtype=np.uint32)[_tile_index(N, K)]
    return decode_words(words)[:N, :K]


# ---------------------------------------------------------------------------
# scale decomposition  ([P1] §4, int8 prefill)
# ---------------------------------------------------------------------------
def decompose_scales(scales: np.ndarray):
    """q[n,g] = round(127 * s[n,g] / smax[n]);  row_scale[n] = smax[n] / 127.

    scales : fp16 [N, G].  smax[n] is the row maximum of |s| ([P1] §4 calls it
    the per-row maximum; the absolute value keeps a sign in q if a scale is ever
    negative -- READING).
    Precision and tie rule (READING): the product 127*s is exact in float32, the
    quotient is the correctly rounded float32 division, and round() is
    nearest-ties-to-even (torch.round).  The tests pin this against exact
    rational rounding for every fp16 value.  A row with smax = 0 gives q = 0 and
    row_scale = 0.
    Returns (q int8 [N, G], row_scale float32 [N], smax float32 [N]).
    """
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    smax = np.max(np.abs(s), axis=1)
    num = np.float32(127.0) * s
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = num / smax[:, None]
    quo = np.where(smax[:, None] > 0, quo, np.float32(0.0))
    q = np.rint(quo).astype(np.int8)
    row_scale = (smax / np.float32(127.0)).astype(np.float32)
    return q, row_scale, smax


def int8_weight(codes: np.ndarray, q: np.ndarray) -> np.ndarray:
    """W_int8[n, k] = code[n, k] * q[n, k // 128]  ([P1] §4; exact in int8)."""
    codes = np.asarray(codes, dtype=np.int16)
    qq = np.repeat(np.asarray(q, dtype=np.int16), GROUP, axis=1)
    return (codes * qq).astype(np.int8)


# ---------------------------------------------------------------------------
# per-token int8 activations  ([P1] §4: quantised per token after the rotation)
# ---------------------------------------------------------------------------
def quant_act_int8(xr: np.ndarray):
    """Symmetric per-token int8: sx = amax/127, xq = round(xr / sx).

    READING: the page says only "per token, int8".  Symmetric absmax with range
    +-127 (matching the weights' 127), the scale as the float32 quotient
    amax/127, the code as the correctly rounded float32 quotient xr/sx rounded
    to nearest-even, clamped to [-127, 127].  A row with amax = 0 gives sx = 0 and
    xq = 0.  Returns (xq int8 [T, K], sx float32 [T]).
    """
    x = np.asarray(xr, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    sx = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = x / sx[:, None]
    quo = np.where(sx[:, None] > 0, quo, np.float32(0.0))
    xq = np.clip(np.rint(quo), -127, 127).astype(np.int8)
    return xq, sx


# ---------------------------------------------------------------------------
# decode GEMV  ([P1] "前提": y = W (H_blk x) with W = code * group scale)
# ---------------------------------------------------------------------------
def gemv_ternary(xr: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_g s[n, g] * sum_{k in group g} code[n, k] * xr[t, k]  (binary64).

    xr [b, K] (any float), codes int8 [N, K], scales fp16 [N, K/128] -> y [b, N].
    One library matmul per group computes the inner sums.
    """
    xr = np.asarray(xr, dtype=np.float64)
    codes = np.asarray(codes)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    b, K = xr.shape
    N = codes.shape[0]
    y = np.zeros((b, N), dtype=np.float64)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        inner = xr[:, ks] @ codes[:, ks].astype(np.float64).T      # [b, N]
        y += inner * s[:, g][None, :]
    return y


def gemv_ternary_q8(xq: np.ndarray, sx: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The decode GEMV on the per-token int8 activations of [P1] §4:
    y[t, n] = sx[t] * sum_g s[n, g] * sum_{k in g} code[n, k] * xq[t, k]  (binary64).

    [P1] "5." weighs an int8 (dp4a) decode kernel and sets it aside for its extra
    error; this is that computation, on the same int8 activations the prefill path
    uses.  It is the decode GEMV of the dequantised activations xq * sx (exact in
    binary64: an int8 times a float32).
    """
    xd = np.asarray(xq, dtype=np.float64) * np.asarray(sx, dtype=np.float64)[:, None]
    return gemv_ternary(xd, codes, scales)


# ---------------------------------------------------------------------------
# prefill int8 GEMM and rescale  ([P1] §4)
# ---------------------------------------------------------------------------
def gemm_int8_acc(xq: np.ndarray, codes: np.ndarray, q: np.ndarray, row_chunk: int = 4096) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * W_int8[n, k]  as exact integers (int64).

    The library matmul runs in binary64: every product is an integer of
    magnitude <= 127*127 and every partial sum is an integer below
    K * 127**2 < 2**53, so each step is exact whatever the summation order.
    Rows of W are taken in chunks only to bound memory.
    """
    A = np.asarray(xq, dtype=np.float64)
    N = codes.shape[0]
    out = np.empty((A.shape[0], N), dtype=np.int64)
    for r0 in range(0, N, row_chunk):
        W = int8_weight(codes[r0:r0 + row_chunk], q[r0:r0 + row_chunk]).astype(np.float64)
        out[:, r0:r0 + row_chunk] = np.rint(A @ W.T).astype(np.int64)
    return out


def rescale(acc: np.ndarray, row_scale: np.ndarray, sx: np.ndarray) -> np.ndarray:
    """y[m, n] = acc[m, n] * row_scale[n] * sx[m]  in binary64 ([P1] §4)."""
    return (np.asarray(acc, dtype=np.float64)
            * np.asarray(row_scale, dtype=np.float64)[None, :]
            * np.asarray(sx, dtype=np.float64)[:, None])


# ---------------------------------------------------------------------------
# comparison helpers
# ---------------------------------------------------------------------------
def rel_fro(y: np.ndarray, ref: np.ndarray) -> float:
    """||y - ref||_F / ||ref||_F over the whole tensor; inf if y is not finite."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    den = np.linalg.norm(ref)
    num = np.linalg.norm(y - ref)
    return float(num / den) if den > 0 else float(num)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round binary64 values to the nearest bfloat16 (ties to even), as float64.

    Rounds directly from binary64 (no intermediate float32) by splitting off the
    bits below the bf16 ulp with exact float arithmetic.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    nz = a != 0
    m, e = np.frexp(a[nz])                 # a = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: round m * 2**8 to an integer, ties to even
    out[nz] = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return out
