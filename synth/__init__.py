"""Seeded synthetic inputs for the ternary linear layer.

This module only draws inputs: it holds none of the layer's arithmetic (no
rotation, packing, scale decomposition, quantisation or contraction). Both the
CPU oracle (through the tests) and the HIP path (through the tests and the
benchmark) take their inputs from here, and from nowhere else.

Value distributions follow the workloads of the ternary 27B model described in
qiita.com/nakanokensetsu/items/ecc183fae033565af7cb ("前提": 2-bit {-1,0,+1}
codes with one scale per 128 weights, bf16 activations):

* codes  : i.i.d. uniform over {-1, 0, +1}
* scales : fp16, lognormal(mu=-4, sigma=0.5), one per (row, 128-group)
* x      : bf16, N(0, 1), with round(0.005*K) outlier input channels (the same
           channels for every token) multiplied by 20.  |x| < 2**-24 is flushed
           to 0 and |x| is kept below 256, so every value is a multiple of
           2**-31 of magnitude < 2**8 (this keeps a 1024-term sum of them exact
           in binary64).

Codes come from a counter-based generator (murmur3's 32-bit finaliser applied
twice to the element index, keyed per layer) so that any row of any layer can
be regenerated on its own, on the host with numpy or on the device with torch,
bit-identically.  Scales and activations use numpy's PCG64 with a SeedSequence
keyed by (seed, stream, layer, tensor); a stream is the number of one workload's
random streams (see WORKLOADS).
"""
from __future__ import annotations

import numpy as np

GROUP = 128          # weights per scale group
HBLOCK = 1024        # Hadamard block width

_M32 = 0xFFFFFFFF
_C1 = 0x85EBCA6B
_C2 = 0xC2B2AE35

TENSOR_CODES, TENSOR_SCALES, TENSOR_X = 1, 2, 3


# ---------------------------------------------------------------------------
# counter-based code generator (numpy and torch twins, bit-identical)
# ---------------------------------------------------------------------------
def _fmix32_np(h):
    h = h & _M32
    h ^= h >> np.uint64(16)
    h = (h * np.uint64(_C1)) & np.uint64(_M32)
    h ^= h >> np.uint64(13)
    h = (h * np.uint64(_C2)) & np.uint64(_M32)
    h ^= h >> np.uint64(16)
    return h


def _key_words(key: int):
    key &= (1 << 64) - 1
    return key & _M32, (key >> 32) & _M32


def ternary_codes(key: int, row0: int, nrows: int, K: int) -> np.ndarray:
    """int8 codes in {-1,0,1} for rows [row0, row0+nrows) of a K-wide layer."""
    k1, k2 = _key_words(key)
    n = np.arange(row0, row0 + nrows, dtype=np.uint64)[:, None]
    k = np.arange(K, dtype=np.uint64)[None, :]
    idx = n * np.uint64(K) + k
    h = _fmix32_np((idx + np.uint64(k1)) & np.uint64(_M32))
    h = _fmix32_np(h ^ np.uint64(k2))
    u = (h * np.uint64(3)) >> np.uint64(32)          # uniform over {0,1,2}
    return (u.astype(np.int16) - 1).astype(np.int8)


def _mul32_t(a, c: int):
    # (a * c) mod 2**32 for 0 <= a < 2**32 held in int64, without overflow
    lo = (a * (c & 0xFFFF)) & _M32
    hi = ((a * (c >> 16)) & 0xFFFF) << 16
    return (lo + hi) & _M32


def _fmix32_t(h):
    h = h & _M32
    h = h ^ (h >> 16)
    h = _mul32_t(h, _C1)
    h = h ^ (h >> 13)
    h = _mul32_t(h, _C2)
    h = h ^ (h >> 16)
    return h


def ternary_codes_torch(key: int, row0: int, nrows: int, K: int, device="cpu"):
    """torch twin of :func:`ternary_codes` (same bits), built on ``device``."""
    import torch
    k1, k2 = _key_words(key)
    n = torch.arange(row0, row0 + nrows, dtype=torch.int64, device=device)[:, None]
    k = torch.arange(K, dtype=torch.int64, device=device)[None, :]
    idx = n * K + k
    h = _fmix32_t((idx + k1) & _M32)
    h = _fmix32_t(h ^ k2)
    u = (h * 3) >> 32
    return (u - 1).to(torch.int8)


# ---------------------------------------------------------------------------
# scales and activations
# ---------------------------------------------------------------------------
def _rng(seed: int, stream: int, layer: int, tensor: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(stream, layer, tensor))
    return np.random.Generator(np.random.PCG64(ss))


def group_scales(seed: int, stream: int, layer: int, N: int, K: int) -> np.ndarray:
    """fp16 scales [N, K/128], lognormal(-4, 0.5) rounded to nearest fp16."""
    rng = _rng(seed, stream, layer, TENSOR_SCALES)
    z = rng.standard_normal((N, K // GROUP))
    return np.exp(-4.0 + 0.5 * z).astype(np.float16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(seed: int, stream: int, layer: int, K: int) -> np.ndarray:
    rng = _rng(seed, stream, layer, TENSOR_X)
    n_out = int(round(0.005 * K))
    return np.sort(rng.permutation(K)[:n_out])


def activations(seed: int, stream: int, layer: int, T: int, K: int) -> np.ndarray:
    """bf16 bit patterns [T, K]: N(0,1) with 0.5% of channels scaled by 20."""
    rng = _rng(seed, stream, layer, TENSOR_X)
    n_out = int(round(0.005 * K))
    chans = np.sort(rng.permutation(K)[:n_out])
    z = rng.standard_normal((T, K))
    z[:, chans] *= 20.0
    z[np.abs(z) < 2.0 ** -24] = 0.0
    z = np.clip(z, -255.0, 255.0)
    return f32_to_bf16_bits(z.astype(np.float32))


# ---------------------------------------------------------------------------
# workload recipes (shapes of the ternary 27B layers)
# ---------------------------------------------------------------------------
# layer types of one decoder block: name -> (K, N)
LAYER_SHAPES = {
    "qkv": (5120, 10240),
    "o": (5120, 5120),
    "gate_up": (5120, 34816),
    "down": (17408, 5120),
}

# the workloads, by name; `stream` numbers each one's random streams (the
# inputs of workload w, layer l come from streams (seed, w["stream"], l, tensor))
WORKLOADS = {
    "tiny": dict(stream=0, layers=[("tiny", 1024, 256)], decode_b=[1], prefill_m=[1]),
    "decode_qkv": dict(stream=1, layers=[("qkv", 5120, 10240)], decode_b=[1, 4, 8, 16], prefill_m=[]),
    "decode_mlp": dict(stream=2, layers=[("gate_up", 5120, 34816), ("down", 17408, 5120)],
                       decode_b=[1, 16], prefill_m=[]),
    "prefill_mlp": dict(stream=3, layers=[("gate_up", 5120, 34816), ("down", 17408, 5120)],
                        decode_b=[], prefill_m=[512]),
    "stack64": dict(stream=4, blocks=64, layers=[(n, *LAYER_SHAPES[n]) for n in ("qkv", "o", "gate_up", "down")],
                    decode_b=[16], prefill_m=[2048]),
}


def layer_key(seed: int, stream: int, layer: int) -> int:
    """64-bit key of the code generator for one layer of one workload stream."""
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(stream, layer, TENSOR_CODES))
    w = ss.generate_state(2, dtype=np.uint32)
    return int(w[0]) | (int(w[1]) << 32)


class LayerInputs:
    """Inputs of one ternary linear layer: codes [N,K] int8, scales [N,K/128] fp16."""

    def __init__(self, seed: int, stream: int, layer: int, K: int, N: int):
        self.seed, self.stream, self.layer, self.K, self.N = seed, stream, layer, K, N
        self.key = layer_key(seed, stream, layer)

    def codes(self, row0: int = 0, nrows: int | None = None) -> np.ndarray:
        nrows = self.N - row0 if nrows is None else nrows
        return ternary_codes(self.key, row0, nrows, self.K)

    def codes_torch(self, device, row0: int = 0, nrows: int | None = None):
        nrows = self.N - row0 if nrows is None else nrows
        return ternary_codes_torch(self.key, row0, nrows, self.K, device)

    def scales(self) -> np.ndarray:
        return group_scales(self.seed, self.stream, self.layer, self.N, self.K)

    def x(self, T: int) -> np.ndarray:
        return activations(self.seed, self.stream, self.layer, T, self.K)
