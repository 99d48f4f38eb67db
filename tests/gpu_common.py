"""Shared helpers of the GPU parity tests (device placement of synth inputs)."""
from __future__ import annotations

import sys

import numpy as np

import synth

REL_TOL = 1e-3   # relative Frobenius bound for floating-point outputs


def announce(msg: str):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, d):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def bf16_dev(bits: np.ndarray, d):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(d).view(torch.bfloat16)


def poison_(t):
    """Fill an output with a value no correct kernel produces before the call."""
    import torch
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    elif t.dtype == torch.int8:
        t.fill_(0x7F)
    else:
        t.fill_(-0x5A5A5A5B)
    return t


class Layer:
    """Host and device copies of one synthetic ternary layer."""

    def __init__(self, seed, stream, layer, K, N, d):
        self.L = synth.LayerInputs(seed, stream, layer, K, N)
        self.K, self.N = K, N
        self.codes = self.L.codes()
        self.scales = self.L.scales()
        self.d = d
        self.codes_d = to_dev(self.codes, d)
        self.scales_d = to_dev(self.scales, d)

    def pack(self):
        import quantized_gemv_gemm_amd as tl
        self.packed, self.q, self.rs = tl.pack_weights(self.codes_d, self.scales_d)
        return self
