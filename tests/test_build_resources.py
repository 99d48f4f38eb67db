"""Compiler resource figures of every kernel in libtl (no GPU needed).

The build records, per kernel, what hipcc's kernel-resource-usage remarks report
(registers, scratch bytes per lane, spills, LDS).  The weight-streaming GEMV and
int8 GEMM kernels must never touch scratch memory: a spill there puts per-lane
memory traffic on the hot path, which no timing would explain."""
from __future__ import annotations

import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_gemv_gemm_amd")

# Kernels allowed a few spilled registers: the fused rotation kernels with four
# 1024-blocks per wave, which only inputs wider than 48 blocks (K > 49152) use.
ALLOWED_SPILLS = ("gemv_prep_x_kernelILi4E", "quant_x_kernelILi4E")


@pytest.fixture(scope="module")
def resources():
    from quantized_gemv_gemm_amd import _build
    path = _build.RESOURCES
    srcs = glob.glob(os.path.join(PKG, "csrc", "*"))
    stale = not os.path.exists(path) or os.path.getmtime(path) < max(os.path.getmtime(s) for s in srcs)
    if stale:
        _build.build()
    with open(path) as f:
        return json.load(f)


def test_every_source_reports(resources):
    hip = {os.path.basename(p) for p in glob.glob(os.path.join(PKG, "csrc", "*.hip"))}
    assert {v["source"] for v in resources.values()} == hip


def test_hot_kernels_use_no_scratch(resources):
    hot = {k: v for k, v in resources.items() if v["source"] in ("k_gemv.hip", "k_gemm.hip")}
    assert any("gemm_i8_kernel" in k for k in hot) and any("gemv_stream_kernel" in k for k in hot)
    bad = {k: v for k, v in hot.items() if v.get("scratch", 0) or v.get("vgpr_spill", 0) or v.get("sgpr_spill", 0)}
    assert not bad, f"GEMV/GEMM kernels with scratch or spills: {bad}"


def test_other_kernels_use_no_scratch(resources):
    bad = {k: v for k, v in resources.items()
           if (v.get("scratch", 0) or v.get("vgpr_spill", 0)) and not any(a in k for a in ALLOWED_SPILLS)}
    assert not bad, f"kernels with scratch or spills: {bad}"


def test_gemm_holds_two_workgroups_per_cu(resources):
    """The GEMM schedule assumes two 256-thread workgroups per compute unit: its
    registers must leave two waves per SIMD and its LDS two workgroups."""
    figs = [v for k, v in resources.items() if "gemm_i8_kernel" in k]
    assert len(figs) == 2          # the launches with and without the raised issue priority
    for fig in figs:
        assert fig["occupancy"] >= 2
        assert 2 * fig["lds"] <= 160 * 1024
