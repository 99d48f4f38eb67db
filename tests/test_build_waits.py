"""Counted memory waits in the compiled weight-streaming kernels (no GPU needed).

The GEMV kernels copy limbs, scales and limb scales straight into LDS with
direct (LDS-DMA) loads, then issue their weight-tile (and A-fragment) loads and
wait with s_waitcnt vmcnt(N), N = the number of those later loads, so that the
direct loads are done while the tiles stay in flight.  The counter is in order,
so the wait is only right if at least N loads really are issued after the last
direct load on the way to it; the compiler is free to move ordinary loads (it
once moved two scale loads below the wait, which let a workgroup read LDS
before the direct loads had landed).  This test reads the device assembly the
build writes and checks every such wait: in the straight-line block that ends
at the wait, after the last direct load, at least N loads."""
from __future__ import annotations

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_gemv_gemm_amd")
KERNELS = ("gemv_stream_kernel", "gemv_q8_kernel", "gemv_rot_kernel")


def _read_listing(src):
    from quantized_gemv_gemm_amd import _build
    path = _build.asm_path(src)
    srcs = [os.path.join(PKG, "csrc", f) for f in os.listdir(os.path.join(PKG, "csrc"))]
    if not os.path.exists(path) or os.path.getmtime(path) < max(os.path.getmtime(s) for s in srcs):
        _build.build()
    with open(path) as f:
        return f.read()


@pytest.fixture(scope="module")
def listing():
    return _read_listing("k_gemv.hip")


@pytest.fixture(scope="module")
def gemm_listing():
    return _read_listing("k_gemm.hip")


def _functions(text, kernels=KERNELS):
    pat = r"^(_ZN2tl[^:\n]*(?:%s)[^:\n]*):[^\n]*\n(.*?)^\.Lfunc_end" % "|".join(kernels)
    for name, body in re.findall(pat, text, re.S | re.M):
        lines = []
        for raw in body.split("\n"):
            s = re.sub(r"\s*;.*", "", raw.strip())
            if s and not (s.startswith(".") and not s.endswith(":")):
                lines.append(s)
        yield name, lines


def _is_dma(line):
    op = line.split()[0]
    return op.startswith("global_load_lds") or (op.startswith("buffer_load") and " lds" in line)


def _is_load(line):
    op = line.split()[0]
    return (op.startswith("global_load") or op.startswith("buffer_load")) and not _is_dma(line)


def _counted_wait(name, lines):
    """Index of the hand-counted vmcnt wait: the last vmcnt wait before the first
    barrier (stream, q8), or the first one after the last direct load (rot)."""
    if "gemv_rot_kernel" in name:
        last_dma = max(i for i, l in enumerate(lines) if _is_dma(l))
        return next(i for i in range(last_dma, len(lines)) if lines[i].startswith("s_waitcnt") and "vmcnt(" in lines[i])
    bar = next(i for i, l in enumerate(lines) if l.startswith("s_barrier"))
    return max(i for i in range(bar) if lines[i].startswith("s_waitcnt") and "vmcnt(" in lines[i])


def _claim_and_loads(name, lines):
    """(N of the counted wait, loads issued after the last direct load in the
    straight-line block that ends at it)."""
    w = _counted_wait(name, lines)
    n = int(re.search(r"vmcnt\((\d+)\)", lines[w]).group(1))
    start = max([i for i in range(w) if lines[i].endswith(":") or _is_dma(lines[i])], default=-1)
    return n, sum(1 for l in lines[start + 1:w] if _is_load(l))


def test_listing_has_the_kernels(listing):
    names = [n for n, _ in _functions(listing)]
    for k in KERNELS:
        assert any(k in n for n in names), k


def test_counted_waits_cover_their_loads(listing):
    checked, bad = 0, []
    for name, lines in _functions(listing):
        n, loads = _claim_and_loads(name, lines)
        checked += 1
        if loads < n:
            bad.append(f"{name}: vmcnt({n}) after {loads} loads")
    assert checked > 100
    assert not bad, "\n".join(bad[:10])


def test_checker_flags_a_short_count():
    """The checker itself: a wait that claims more loads than were issued after
    the last direct load (two scale loads sunk below it) is reported; with a
    join label in between only the block after it counts."""
    fake = (
        "_ZN2tl12_GLOBAL__N_118gemv_stream_kernelILi1EEEv: ; @x\n"
        "\tglobal_load_lds_dwordx4 v[4:5], off\n"
        "\tglobal_load_dwordx4 v[6:9], v[2:3], off\n"
        "\tglobal_load_dword v10, v[2:3], off\n"
        "\ts_waitcnt vmcnt(3) lgkmcnt(0)\n"
        "\ts_barrier\n"
        "\tglobal_load_dword v11, v[2:3], off\n"
        "\ts_endpgm\n"
        ".Lfunc_end0:\n"
        "_ZN2tl12_GLOBAL__N_114gemv_q8_kernelILi1EEEv: ; @y\n"
        "\tglobal_load_lds_dwordx4 v[4:5], off\n"
        "\tglobal_load_ushort v1, v[2:3], off\n"
        ".LBB1_2:\n"
        "\tglobal_load_dwordx4 v[6:9], v[2:3], off\n"
        "\ts_waitcnt vmcnt(2)\n"
        "\ts_barrier\n"
        "\ts_endpgm\n"
        ".Lfunc_end1:\n")
    found = {}
    for name, lines in _functions(fake):
        found[name.split("N_")[1][:10]] = _claim_and_loads(name, lines)
    assert found == {"118gemv_st": (3, 2), "114gemv_q8": (2, 1)}


# The GEMM's pair loop: the next pair's activation stage is copied into LDS with
# direct loads at the start of the pair, the weight words of pair p + 2 are
# loaded at its last k-step, and the pair ends with s_waitcnt vmcnt(4 J) and the
# workgroup barrier: the stage must have landed, the 4 J weight loads (two
# 16-byte code loads and two scale bytes per weight column) may stay in flight.


def _gemm_waits(lines):
    """(N, loads after the last direct load, a direct load in the block) for every
    vmcnt(N) wait, 0 < N < 63, that a barrier follows."""
    out = []
    for i, line in enumerate(lines):
        if not (line.startswith("s_barrier") and i and lines[i - 1].startswith("s_waitcnt")):
            continue
        m = re.search(r"vmcnt\((\d+)\)", lines[i - 1])
        if not m or not 0 < int(m.group(1)) < 63:
            continue
        w = i - 1
        start = max([j for j in range(w) if lines[j].endswith(":") or _is_dma(lines[j])], default=-1)
        out.append((int(m.group(1)), sum(1 for l in lines[start + 1:w] if _is_load(l)),
                    start >= 0 and _is_dma(lines[start])))
    return out


def test_gemm_counted_waits_cover_their_loads(gemm_listing):
    checked, bad = 0, []
    for name, lines in _functions(gemm_listing, ("gemm_i8_kernel",)):
        for n, loads, dma in _gemm_waits(lines):
            checked += 1
            if not dma or loads < n:
                bad.append(f"{name[:60]}: vmcnt({n}) after {loads} loads (direct load in the block: {dma})")
    assert checked >= 8
    assert not bad, "\n".join(bad[:10])


def test_gemm_checker_flags_a_short_count():
    """A pair whose weight loads were moved above its direct loads is reported."""
    fake = (
        "_ZN2tl12_GLOBAL__N_114gemm_i8_kernelILb1EEEv: ; @z\n"
        "\tbuffer_load_dwordx4 v[6:9], v1, s[0:3], 0 offen\n"
        "\tbuffer_load_dwordx4 v168, s[28:31], s55 offen lds\n"
        "\tv_mfma_i32_32x32x32_i8 v[18:33], v[226:229], v[130:133], v[18:33]\n"
        "\tbuffer_load_ubyte v2, v3, s[4:7], 0 offen\n"
        "\ts_waitcnt vmcnt(2)\n"
        "\ts_barrier\n"
        "\ts_endpgm\n"
        ".Lfunc_end2:\n")
    ((name, lines),) = list(_functions(fake, ("gemm_i8_kernel",)))
    assert _gemm_waits(lines) == [(2, 1, True)]
