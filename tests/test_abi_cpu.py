"""The C ABI library loads and exports what include/tl.h declares; host-side checks.

No compute call reaches the GPU here: every call below is rejected by the
library's host-side argument checks (or is a zero-size no-op) before any HIP
runtime call, so these tests run without a GPU.
"""
import ctypes
import os
import re

import pytest

import quantized_gemv_gemm_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tl.LIB_PATH), reason="libtl.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(tl_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert {"tl_pack_weights", "tl_hadamard_blk", "tl_gemv_ternary", "tl_quant_act_int8",
            "tl_gemm_int8_rescale"} <= set(names)
    L = ctypes.CDLL(tl.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # the binding declares exactly the header's functions
    assert set(tl._SIGS) == set(names)


def test_version_and_status_strings():
    assert tl.abi_version() == 2
    assert tl.packed_words(16, 256) == 256 and tl.packed_words(17, 384) == 1024
    assert tl.packed_words(40, 1024) == 3072 and tl.lib().tl_packed_bytes(4, 100) == 0
    for s in range(0, 9):
        assert tl.status_string(s)
    assert tl.status_string(0) == "ok"
    assert tl.status_string(99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(0x20000000)
FAKE3 = ctypes.c_void_p(0x40000000)
FAKE4 = ctypes.c_void_p(0x60000000)
FAKE5 = ctypes.c_void_p(0x80000000)
ODD = ctypes.c_void_p(0x10004)


def test_pack_rejections():
    L = tl.lib()
    assert L.tl_pack_weights(FAKE, FAKE2, 4, 100, FAKE3, FAKE4, FAKE5, None, None) == 2   # K % 128
    assert L.tl_pack_weights(FAKE, FAKE2, -1, 128, FAKE3, FAKE4, FAKE5, None, None) == 2
    assert L.tl_pack_weights(FAKE, FAKE2, 4, 0, FAKE3, FAKE4, FAKE5, None, None) == 2
    assert L.tl_pack_weights(None, FAKE2, 4, 128, FAKE3, FAKE4, FAKE5, None, None) == 1
    assert L.tl_pack_weights(ODD, FAKE2, 4, 128, FAKE3, FAKE4, FAKE5, None, None) == 3
    assert L.tl_pack_weights(FAKE, FAKE2, 4, 128, FAKE, FAKE4, FAKE5, None, None) == 8   # packed aliases codes
    assert L.tl_pack_weights(FAKE, FAKE2, 0, 128, FAKE3, FAKE4, FAKE5, None, None) == 0   # empty: no-op


def test_hadamard_rejections():
    L = tl.lib()
    assert L.tl_hadamard_blk(FAKE, 2, 1536, None, FAKE2, None) == 2       # K % 1024
    assert L.tl_hadamard_blk(FAKE, 2, 1024, None, None, None) == 1
    assert L.tl_hadamard_blk(FAKE, 2, 1024, ODD, FAKE2, None) == 3        # signs misaligned
    assert L.tl_hadamard_blk(FAKE, 2, 1024, None, FAKE, None) == 8
    assert L.tl_hadamard_blk(FAKE, 0, 1024, None, FAKE2, None) == 0


def test_gemv_rejections():
    L = tl.lib()
    ws = L.tl_gemv_workspace_size(4, 1024, 256)
    assert ws >= 2 * 4 * 1024
    assert L.tl_gemv_workspace_size(65, 1024, 256) == 0
    assert L.tl_gemv_workspace_size(64, 1024, 256) >= 2 * 64 * 1024
    args = lambda b=4, K=1024, N=256, y=FAKE4, dt=0, w=FAKE5, wb=ws: (FAKE, b, K, N, FAKE2, FAKE3, y, dt, w, wb, None)
    assert L.tl_gemv_ternary(*args(b=65)) == 2
    assert L.tl_gemv_ternary(*args(b=64, wb=ws)) == 7   # 64 tokens need a larger workspace
    assert L.tl_gemv_ternary(*args(K=1000)) == 2
    assert L.tl_gemv_ternary(*args(dt=7)) == 4
    assert L.tl_gemv_ternary(*args(y=None)) == 1
    assert L.tl_gemv_ternary(*args(w=None)) == 7
    assert L.tl_gemv_ternary(*args(wb=ws - 1)) == 7
    assert L.tl_gemv_ternary(*args(y=ODD)) == 3
    assert L.tl_gemv_ternary(*args(y=FAKE)) == 8
    assert L.tl_gemv_ternary(*args(b=0)) == 0
    assert L.tl_gemv_ternary(*args(N=0)) == 0


def test_gemv_q8_rejections():
    L = tl.lib()
    args = lambda b=4, K=1024, N=256, sx=FAKE5, y=FAKE4, dt=0: (FAKE, sx, b, K, N, FAKE2, FAKE3, y, dt, None)
    assert L.tl_gemv_ternary_q8(*args(b=17)) == 2
    assert L.tl_gemv_ternary_q8(*args(K=1000)) == 2
    assert L.tl_gemv_ternary_q8(*args(dt=7)) == 4
    assert L.tl_gemv_ternary_q8(*args(y=None)) == 1
    assert L.tl_gemv_ternary_q8(*args(sx=None)) == 1
    assert L.tl_gemv_ternary_q8(*args(y=ODD)) == 3
    assert L.tl_gemv_ternary_q8(*args(y=FAKE)) == 8
    assert L.tl_gemv_ternary_q8(*args(b=16, K=128 * 200)) == 6   # too many group pairs per wave
    assert L.tl_gemv_ternary_q8(*args(b=0)) == 0
    assert L.tl_gemv_ternary_q8(*args(N=0)) == 0


def test_quant_rejections():
    L = tl.lib()
    assert L.tl_quant_act_int8(FAKE, 3, 100, FAKE2, FAKE3, None) == 2
    assert L.tl_quant_act_int8(FAKE, 3, 128, None, FAKE3, None) == 1
    assert L.tl_quant_act_int8(FAKE, 3, 128, FAKE2, ODD, None) == 3
    assert L.tl_quant_act_int8(FAKE, 3, 128, FAKE, FAKE3, None) == 8
    assert L.tl_quant_act_int8(FAKE, 0, 128, FAKE2, FAKE3, None) == 0


def test_gemm_rejections():
    L = tl.lib()
    args = lambda M=8, K=1024, N=256, y=FAKE4, dt=1, acc=None: (
        FAKE, FAKE2, M, K, N, FAKE3, FAKE4, FAKE5, y, dt, acc, None, 0, None)
    assert L.tl_gemm_int8_rescale(*args(K=133248)) == 2     # accumulator could overflow int32
    assert L.tl_gemm_int8_rescale(*args(K=1000)) == 2
    assert L.tl_gemm_int8_rescale(*args(dt=3)) == 4
    assert L.tl_gemm_int8_rescale(*args(y=None)) == 1
    assert L.tl_gemm_int8_rescale(*args(acc=ODD, y=ctypes.c_void_p(0xA0000000))) == 3
    assert L.tl_gemm_int8_rescale(*args(y=FAKE, K=128)) == 8   # one pair of groups: no workspace
    assert L.tl_gemm_int8_rescale(*args(y=FAKE)) == 7            # 8 x 1024 x 256 is split along K
    assert L.tl_gemm_int8_rescale(*args(M=0)) == 0
    assert L.tl_gemm_int8_rescale(*args(N=0)) == 0
    assert L.tl_gemm_int8_rescale(*args(M=-1)) == 2
    # 512 x 40960 leaves 128 of 640 tiles for a last round: they are split along K;
    # 512 x 34816 leaves 32 of 544, cut into sub-tiles that need no workspace
    need = L.tl_gemm_workspace_size(512, 5120, 40960)
    assert need > 0 and L.tl_gemm_workspace_size(512, 5120, 32768) == 0
    assert L.tl_gemm_workspace_size(512, 5120, 34816) == 0
    big = lambda ws, wb: (FAKE, FAKE2, 512, 5120, 40960, FAKE3, FAKE4, FAKE5, ctypes.c_void_p(0xA0000000),
                          1, None, ws, wb, None)
    assert L.tl_gemm_int8_rescale(*big(None, 0)) == 7
    assert L.tl_gemm_int8_rescale(*big(ctypes.c_void_p(0xC0000000), need - 1)) == 7
    assert L.tl_gemm_int8_rescale(*big(ctypes.c_void_p(0xC0000008), need)) == 3


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        tl.hadamard_blk(torch.zeros((1, 1024), dtype=torch.bfloat16))


def test_fused_input_rejections():
    L = tl.lib()
    ws = L.tl_gemv_workspace_size(4, 1024, 256)
    assert L.tl_gemv_prepare_x(FAKE, 4, 1536, None, FAKE2, ws, None) == 2          # K % 1024
    assert L.tl_gemv_prepare_x(FAKE, 4, 66560, None, FAKE2, 1 << 30, None) == 6    # K > 65536: unfused calls
    assert L.tl_gemv_prepare_x(FAKE, 65, 1024, None, FAKE2, ws, None) == 2
    assert L.tl_gemv_prepare_x(None, 4, 1024, None, FAKE2, ws, None) == 1
    assert L.tl_gemv_prepare_x(FAKE, 4, 1024, None, FAKE2, ws - 1, None) == 7
    assert L.tl_gemv_prepare_x(FAKE, 4, 1024, ODD, FAKE2, ws, None) == 3
    assert L.tl_gemv_prepare_x(FAKE, 4, 1024, None, FAKE, ws, None) == 8
    assert L.tl_gemv_prepare_x(FAKE, 0, 1024, None, FAKE2, ws, None) == 0
    gx = lambda b=4, K=1024, N=256, dt=0, w=FAKE5, wb=ws: (FAKE, b, K, N, None, FAKE2, FAKE3, FAKE4, dt, w, wb, None)
    assert L.tl_gemv_ternary_x(*gx(K=1152)) == 2
    assert L.tl_gemv_ternary_x(*gx(dt=5)) == 4
    assert L.tl_gemv_ternary_x(*gx(w=None)) == 7
    assert L.tl_gemv_ternary_x(*gx(N=0)) == 0
    assert L.tl_quant_act_int8_x(FAKE, 3, 1152, None, FAKE2, FAKE3, None) == 2
    assert L.tl_quant_act_int8_x(FAKE, 3, 66560, None, FAKE2, FAKE3, None) == 6
    assert L.tl_quant_act_int8_x(FAKE, 3, 1024, None, None, FAKE3, None) == 1
    assert L.tl_quant_act_int8_x(FAKE, 3, 1024, None, FAKE2, ODD, None) == 3
    assert L.tl_quant_act_int8_x(FAKE, 3, 1024, None, FAKE, FAKE3, None) == 8
    assert L.tl_quant_act_int8_x(FAKE, 0, 1024, None, FAKE2, FAKE3, None) == 0


def test_linear_path_rule():
    """Up to 16 tokens the GEMV; 17..64 while ceil(T/16) N K <= 2^27; above 64 the int8 path."""
    P = tl.linear_path
    for T in (0, 1, 8, 16):
        assert P(T, 5120, 34816) == tl.PATH_GEMV and P(T, 17408, 1 << 20) == tl.PATH_GEMV
    assert P(32, 5120, 10240) == tl.PATH_GEMV      # qkv: 2 chunks x 52.4e6 weights
    assert P(33, 5120, 10240) == tl.PATH_INT8      # 3 chunks
    assert P(17, 17408, 5120) == tl.PATH_INT8      # down: 2 chunks x 89.1e6
    assert P(17, 5120, 34816) == tl.PATH_INT8      # gate_up: 2 chunks x 178e6
    assert P(17, 1024, 65536) == tl.PATH_GEMV      # exactly 2^27 streamed weights
    assert P(17, 1024, 65537) == tl.PATH_INT8
    assert P(65, 1024, 64) == tl.PATH_INT8 and P(512, 5120, 10240) == tl.PATH_INT8

def test_linear_rejections():
    L = tl.lib()
    ws = L.tl_linear_workspace_size(5, 1024, 256)
    assert ws >= 1024 + L.tl_gemv_workspace_size(5, 1024, 256)
    ws8 = L.tl_linear_workspace_size(100, 1024, 256)   # int8 path: counters, xq, tok_scale
    assert ws8 >= 1024 + 100 * 1024 + 400
    assert L.tl_linear_workspace_size(5, 1000, 256) == 0
    W = ctypes.c_void_p(0xC0000000)
    args = lambda T=5, K=1024, N=256, y=FAKE4, dt=0, w=W, wb=ws, qq=FAKE3: (
        FAKE, T, K, N, None, FAKE2, ctypes.c_void_p(0x30000000), qq, FAKE5, y, dt, w, wb, None)
    assert L.tl_linear_apply(*args(K=1152)) == 2
    assert L.tl_linear_apply(*args(K=66560, wb=1 << 40)) == 6
    assert L.tl_linear_apply(*args(dt=9)) == 4
    assert L.tl_linear_apply(*args(qq=None)) == 1
    assert L.tl_linear_apply(*args(w=None)) == 7
    assert L.tl_linear_apply(*args(wb=ws - 1)) == 7
    assert L.tl_linear_apply(*args(T=100, wb=ws)) == 7            # the int8 path needs more
    assert L.tl_linear_apply(*args(y=ODD)) == 3
    assert L.tl_linear_apply(*args(y=FAKE)) == 8
    assert L.tl_linear_apply(*args(T=0)) == 0 and L.tl_linear_apply(*args(N=0)) == 0


def test_split_block_rejections():
    L = tl.lib()
    assert L.tl_hadamard_half(FAKE, 2, 500, None, FAKE2, None) == 2          # ldx < 512
    assert L.tl_hadamard_half(FAKE, 2, 8704, None, None, None) == 1
    assert L.tl_hadamard_half(FAKE, 2, 8700, None, FAKE2, None) == 3         # rows not 16-byte aligned
    assert L.tl_hadamard_half(FAKE, 2, 8704, None, ODD, None) == 3
    assert L.tl_hadamard_half(FAKE, 2, 512, None, FAKE, None) == 8
    assert L.tl_hadamard_half(FAKE, 0, 512, None, FAKE2, None) == 0
    assert L.tl_hadamard_join(FAKE, FAKE2, 2, 2, FAKE3, 512, None) == 2       # half must be 0 or 1
    assert L.tl_hadamard_join(FAKE, FAKE2, 2, 0, FAKE3, 100, None) == 2
    assert L.tl_hadamard_join(FAKE, None, 2, 0, FAKE3, 512, None) == 1
    assert L.tl_hadamard_join(FAKE, FAKE2, 2, 1, FAKE3, 514, None) == 3
    assert L.tl_hadamard_join(FAKE, FAKE2, 2, 1, FAKE2, 512, None) == 8
    assert L.tl_hadamard_join(FAKE, FAKE2, 0, 1, FAKE3, 512, None) == 0


def test_gemv_plan_that_does_not_fit_is_unsupported():
    """A weight-stream variant whose LDS would exceed a compute unit's 160 KB is
    refused on the host (TL_ERR_UNSUPPORTED), before any launch: K = 409600 puts
    3200 group scales of 32 rows (204 KB) into the long-K variant's LDS."""
    L = tl.lib()
    K, N = 409600, 8192
    ws = L.tl_gemv_workspace_size(1, K, N)
    assert ws > 0
    big = ctypes.c_size_t(1 << 40)
    assert L.tl_gemv_prepared(FAKE, big, 1, K, N, FAKE2, FAKE3, FAKE4, 1, None) == 6


def test_read_probe_rejections():
    L = tl.lib()
    assert L.tl_read_probe(FAKE, 100, FAKE2, None) == 2      # not a multiple of 16
    assert L.tl_read_probe(FAKE, 0, FAKE2, None) == 2
    assert L.tl_read_probe(None, 1024, FAKE2, None) == 1
    assert L.tl_read_probe(ODD, 1024, FAKE2, None) == 3
    assert L.tl_read_probe(FAKE, 1024, FAKE, None) == 8      # sink inside the source
    assert L.tl_mfma_probe(1, 0, FAKE2, None) == 2            # no iterations
    assert L.tl_mfma_probe(0, 10, None, None) == 1
    assert L.tl_mfma_probe(1, 10, ODD, None) == 3
