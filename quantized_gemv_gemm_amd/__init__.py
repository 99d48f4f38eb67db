"""Python binding of libtl, the ternary linear-layer library for MI355X (gfx950).

The functions mirror the C ABI in include/tl.h one to one.  They only check
tensor dtypes/devices/contiguity, allocate outputs with torch when none are
given, and pass raw pointers and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if
libtl.so is missing or a call fails, a RuntimeError is raised.

Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb ("前提",
"1. TP=2 への移植", "4. 効いた高速化").
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtl.so")

TL_BF16, TL_F32 = 0, 1
GROUP, HBLOCK = 128, 1024

_lib = None

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tl.h
_SIGS = {
    "tl_abi_version": (ctypes.c_int, []),
    "tl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tl_last_kernel_name": (ctypes.c_char_p, []),
    "tl_last_error_detail": (ctypes.c_char_p, []),
    "tl_packed_bytes": (_c_sz, [_c_i64, _c_i64]),
    "tl_pack_weights": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "tl_hadamard_blk": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "tl_hadamard_half": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "tl_hadamard_join": (ctypes.c_int, [_c_p, _c_p, _c_i64, ctypes.c_int, _c_p, _c_i64, _c_p]),
    "tl_gemv_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "tl_gemv_ternary": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, ctypes.c_int,
                                       _c_p, _c_sz, _c_p]),
    "tl_gemv_prepare": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_sz, _c_p]),
    "tl_gemv_prepared": (ctypes.c_int, [_c_p, _c_sz, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, ctypes.c_int,
                                        _c_p]),
    "tl_gemv_ternary_q8": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, ctypes.c_int,
                                          _c_p]),
    "tl_quant_act_int8": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "tl_gemv_prepare_x": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_sz, _c_p]),
    "tl_gemv_ternary_x": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, ctypes.c_int,
                                         _c_p, _c_sz, _c_p]),
    "tl_quant_act_int8_x": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "tl_gemm_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "tl_gemm_int8_rescale": (ctypes.c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                            ctypes.c_int, _c_p, _c_p, _c_sz, _c_p]),
    "tl_linear_path": (ctypes.c_int, [_c_i64, _c_i64, _c_i64]),
    "tl_linear_workspace_size": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "tl_linear_apply": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                       ctypes.c_int, _c_p, _c_sz, _c_p]),
    "tl_noalloc_scratch_bytes": (_c_sz, []),
    "tl_read_probe": (ctypes.c_int, [_c_p, _c_sz, _c_p, _c_p]),
    "tl_mfma_probe": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_p, _c_p]),
    "tl_linear_apply_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                               _c_p, ctypes.c_int, _c_p]),
}

PATH_GEMV, PATH_INT8 = 0, 1


def lib():
    """The loaded libtl.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        # One HIP runtime per process: torch ships its own libamdhip64 (needed as
        # "libamdhip64.so"), libtl needs "libamdhip64.so.7".  Loading torch first makes
        # the dynamic linker resolve libtl's dependency to torch's copy (same SONAME),
        # so device memory, streams and kernels all live in one runtime.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().tl_status_string(s).decode()


def last_kernel_name() -> str:
    return lib().tl_last_kernel_name().decode()


def abi_version() -> int:
    return lib().tl_abi_version()


def _check(name: str, status: int):
    if status != 0:
        detail = lib().tl_last_error_detail().decode() if status == 5 else ""
        raise RuntimeError(f"{name} failed: {status_string(status)} (status {status}) {detail}".rstrip())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _out_code(dtype):
    import torch
    if dtype == torch.bfloat16:
        return TL_BF16
    if dtype == torch.float32:
        return TL_F32
    raise TypeError("output dtype must be torch.bfloat16 or torch.float32")


# ---------------------------------------------------------------------------
# the five calls
# ---------------------------------------------------------------------------
def packed_words(N: int, K: int) -> int:
    """Number of uint32 words of the packed (tiled) weights of an [N, K] layer."""
    return int(lib().tl_packed_bytes(N, K)) // 4


def _check_packed(packed, N, K):
    import torch
    _need(packed, "packed", torch.int32, 1)
    if packed.numel() != packed_words(N, K):
        raise ValueError(f"packed must hold {packed_words(N, K)} words for N={N}, K={K}")


def pack_weights(codes, scales, packed=None, q=None, row_scale=None, invalid_count=None):
    """codes int8 [N,K], scales fp16 [N,K/128] -> (packed int32 [packed_words(N,K)] (the uint32
    tile words of the layout in include/tl.h), q int8 [N,K/128], row_scale f32 [N])."""
    import torch
    _need(codes, "codes", torch.int8, 2)
    _need(scales, "scales", torch.float16, 2)
    N, K = codes.shape
    dev = codes.device
    packed = torch.empty((packed_words(N, K),), dtype=torch.int32, device=dev) if packed is None else packed
    q = torch.empty((N, K // GROUP), dtype=torch.int8, device=dev) if q is None else q
    row_scale = torch.empty((N,), dtype=torch.float32, device=dev) if row_scale is None else row_scale
    _check_packed(packed, N, K)
    _need(q, "q", torch.int8, 2)
    _need(row_scale, "row_scale", torch.float32, 1)
    if invalid_count is not None:
        _need(invalid_count, "invalid_count", torch.int32, 1)
    if scales.shape != (N, K // GROUP) or q.shape != (N, K // GROUP) or row_scale.shape != (N,):
        raise ValueError("shape mismatch in pack_weights")
    _check("tl_pack_weights", lib().tl_pack_weights(
        _ptr(codes), _ptr(scales), N, K, _ptr(packed), _ptr(q), _ptr(row_scale), _ptr(invalid_count),
        _stream(dev)))
    return packed, q, row_scale


def hadamard_blk(x, signs=None, out=None):
    """x bf16 [T,K] -> xr f32 [T,K]: exact block rotation (1/32) H1024 (d * x), rounded once."""
    import torch
    _need(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    if signs is not None:
        _need(signs, "signs", torch.int8, 1)
        if signs.shape != (K,):
            raise ValueError("signs must be [K]")
    out = torch.empty((T, K), dtype=torch.float32, device=x.device) if out is None else out
    _need(out, "out", torch.float32, 2)
    if out.shape != (T, K):
        raise ValueError("out must be [T, K]")
    _check("tl_hadamard_blk", lib().tl_hadamard_blk(_ptr(x), T, K, _ptr(signs), _ptr(out), _stream(x.device)))
    return out


def _check_x(x, signs):
    import torch
    _need(x, "x", torch.bfloat16, 2)
    if signs is not None:
        _need(signs, "signs", torch.int8, 1)
        if signs.shape != (x.shape[1],):
            raise ValueError("signs must be [K]")


def gemv_prepare_x(x, workspace, signs=None):
    """Fused rotation + GEMV prep: limbs of the rotated x bf16 [b,K] into ``workspace``
    (bit-identical to gemv_prepare(hadamard_blk(x, signs)))."""
    import torch
    _check_x(x, signs)
    _need(workspace, "workspace", torch.uint8, 1)
    b, K = x.shape
    _check("tl_gemv_prepare_x", lib().tl_gemv_prepare_x(_ptr(x), b, K, _ptr(signs), _ptr(workspace),
                                                        workspace.numel(), _stream(x.device)))
    return workspace


def gemv_ternary_x(x, packed, scales, signs=None, out_dtype=None, out=None, workspace=None):
    """Decode layer from the raw input: x bf16 [b,K] -> y [b,N] (rotation fused into the prep)."""
    import torch
    _check_x(x, signs)
    _need(scales, "scales", torch.float16, 2)
    b, K = x.shape
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP):
        raise ValueError("shape mismatch in gemv_ternary_x")
    if out is None:
        out = torch.empty((b, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (b, N):
        raise ValueError("out must be [b, N]")
    need = gemv_workspace_size(b, K, N)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check("tl_gemv_ternary_x", lib().tl_gemv_ternary_x(
        _ptr(x), b, K, N, _ptr(signs), _ptr(packed), _ptr(scales), _ptr(out), code, _ptr(workspace),
        workspace.numel(), _stream(x.device)))
    return out


def quant_act_int8_x(x, signs=None, xq=None, tok_scale=None):
    """Fused rotation + per-token int8: x bf16 [T,K] -> (xq int8 [T,K], tok_scale f32 [T])
    (bit-identical to quant_act_int8(hadamard_blk(x, signs)))."""
    import torch
    _check_x(x, signs)
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.int8, device=x.device) if xq is None else xq
    tok_scale = torch.empty((T,), dtype=torch.float32, device=x.device) if tok_scale is None else tok_scale
    _need(xq, "xq", torch.int8, 2)
    _need(tok_scale, "tok_scale", torch.float32, 1)
    if xq.shape != (T, K) or tok_scale.shape != (T,):
        raise ValueError("shape mismatch in quant_act_int8_x")
    _check("tl_quant_act_int8_x", lib().tl_quant_act_int8_x(_ptr(x), T, K, _ptr(signs), _ptr(xq),
                                                            _ptr(tok_scale), _stream(x.device)))
    return xq, tok_scale


def gemv_workspace_size(b: int, K: int, N: int) -> int:
    return int(lib().tl_gemv_workspace_size(b, K, N))


def gemv_ternary(xr, packed, scales, out_dtype=None, out=None, workspace=None):
    """xr f32 [b,K] (b <= 64), packed tiles, scales fp16 [N,K/128] -> y [b,N]."""
    import torch
    _need(xr, "xr", torch.float32, 2)
    _need(scales, "scales", torch.float16, 2)
    b, K = xr.shape
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP):
        raise ValueError("shape mismatch in gemv_ternary")
    if out is None:
        out = torch.empty((b, N), dtype=out_dtype or torch.bfloat16, device=xr.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (b, N):
        raise ValueError("out must be [b, N]")
    need = gemv_workspace_size(b, K, N)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=xr.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check("tl_gemv_ternary", lib().tl_gemv_ternary(
        _ptr(xr), b, K, N, _ptr(packed), _ptr(scales), _ptr(out), code, _ptr(workspace),
        workspace.numel(), _stream(xr.device)))
    return out


def gemv_ternary_q8(xq, tok_scale, packed, scales, out_dtype=None, out=None):
    """Decode GEMV against int8 activations: xq int8 [b,K] and tok_scale f32 [b]
    (from quant_act_int8 / quant_act_int8_x), packed tiles, scales -> y [b,N]."""
    import torch
    _need(xq, "xq", torch.int8, 2)
    _need(tok_scale, "tok_scale", torch.float32, 1)
    _need(scales, "scales", torch.float16, 2)
    b, K = xq.shape
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP) or tok_scale.shape != (b,):
        raise ValueError("shape mismatch in gemv_ternary_q8")
    if out is None:
        out = torch.empty((b, N), dtype=out_dtype or torch.bfloat16, device=xq.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (b, N):
        raise ValueError("out must be [b, N]")
    _check("tl_gemv_ternary_q8", lib().tl_gemv_ternary_q8(
        _ptr(xq), _ptr(tok_scale), b, K, N, _ptr(packed), _ptr(scales), _ptr(out), code, _stream(xq.device)))
    return out


def gemv_prepare(xr, workspace):
    """First stage of gemv_ternary: activation limbs of xr f32 [b,K] into ``workspace``."""
    import torch
    _need(xr, "xr", torch.float32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    b, K = xr.shape
    _check("tl_gemv_prepare", lib().tl_gemv_prepare(_ptr(xr), b, K, _ptr(workspace), workspace.numel(),
                                                    _stream(xr.device)))
    return workspace


def gemv_prepared(workspace, b, K, packed, scales, out):
    """Second stage of gemv_ternary: y [b,N] from a workspace filled by gemv_prepare(b, K)."""
    import torch
    _need(workspace, "workspace", torch.uint8, 1)
    _need(scales, "scales", torch.float16, 2)
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP) or out.shape != (b, N):
        raise ValueError("shape mismatch in gemv_prepared")
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    _check("tl_gemv_prepared", lib().tl_gemv_prepared(
        _ptr(workspace), workspace.numel(), b, K, N, _ptr(packed), _ptr(scales), _ptr(out), code,
        _stream(out.device)))
    return out


def quant_act_int8(xr, xq=None, tok_scale=None):
    """xr f32 [T,K] -> (xq int8 [T,K], tok_scale f32 [T])."""
    import torch
    _need(xr, "xr", torch.float32, 2)
    T, K = xr.shape
    xq = torch.empty((T, K), dtype=torch.int8, device=xr.device) if xq is None else xq
    tok_scale = torch.empty((T,), dtype=torch.float32, device=xr.device) if tok_scale is None else tok_scale
    _need(xq, "xq", torch.int8, 2)
    _need(tok_scale, "tok_scale", torch.float32, 1)
    if xq.shape != (T, K) or tok_scale.shape != (T,):
        raise ValueError("shape mismatch in quant_act_int8")
    _check("tl_quant_act_int8", lib().tl_quant_act_int8(_ptr(xr), T, K, _ptr(xq), _ptr(tok_scale),
                                                        _stream(xr.device)))
    return xq, tok_scale


_GEMM_WS = {}


def _gemm_workspace(device, nbytes):
    """A zero-filled GEMM workspace per (device, stream), grown on demand.

    The kernels return the workspace's counters to zero at the end of every
    call, so one buffer serves every call issued on that stream."""
    import torch
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _GEMM_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device=device)
        _GEMM_WS[key] = ws
    return ws


def gemm_workspace_size(M: int, K: int, N: int) -> int:
    return int(lib().tl_gemm_workspace_size(M, K, N))


def gemm_int8_rescale(xq, tok_scale, packed, q, row_scale, out_dtype=None, out=None, acc_out=None,
                      want_acc=False, workspace=None):
    """xq int8 [M,K], tok_scale f32 [M], packed/q/row_scale from pack_weights -> y [M,N]
    (and the exact int32 accumulator when ``want_acc`` or ``acc_out`` is given)."""
    import torch
    _need(xq, "xq", torch.int8, 2)
    _need(tok_scale, "tok_scale", torch.float32, 1)
    _need(q, "q", torch.int8, 2)
    _need(row_scale, "row_scale", torch.float32, 1)
    M, K = xq.shape
    N = q.shape[0]
    _check_packed(packed, N, K)
    if tok_scale.shape != (M,) or q.shape != (N, K // GROUP) or row_scale.shape != (N,):
        raise ValueError("shape mismatch in gemm_int8_rescale")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=xq.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (M, N):
        raise ValueError("out must be [M, N]")
    if acc_out is None and want_acc:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    if acc_out is not None:
        _need(acc_out, "acc_out", torch.int32, 2)
        if acc_out.shape != (M, N):
            raise ValueError("acc_out must be [M, N]")
    need = gemm_workspace_size(M, K, N)
    if workspace is None and need:
        workspace = _gemm_workspace(xq.device, need)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check("tl_gemm_int8_rescale", lib().tl_gemm_int8_rescale(
        _ptr(xq), _ptr(tok_scale), M, K, N, _ptr(packed), _ptr(q), _ptr(row_scale), _ptr(out), code,
        _ptr(acc_out), _ptr(workspace), ws_bytes, _stream(xq.device)))
    return (out, acc_out) if acc_out is not None else out


def linear_path(T: int, K: int, N: int) -> int:
    """PATH_GEMV or PATH_INT8: the path linear_apply takes for T tokens of a K -> N layer."""
    return int(lib().tl_linear_path(T, K, N))


def linear_workspace_size(T: int, K: int, N: int) -> int:
    return int(lib().tl_linear_workspace_size(T, K, N))


_LIN_WS = {}


def _linear_workspace(device, nbytes):
    """A zero-filled layer workspace per (device, stream), grown on demand (every
    call leaves its counter region at zero, so one buffer serves every call)."""
    import torch
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _LIN_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device=device)
        _LIN_WS[key] = ws
    return ws


def linear_apply(x, packed, scales, q, row_scale, signs=None, out_dtype=None, out=None, workspace=None):
    """The whole layer from the raw input: x bf16 [T,K] -> y [T,N], on the path
    linear_path(T, K, N) names (two-limb GEMV, or int8 quantisation + int8 GEMM)."""
    import torch
    _check_x(x, signs)
    _need(scales, "scales", torch.float16, 2)
    _need(q, "q", torch.int8, 2)
    _need(row_scale, "row_scale", torch.float32, 1)
    T, K = x.shape
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP) or q.shape != (N, K // GROUP) or row_scale.shape != (N,):
        raise ValueError("shape mismatch in linear_apply")
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (T, N):
        raise ValueError("out must be [T, N]")
    need = linear_workspace_size(T, K, N)
    if workspace is None:
        workspace = _linear_workspace(x.device, max(need, 1))
    _need(workspace, "workspace", torch.uint8, 1)
    _check("tl_linear_apply", lib().tl_linear_apply(
        _ptr(x), T, K, N, _ptr(signs), _ptr(packed), _ptr(scales), _ptr(q), _ptr(row_scale), _ptr(out), code,
        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out


def read_probe(src, sink):
    """Measurement helper: one launch that only reads the bytes of ``src`` (see
    tl_read_probe); ``sink`` is a 4-byte (or larger) device tensor."""
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous()):
        raise ValueError("read_probe needs contiguous device tensors")
    nbytes = src.numel() * src.element_size() // 16 * 16
    _check("tl_read_probe", lib().tl_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(src.device)))


def mfma_probe(random_operands, iters, sink):
    """Measurement helper: one launch that only issues int8 matrix instructions
    (see tl_mfma_probe); ``sink`` is a 4-byte (or larger) device tensor."""
    if not sink.is_cuda:
        raise ValueError("mfma_probe needs a device tensor")
    _check("tl_mfma_probe", lib().tl_mfma_probe(1 if random_operands else 0, int(iters), _ptr(sink),
                                                _stream(sink.device)))


def noalloc_scratch_bytes() -> int:
    """Size of the static per-GPU scratch array behind linear_apply_noalloc."""
    return int(lib().tl_noalloc_scratch_bytes())


def linear_apply_noalloc(x, packed, scales, q, row_scale, signs=None, out_dtype=None, out=None):
    """linear_apply without a workspace: the library's static per-GPU scratch array
    serves instead (same kernels, same outputs).  Calls that overlap in time on
    one GPU share that array and race.  ``out`` may be given so that the call
    allocates nothing at all."""
    import torch
    _check_x(x, signs)
    _need(scales, "scales", torch.float16, 2)
    _need(q, "q", torch.int8, 2)
    _need(row_scale, "row_scale", torch.float32, 1)
    T, K = x.shape
    N = scales.shape[0]
    _check_packed(packed, N, K)
    if scales.shape != (N, K // GROUP) or q.shape != (N, K // GROUP) or row_scale.shape != (N,):
        raise ValueError("shape mismatch in linear_apply_noalloc")
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    code = _out_code(out.dtype)
    _need(out, "out", out.dtype, 2)
    if out.shape != (T, N):
        raise ValueError("out must be [T, N]")
    _check("tl_linear_apply_noalloc", lib().tl_linear_apply_noalloc(
        _ptr(x), T, K, N, _ptr(signs), _ptr(packed), _ptr(scales), _ptr(q), _ptr(row_scale), _ptr(out), code,
        _stream(x.device)))
    return out


def _need_rows(t, name, dtype, cols):
    """A 2-D device tensor of ``cols`` contiguous columns whose rows may be further apart."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype or t.dim() != 2 or t.shape[1] != cols or t.stride(1) != 1:
        raise ValueError(f"{name} must be a {dtype} [T, {cols}] view with unit column stride")


def hadamard_half(x, signs=None, u=None):
    """First split-block stage: x bf16 [T,512] (rows may be a column slice of a wider
    input) -> u f64 [T,512] = H512 (d * x), exact, no 1/32."""
    import torch
    _need_rows(x, "x", torch.bfloat16, 512)
    if signs is not None:
        _need(signs, "signs", torch.int8, 1)
        if signs.shape != (512,):
            raise ValueError("signs must be [512]")
    T = x.shape[0]
    u = torch.empty((T, 512), dtype=torch.float64, device=x.device) if u is None else u
    _need(u, "u", torch.float64, 2)
    if u.shape != (T, 512):
        raise ValueError("u must be [T, 512]")
    _check("tl_hadamard_half", lib().tl_hadamard_half(_ptr(x), T, x.stride(0) if T > 1 else 512, _ptr(signs),
                                                      _ptr(u), _stream(x.device)))
    return u


def hadamard_join(u_lo, u_hi, half, out=None):
    """Second split-block stage: the rank's 512 rotated columns, f32 [T,512]
    (``out`` may be a column slice of the rank's rotated input)."""
    import torch
    _need(u_lo, "u_lo", torch.float64, 2)
    _need(u_hi, "u_hi", torch.float64, 2)
    T = u_lo.shape[0]
    if u_lo.shape != (T, 512) or u_hi.shape != (T, 512):
        raise ValueError("u_lo and u_hi must be [T, 512]")
    out = torch.empty((T, 512), dtype=torch.float32, device=u_lo.device) if out is None else out
    _need_rows(out, "out", torch.float32, 512)
    if out.shape[0] != T:
        raise ValueError("out must have T rows")
    _check("tl_hadamard_join", lib().tl_hadamard_join(_ptr(u_lo), _ptr(u_hi), T, int(half), _ptr(out),
                                                      out.stride(0) if T > 1 else 512, _stream(u_lo.device)))
    return out
