"""Python binding of libjetfp8.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/jetfp8.h)
and takes torch tensors: torch provides device memory and the current HIP
stream, nothing else.  Every step of the computation runs in the library's
HIP kernels; if the library is missing, importing this module fails.

E4M3 codes are held in torch.uint8 tensors (torch.float8_e4m3fn tensors are
accepted and viewed as bytes).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libjetfp8.so")

JET_OK, JET_ERR_NULL, JET_ERR_SHAPE, JET_ERR_ALIGN, JET_ERR_DTYPE, JET_ERR_WORKSPACE, JET_ERR_HIP = range(7)
JET_BF16, JET_F32, JET_E4M3 = 1, 2, 3
JET_OP_FWD, JET_OP_DGRAD, JET_OP_WGRAD = 0, 1, 2

_p, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float

# name -> argtypes, in header order
SIGNATURES = {
    "jet_abi_version": [],
    "jet_status_string": [_i32],
    "jet_last_error": [],
    "jet_quant_act_1x128": [_p, _i64, _i64, _i64, _p, _i64, _p, _p],
    "jet_quant_act_128x1_T": [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _p],
    "jet_quant_act_1x128_128x1_T": [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _i32, _p],
    "jet_quant_weight_128x128": [_p, _i64, _i64, _i64, _p, _p, _p, _p],
    "jet_rmsnorm_quant_1x128": [_p, _p, _i64, _i64, _i64, _f32, _p, _i64, _p, _i64, _p, _p],
    "jet_kv_calibrate": [_p, _p, _i64, _i64, _i64, _i64, _p, _p],
    "jet_kv_append": [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _i64, _i64, _p],
    "jet_swiglu_quant_1x128": [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p],
    "jet_fp8_linear_fwd": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _sz, _p],
    "jet_fp8_linear_fwd_batch_invariant": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _p, _p],
    "jet_fp8_linear_dgrad": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _sz, _p],
    "jet_fp8_linear_wgrad": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _i32, _p, _sz, _p],
    "jet_workspace_bytes": [_i32, _i64, _i64, _i64],
    "jet_quant_act_128x1_T_grouped": [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p],
    "jet_fp8_grouped_fwd": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _p, _p, _sz, _p],
    "jet_fp8_grouped_dgrad": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _sz, _p],
    "jet_fp8_grouped_wgrad": [_p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i32, _i32, _p,
                              _sz, _p],
    "jet_quant_act_1x128_pow2": [_p, _i64, _i64, _i64, _p, _i64, _p, _p],
    "jet_quant_act_128x1_T_pow2": [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _p],
    "jet_quant_act_1x128_128x1_T_pow2": [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _i32, _p],
    "jet_quant_weight_128x128_pow2": [_p, _i64, _i64, _i64, _p, _p, _p, _p],
    "jet_fp8_linear_fwd_pow2": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _p, _p],
    "jet_fp8_linear_dgrad_pow2": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p],
    "jet_fp8_linear_wgrad_pow2": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _i32, _p],
    "jet_rmsnorm_quant_1x128_pow2": [_p, _p, _i64, _i64, _i64, _f32, _p, _i64, _p, _i64, _p, _p],
    "jet_swiglu_quant_1x128_pow2": [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p],
    "jet_quant_act_128x1_T_grouped_pow2": [_p, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _p],
    "jet_fp8_grouped_fwd_pow2": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _i32, _p, _p, _p],
    "jet_fp8_grouped_dgrad_pow2": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, _i32, _p],
    "jet_fp8_grouped_wgrad_pow2": [_p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i32, _i32, _p],
}
_RESTYPES = {"jet_status_string": ctypes.c_char_p, "jet_last_error": ctypes.c_char_p,
             "jet_workspace_bytes": _sz}


class JetError(RuntimeError):
    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed: {_status_name(status)}: {detail}")
        self.status = status


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m fp8_blockwise_quantized_amd._build`")
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    return lib


_lib = load_library()


def _status_name(status: int) -> str:
    return _lib.jet_status_string(status).decode()


def _check(name: str, status: int) -> None:
    if status != JET_OK:
        raise JetError(name, status, _lib.jet_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _codes(t):
    if t is None:
        return None
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError("E4M3 codes must be uint8 or float8_e4m3fn tensors")
    return t


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with a contiguous last dimension")
    return t


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------------------
def jet_abi_version() -> int:
    return _lib.jet_abi_version()


def jet_status_string(status: int) -> str:
    return _status_name(status)


def jet_last_error() -> str:
    return _lib.jet_last_error().decode()


def jet_workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(_lib.jet_workspace_bytes(op, M, N, K))


def jet_quant_act_1x128(x, q=None, s=None, stream=None):
    """x BF16 [M, K] -> (q uint8 [M, K], s float32 [K/128, M])."""
    return _quant_1x128("jet_quant_act_1x128", x, q, s, stream)


def jet_quant_act_1x128_pow2(x, q=None, s=None, stream=None):
    """As jet_quant_act_1x128 with power-of-two scales."""
    return _quant_1x128("jet_quant_act_1x128_pow2", x, q, s, stream)


def _quant_1x128(name, x, q, s, stream):
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    q = _codes(q) if q is not None else _empty((M, K), torch.uint8, x)
    s = s if s is not None else _empty((K // 128, M), torch.float32, x)
    _rowmajor(q, "q")
    _check(name, getattr(_lib, name)(
        _ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(s), _stream(stream)))
    return q, s


def jet_kv_calibrate(k, v, kv_scales=None, stream=None):
    """Per-tensor FP8 KV-cache scales from the BF16 K and V rows [T, D] of a
    calibration batch.  Returns kv_scales float32 [6]: s_k, r_k, s_v, r_v
    (then two working words)."""
    _rowmajor(k, "k")
    _rowmajor(v, "v")
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("k and v must be bfloat16")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    T, D = k.shape
    kv_scales = kv_scales if kv_scales is not None else _empty((6,), torch.float32, k)
    _check("jet_kv_calibrate", _lib.jet_kv_calibrate(
        _ptr(k), _ptr(v), T, D, k.stride(0), v.stride(0), _ptr(kv_scales), _stream(stream)))
    return kv_scales


def jet_kv_append(k, v, slots, kv_scales, k_cache, v_cache, stream=None):
    """Quantize the BF16 K and V rows [T, D] with the stored multipliers and
    write them to cache rows slots[t] (int64 [T]; outside [0, rows) skipped)."""
    _rowmajor(k, "k")
    _rowmajor(v, "v")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if slots.dtype != torch.int64 or slots.dim() != 1 or not slots.is_contiguous() or slots.numel() != k.shape[0]:
        raise TypeError("slots must be a contiguous int64 tensor [T]")
    k_cache, v_cache = _codes(k_cache), _codes(v_cache)
    _rowmajor(k_cache, "k_cache")
    if k_cache.shape != v_cache.shape or k_cache.stride(0) != v_cache.stride(0):
        raise ValueError("k_cache and v_cache must have the same shape and row stride")
    T, D = k.shape
    _check("jet_kv_append", _lib.jet_kv_append(
        _ptr(k), _ptr(v), T, D, k.stride(0), v.stride(0), _ptr(slots), _ptr(kv_scales), _ptr(k_cache),
        _ptr(v_cache), k_cache.stride(0), k_cache.shape[0], _stream(stream)))


def jet_rmsnorm_quant_1x128(x, gamma, eps, y=None, return_y=False, q=None, s=None, stream=None):
    """RMSNorm of each row of x BF16 [M, H] with weight gamma BF16 [H], fused
    with its 1x128 quantization.  Returns (q uint8 [M, H], s float32 [H/128, M]),
    or (y, q, s) with the BF16 RMSNorm output y when return_y (or y given)."""
    return _rmsnorm_quant("jet_rmsnorm_quant_1x128", x, gamma, eps, y, return_y, q, s, stream)


def jet_rmsnorm_quant_1x128_pow2(x, gamma, eps, y=None, return_y=False, q=None, s=None, stream=None):
    """As jet_rmsnorm_quant_1x128 with power-of-two scales."""
    return _rmsnorm_quant("jet_rmsnorm_quant_1x128_pow2", x, gamma, eps, y, return_y, q, s, stream)


def _rmsnorm_quant(name, x, gamma, eps, y, return_y, q, s, stream):
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16:
        raise TypeError("x and gamma must be bfloat16")
    if gamma.dim() != 1 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous 1-D tensor")
    M, H = x.shape
    if gamma.numel() != H:
        raise ValueError("gamma must have H elements")
    if y is None and return_y:
        y = _empty((M, H), torch.bfloat16, x)
    if y is not None:
        _rowmajor(y, "y")
    q = _codes(q) if q is not None else _empty((M, H), torch.uint8, x)
    s = s if s is not None else _empty((H // 128, M), torch.float32, x)
    _rowmajor(q, "q")
    _check(name, getattr(_lib, name)(
        _ptr(x), _ptr(gamma), M, H, x.stride(0), float(eps), _ptr(y), 0 if y is None else y.stride(0),
        _ptr(q), q.stride(0), _ptr(s), _stream(stream)))
    return (y, q, s) if y is not None else (q, s)


def jet_swiglu_quant_1x128(gu, inter=None, h=None, return_h=False, q=None, s=None, stream=None):
    """SwiGLU of the fused gate+up output gu BF16 [M, 2I] (gate = columns
    0..I-1, up = I..2I-1), fused with its 1x128 quantization.  Returns
    (q uint8 [M, I], s float32 [I/128, M]), or (h, q, s) with the BF16 h when
    return_h (or h given)."""
    return _swiglu_quant("jet_swiglu_quant_1x128", gu, inter, h, return_h, q, s, stream)


def jet_swiglu_quant_1x128_pow2(gu, inter=None, h=None, return_h=False, q=None, s=None, stream=None):
    """As jet_swiglu_quant_1x128 with power-of-two scales."""
    return _swiglu_quant("jet_swiglu_quant_1x128_pow2", gu, inter, h, return_h, q, s, stream)


def _swiglu_quant(name, gu, inter, h, return_h, q, s, stream):
    _rowmajor(gu, "gu")
    if gu.dtype != torch.bfloat16:
        raise TypeError("gu must be bfloat16")
    M = gu.shape[0]
    I = gu.shape[1] // 2 if inter is None else int(inter)
    if h is None and return_h:
        h = _empty((M, I), torch.bfloat16, gu)
    if h is not None:
        _rowmajor(h, "h")
    q = _codes(q) if q is not None else _empty((M, I), torch.uint8, gu)
    s = s if s is not None else _empty((I // 128, M), torch.float32, gu)
    _rowmajor(q, "q")
    _check(name, getattr(_lib, name)(
        _ptr(gu), M, I, gu.stride(0), _ptr(h), 0 if h is None else h.stride(0), _ptr(q), q.stride(0),
        _ptr(s), _stream(stream)))
    return (h, q, s) if h is not None else (q, s)


def jet_quant_act_128x1_T(src, src_s=None, qT=None, sT=None, stream=None):
    """128x1 groups along rows, written transposed.

    src BF16 [M, K] (src_s None), or E4M3 codes [M, K] with 1x128 scales
    src_s [K/128, M].  Returns (qT uint8 [K, Mp], sT float32 [Mp/128, K]),
    Mp = ceil(M/128)*128.
    """
    return _quant_128x1_T("jet_quant_act_128x1_T", src, src_s, qT, sT, stream)


def jet_quant_act_128x1_T_pow2(src, src_s=None, qT=None, sT=None, stream=None):
    """As jet_quant_act_128x1_T with power-of-two scales."""
    return _quant_128x1_T("jet_quant_act_128x1_T_pow2", src, src_s, qT, sT, stream)


def _quant_128x1_T(name, src, src_s, qT, sT, stream):
    _rowmajor(src, "src")
    M, K = src.shape
    if src_s is None:
        if src.dtype != torch.bfloat16:
            raise TypeError("src must be bfloat16 when src_s is None")
        dt = JET_BF16
    else:
        src = _codes(src)
        dt = JET_E4M3
    Mp = -(-M // 128) * 128
    qT = _codes(qT) if qT is not None else _empty((K, Mp), torch.uint8, src)
    sT = sT if sT is not None else _empty((Mp // 128, K), torch.float32, src)
    _rowmajor(qT, "qT")
    _check(name, getattr(_lib, name)(
        _ptr(src), dt, _ptr(src_s), M, K, src.stride(0), _ptr(qT), qT.stride(0), _ptr(sT),
        _stream(stream)))
    return qT, sT


def jet_quant_act_1x128_128x1_T(x, requant, q=None, s=None, qT=None, sT=None, stream=None):
    """Both groupings of a BF16 [M, K] tensor from one read.

    Returns (q uint8 [M, K], s float32 [K/128, M], qT uint8 [K, Mp],
    sT float32 [Mp/128, K]), equal to jet_quant_act_1x128(x) and to
    jet_quant_act_128x1_T(x) (requant False) or jet_quant_act_128x1_T(q, s)
    (requant True).
    """
    return _quant_1x128_128x1_T("jet_quant_act_1x128_128x1_T", x, requant, q, s, qT, sT, stream)


def jet_quant_act_1x128_128x1_T_pow2(x, requant, q=None, s=None, qT=None, sT=None, stream=None):
    """As jet_quant_act_1x128_128x1_T with power-of-two scales."""
    return _quant_1x128_128x1_T("jet_quant_act_1x128_128x1_T_pow2", x, requant, q, s, qT, sT, stream)


def _quant_1x128_128x1_T(name, x, requant, q, s, qT, sT, stream):
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    M, K = x.shape
    Mp = -(-M // 128) * 128
    q = _codes(q) if q is not None else _empty((M, K), torch.uint8, x)
    s = s if s is not None else _empty((K // 128, M), torch.float32, x)
    qT = _codes(qT) if qT is not None else _empty((K, Mp), torch.uint8, x)
    sT = sT if sT is not None else _empty((Mp // 128, K), torch.float32, x)
    _rowmajor(q, "q")
    _rowmajor(qT, "qT")
    _check(name, getattr(_lib, name)(
        _ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(s), _ptr(qT), qT.stride(0),
        _ptr(sT), 1 if requant else 0, _stream(stream)))
    return q, s, qT, sT


def jet_quant_weight_128x128(w, q=None, s=None, qT=None, transposed=True, stream=None):
    """w BF16 [N, K] -> (q uint8 [N, K], s float32 [N/128, K/128], qT uint8 [K, N] or None)."""
    return _quant_weight("jet_quant_weight_128x128", w, q, s, qT, transposed, stream)


def jet_quant_weight_128x128_pow2(w, q=None, s=None, qT=None, transposed=True, stream=None):
    """As jet_quant_weight_128x128 with power-of-two scales."""
    return _quant_weight("jet_quant_weight_128x128_pow2", w, q, s, qT, transposed, stream)


def _quant_weight(name, w, q, s, qT, transposed, stream):
    _rowmajor(w, "w")
    if w.dtype != torch.bfloat16:
        raise TypeError("w must be bfloat16")
    N, K = w.shape
    q = _codes(q) if q is not None else _empty((N, K), torch.uint8, w)
    s = s if s is not None else _empty((N // 128, K // 128), torch.float32, w)
    if transposed and qT is None:
        qT = _empty((K, N), torch.uint8, w)
    qT = _codes(qT)
    _check(name, getattr(_lib, name)(
        _ptr(w), N, K, w.stride(0), _ptr(q), _ptr(s), _ptr(qT), _stream(stream)))
    return q, s, qT


def _dtype_code(dt):
    return {torch.bfloat16: JET_BF16, torch.float32: JET_F32}[dt]


def jet_fp8_linear_fwd(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                       yq=None, ys=None, workspace=None, stream=None):
    """Y = deq(xq) . deq(wq)^T.  Returns y, or (y, yq, ys) with fuse_quant."""
    xq, wq = _codes(xq), _codes(wq)
    M, K = xq.shape
    N = wq.shape[0]
    y = y if y is not None else _empty((M, N), out_dtype, xq)
    if fuse_quant:
        yq = _codes(yq) if yq is not None else _empty((M, N), torch.uint8, xq)
        ys = ys if ys is not None else _empty((N // 128, M), torch.float32, xq)
    need = jet_workspace_bytes(JET_OP_FWD, M, N, K)
    if workspace is None and need:
        workspace = _empty((need,), torch.uint8, xq)
    _check("jet_fp8_linear_fwd", _lib.jet_fp8_linear_fwd(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype),
        _ptr(yq), _ptr(ys), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_fwd_batch_invariant(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                                       yq=None, ys=None, stream=None):
    """As jet_fp8_linear_fwd, with each output row bit-identical at every M
    (no workspace)."""
    xq, wq = _codes(xq), _codes(wq)
    M, K = xq.shape
    N = wq.shape[0]
    y = y if y is not None else _empty((M, N), out_dtype, xq)
    if fuse_quant:
        yq = _codes(yq) if yq is not None else _empty((M, N), torch.uint8, xq)
        ys = ys if ys is not None else _empty((N // 128, M), torch.float32, xq)
    _check("jet_fp8_linear_fwd_batch_invariant", _lib.jet_fp8_linear_fwd_batch_invariant(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype), _ptr(yq), _ptr(ys),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_dgrad(dyq, dys, wqT, ws, dx=None, out_dtype=torch.bfloat16, workspace=None,
                         stream=None):
    """dX = deq(dyq) . deq(W); wqT is the transposed weight codes [K, N]."""
    dyq, wqT = _codes(dyq), _codes(wqT)
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = dx if dx is not None else _empty((M, K), out_dtype, dyq)
    need = jet_workspace_bytes(JET_OP_DGRAD, M, N, K)
    if workspace is None and need:
        workspace = _empty((need,), torch.uint8, dyq)
    _check("jet_fp8_linear_dgrad", _lib.jet_fp8_linear_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), M, N, K, _ptr(dx), _dtype_code(dx.dtype),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))
    return dx


def jet_fp8_linear_wgrad(dyqT, dysT, xqT, xsT, M, dw=None, out_dtype=torch.float32,
                         accumulate=False, workspace=None, stream=None):
    """dW (+)= deq(dyqT) . deq(xqT)^T over the M tokens (operands [N, Mp], [K, Mp])."""
    dyqT, xqT = _codes(dyqT), _codes(xqT)
    N, K = dyqT.shape[0], xqT.shape[0]
    dw = dw if dw is not None else _empty((N, K), out_dtype, dyqT)
    need = jet_workspace_bytes(JET_OP_WGRAD, M, N, K)
    if workspace is None and need:
        workspace = _empty((need,), torch.uint8, dyqT)
    _check("jet_fp8_linear_wgrad", _lib.jet_fp8_linear_wgrad(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), M, N, K, _ptr(dw), _dtype_code(dw.dtype),
        1 if accumulate else 0, _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(stream)))
    return dw


def jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                            yq=None, ys=None, stream=None):
    """Forward on power-of-two-scaled operands (scales applied by the MFMA).
    Returns y, or (y, yq, ys) with the power-of-two 1x128 quantization of Y."""
    xq, wq = _codes(xq), _codes(wq)
    M, K = xq.shape
    N = wq.shape[0]
    y = y if y is not None else _empty((M, N), out_dtype, xq)
    if fuse_quant:
        yq = _codes(yq) if yq is not None else _empty((M, N), torch.uint8, xq)
        ys = ys if ys is not None else _empty((N // 128, M), torch.float32, xq)
    _check("jet_fp8_linear_fwd_pow2", _lib.jet_fp8_linear_fwd_pow2(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype), _ptr(yq), _ptr(ys),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_dgrad_pow2(dyq, dys, wqT, ws, dx=None, out_dtype=torch.bfloat16, stream=None):
    """DGrad on power-of-two-scaled operands; wqT the transposed weight codes [K, N]."""
    dyq, wqT = _codes(dyq), _codes(wqT)
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = dx if dx is not None else _empty((M, K), out_dtype, dyq)
    _check("jet_fp8_linear_dgrad_pow2", _lib.jet_fp8_linear_dgrad_pow2(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), M, N, K, _ptr(dx), _dtype_code(dx.dtype), _stream(stream)))
    return dx


def jet_fp8_linear_wgrad_pow2(dyqT, dysT, xqT, xsT, M, dw=None, out_dtype=torch.float32, accumulate=False,
                              stream=None):
    """WGrad on power-of-two-scaled 128x1 operands ([N, Mp], [K, Mp])."""
    dyqT, xqT = _codes(dyqT), _codes(xqT)
    N, K = dyqT.shape[0], xqT.shape[0]
    dw = dw if dw is not None else _empty((N, K), out_dtype, dyqT)
    _check("jet_fp8_linear_wgrad_pow2", _lib.jet_fp8_linear_wgrad_pow2(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), M, N, K, _ptr(dw), _dtype_code(dw.dtype),
        1 if accumulate else 0, _stream(stream)))
    return dw


# ---------------------------------------------------------------------------
# Grouped (mixture-of-experts) layer: seg_off is a device int32 tensor [E+1]
# ---------------------------------------------------------------------------
def grouped_columns(M: int, E: int) -> int:
    """Column capacity of the padded transposed grouped layout: 128*(ceil(M/128)+E)."""
    return (-(-M // 128) + E) * 128


def _seg(seg_off):
    if seg_off.dtype != torch.int32 or seg_off.dim() != 1 or not seg_off.is_contiguous():
        raise TypeError("seg_off must be a contiguous 1-D int32 device tensor [E+1]")
    return seg_off, seg_off.numel() - 1


def jet_quant_act_128x1_T_grouped(src, seg_off, src_s=None, qT=None, sT=None, stream=None):
    """Grouped 128x1 transposed quantization.  Returns (qT uint8 [K, P], sT float32 [P/128, K]),
    P = grouped_columns(M, E); columns past the padded total are left as allocated."""
    return _quant_128x1_T_grouped("jet_quant_act_128x1_T_grouped", src, seg_off, src_s, qT, sT, stream)


def jet_quant_act_128x1_T_grouped_pow2(src, seg_off, src_s=None, qT=None, sT=None, stream=None):
    """As jet_quant_act_128x1_T_grouped with power-of-two scales."""
    return _quant_128x1_T_grouped("jet_quant_act_128x1_T_grouped_pow2", src, seg_off, src_s, qT, sT, stream)


def _quant_128x1_T_grouped(name, src, seg_off, src_s, qT, sT, stream):
    _rowmajor(src, "src")
    seg_off, E = _seg(seg_off)
    M, K = src.shape
    if src_s is None:
        if src.dtype != torch.bfloat16:
            raise TypeError("src must be bfloat16 when src_s is None")
        dt = JET_BF16
    else:
        src = _codes(src)
        dt = JET_E4M3
    P = grouped_columns(M, E)
    qT = _codes(qT) if qT is not None else _empty((K, P), torch.uint8, src)
    sT = sT if sT is not None else _empty((qT.stride(0) // 128, K), torch.float32, src)
    _rowmajor(qT, "qT")
    _check(name, getattr(_lib, name)(
        _ptr(src), dt, _ptr(src_s), M, K, src.stride(0), _ptr(seg_off), E, _ptr(qT), qT.stride(0),
        _ptr(sT), _stream(stream)))
    return qT, sT


def jet_fp8_grouped_fwd(xq, xs, wq, ws, seg_off, y=None, out_dtype=torch.bfloat16,
                        fuse_quant=False, yq=None, ys=None, workspace=None, stream=None):
    """Y rows of expert e = deq(xq_e) . deq(wq[e])^T; wq [E, N, K], ws [E, N/128, K/128]."""
    xq, wq = _codes(xq), _codes(wq)
    seg_off, E = _seg(seg_off)
    M, K = xq.shape
    N = wq.shape[1]
    y = y if y is not None else _empty((M, N), out_dtype, xq)
    if fuse_quant:
        yq = _codes(yq) if yq is not None else _empty((M, N), torch.uint8, xq)
        ys = ys if ys is not None else _empty((N // 128, M), torch.float32, xq)
    # the grouped GEMMs take no workspace (a caller's buffer is passed through)
    _check("jet_fp8_grouped_fwd", _lib.jet_fp8_grouped_fwd(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(y),
        _dtype_code(y.dtype), _ptr(yq), _ptr(ys), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_grouped_dgrad(dyq, dys, wqT, ws, seg_off, dx=None, out_dtype=torch.bfloat16,
                          workspace=None, stream=None):
    """dX rows of expert e = deq(dyq_e) . deq(W_e); wqT [K, E*N] (stacked transposed codes)."""
    dyq, wqT = _codes(dyq), _codes(wqT)
    seg_off, E = _seg(seg_off)
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = dx if dx is not None else _empty((M, K), out_dtype, dyq)
    # the grouped GEMMs take no workspace (a caller's buffer is passed through)
    _check("jet_fp8_grouped_dgrad", _lib.jet_fp8_grouped_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(dx),
        _dtype_code(dx.dtype), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(stream)))
    return dx


def jet_fp8_grouped_wgrad(dyqT, dysT, xqT, xsT, seg_off, M, dw=None, out_dtype=torch.float32,
                          accumulate=False, workspace=None, stream=None):
    """dW_e (+)= deq(dyqT_e) . deq(xqT_e)^T; operands in the padded grouped layout [N, P], [K, P]."""
    dyqT, xqT = _codes(dyqT), _codes(xqT)
    seg_off, E = _seg(seg_off)
    N, K = dyqT.shape[0], xqT.shape[0]
    if dyqT.stride(0) != xqT.stride(0):
        raise ValueError("dyqT and xqT need the same row stride")
    dw = dw if dw is not None else _empty((E, N, K), out_dtype, dyqT)
    # the grouped GEMMs take no workspace (a caller's buffer is passed through)
    _check("jet_fp8_grouped_wgrad", _lib.jet_fp8_grouped_wgrad(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), dyqT.stride(0), _ptr(seg_off), E, M, N, K,
        _ptr(dw), _dtype_code(dw.dtype), 1 if accumulate else 0, _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    return dw


def jet_fp8_grouped_fwd_pow2(xq, xs, wq, ws, seg_off, y=None, out_dtype=torch.bfloat16,
                             fuse_quant=False, yq=None, ys=None, stream=None):
    """jet_fp8_grouped_fwd on power-of-two-scaled operands (scales applied by the MFMA)."""
    xq, wq = _codes(xq), _codes(wq)
    seg_off, E = _seg(seg_off)
    M, K = xq.shape
    N = wq.shape[1]
    y = y if y is not None else _empty((M, N), out_dtype, xq)
    if fuse_quant:
        yq = _codes(yq) if yq is not None else _empty((M, N), torch.uint8, xq)
        ys = ys if ys is not None else _empty((N // 128, M), torch.float32, xq)
    _check("jet_fp8_grouped_fwd_pow2", _lib.jet_fp8_grouped_fwd_pow2(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(y),
        _dtype_code(y.dtype), _ptr(yq), _ptr(ys), _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_grouped_dgrad_pow2(dyq, dys, wqT, ws, seg_off, dx=None, out_dtype=torch.bfloat16, stream=None):
    """jet_fp8_grouped_dgrad on power-of-two-scaled operands."""
    dyq, wqT = _codes(dyq), _codes(wqT)
    seg_off, E = _seg(seg_off)
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = dx if dx is not None else _empty((M, K), out_dtype, dyq)
    _check("jet_fp8_grouped_dgrad_pow2", _lib.jet_fp8_grouped_dgrad_pow2(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(dx),
        _dtype_code(dx.dtype), _stream(stream)))
    return dx


def jet_fp8_grouped_wgrad_pow2(dyqT, dysT, xqT, xsT, seg_off, M, dw=None, out_dtype=torch.float32,
                               accumulate=False, stream=None):
    """jet_fp8_grouped_wgrad on power-of-two-scaled operands."""
    dyqT, xqT = _codes(dyqT), _codes(xqT)
    seg_off, E = _seg(seg_off)
    N, K = dyqT.shape[0], xqT.shape[0]
    if dyqT.stride(0) != xqT.stride(0):
        raise ValueError("dyqT and xqT need the same row stride")
    dw = dw if dw is not None else _empty((E, N, K), out_dtype, dyqT)
    _check("jet_fp8_grouped_wgrad_pow2", _lib.jet_fp8_grouped_wgrad_pow2(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), dyqT.stride(0), _ptr(seg_off), E, M, N, K,
        _ptr(dw), _dtype_code(dw.dtype), 1 if accumulate else 0, _stream(stream)))
    return dw
