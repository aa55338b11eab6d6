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

# JET_LIB_PATH names another build of the same library (the host-sanitized
# build of the CPU validation tests); the default is the in-tree build.
_LIB_PATH = os.environ.get("JET_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                          "libjetfp8.so")

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
    "jet_fp8_linear_fwd_noalloc": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _p, _p, _p],
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


def _dense(t, name, shape, dtypes):
    """The GEMM entry points take dense operands (no leading dimensions): t
    must be a contiguous tensor of exactly `shape` with a dtype in `dtypes`."""
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")
    return t


def _mult128(name, v):
    if v % 128:
        raise ValueError(f"{name} must be a multiple of 128 (got {v})")


def _codes_out(q, name, rows, cols, like, min_ld=None):
    """A row-major E4M3 output [rows, cols] (row stride >= min_ld, default cols)."""
    q = _codes(q) if q is not None else _empty((rows, cols), torch.uint8, like)
    _rowmajor(q, name)
    if q.shape[0] != rows or q.shape[1] < cols or (min_ld is None and q.shape[1] != cols):
        raise ValueError(f"{name} must have {rows} rows of {cols} codes, not shape {tuple(q.shape)}")
    if rows > 1 and q.stride(0) < (cols if min_ld is None else min_ld):
        raise ValueError(f"{name} row stride {q.stride(0)} is too small")
    return q


def _scales_out(s, name, shape, like):
    s = s if s is not None else _empty(shape, torch.float32, like)
    return _dense(s, name, shape, _F32)


def _workspace(workspace, need, like, stream):
    """The caller's workspace (checked) or, when it needs one and gave none, a
    new one that the caching allocator keeps from other work until `stream`
    has finished with it."""
    if workspace is None:
        if not need:
            return None
        workspace = _empty((need,), torch.uint8, like)
        if stream is not None:
            workspace.record_stream(stream)
        return workspace
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    return workspace


def _ws_bytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


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
    _mult128("K", K)
    q = _codes_out(q, "q", M, K, x)
    s = _scales_out(s, "s", (K // 128, M), x)
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
    kv_scales = _scales_out(kv_scales, "kv_scales", (6,), k)
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
    _dense(kv_scales, "kv_scales", (6,), _F32)
    if k_cache.shape[1] < D:
        raise ValueError("k_cache rows must hold D codes")
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
    _mult128("H", H)
    if y is None and return_y:
        y = _empty((M, H), torch.bfloat16, x)
    if y is not None:
        _rowmajor(y, "y")
        if tuple(y.shape) != (M, H) or y.dtype != torch.bfloat16:
            raise ValueError(f"y must be a bfloat16 tensor of shape {(M, H)}")
    q = _codes_out(q, "q", M, H, x)
    s = _scales_out(s, "s", (H // 128, M), x)
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
    _mult128("I", I)
    if gu.shape[1] < 2 * I:
        raise ValueError(f"gu must hold 2*I = {2 * I} columns")
    if h is None and return_h:
        h = _empty((M, I), torch.bfloat16, gu)
    if h is not None:
        _rowmajor(h, "h")
        if tuple(h.shape) != (M, I) or h.dtype != torch.bfloat16:
            raise ValueError(f"h must be a bfloat16 tensor of shape {(M, I)}")
    q = _codes_out(q, "q", M, I, gu)
    s = _scales_out(s, "s", (I // 128, M), gu)
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
    _mult128("K", K)
    if src_s is None:
        if src.dtype != torch.bfloat16:
            raise TypeError("src must be bfloat16 when src_s is None")
        dt = JET_BF16
    else:
        src = _codes(src)
        _dense(src_s, "src_s", (K // 128, M), _F32)
        dt = JET_E4M3
    Mp = -(-M // 128) * 128
    qT = _codes_out(qT, "qT", K, Mp, src, min_ld=Mp)
    sT = _scales_out(sT, "sT", (Mp // 128, K), src)
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
    _mult128("K", K)
    Mp = -(-M // 128) * 128
    q = _codes_out(q, "q", M, K, x)
    s = _scales_out(s, "s", (K // 128, M), x)
    qT = _codes_out(qT, "qT", K, Mp, x, min_ld=Mp)
    sT = _scales_out(sT, "sT", (Mp // 128, K), x)
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
    _mult128("N", N)
    _mult128("K", K)
    # the weight codes are dense (the entry point takes no leading dimension for them)
    q = _dense(_codes(q) if q is not None else _empty((N, K), torch.uint8, w), "q", (N, K), _U8)
    s = _scales_out(s, "s", (N // 128, K // 128), w)
    if transposed and qT is None:
        qT = _empty((K, N), torch.uint8, w)
    if qT is not None:
        qT = _dense(_codes(qT), "qT", (K, N), _U8)
    _check(name, getattr(_lib, name)(
        _ptr(w), N, K, w.stride(0), _ptr(q), _ptr(s), _ptr(qT), _stream(stream)))
    return q, s, qT


def _dtype_code(dt):
    return {torch.bfloat16: JET_BF16, torch.float32: JET_F32}[dt]


_U8, _F32, _OUT = (torch.uint8,), (torch.float32,), (torch.bfloat16, torch.float32)


def _operands(a, b, name_a, name_b):
    """Codes of the two FP8 GEMM operands: 2-D, dense, sizes multiples of 128
    where the layout needs it.  Returns them as uint8 views."""
    a, b = _codes(a), _codes(b)
    for t, n in ((a, name_a), (b, name_b)):
        if t.dim() != 2:
            raise ValueError(f"{n} must be a 2-D tensor")
    return a, b


def _out(t, name, shape, dtype, like, dtypes=_OUT):
    t = t if t is not None else _empty(shape, dtype, like)
    return _dense(t, name, shape, dtypes)


def _fused_out(fuse_quant, y, yq, ys, M, N, like):
    if not fuse_quant:
        if yq is not None or ys is not None:
            raise ValueError("yq and ys are outputs of the fused quantization (fuse_quant=True)")
        return None, None
    if y.dtype != torch.bfloat16:
        raise TypeError("the fused 1x128 output quantizes a bfloat16 y")
    yq = _dense(_codes(yq) if yq is not None else _empty((M, N), torch.uint8, like), "yq", (M, N), _U8)
    ys = _out(ys, "ys", (N // 128, M), torch.float32, like, _F32)
    return yq, ys


def _fwd_args(xq, xs, wq, ws, y, out_dtype, fuse_quant, yq, ys):
    xq, wq = _operands(xq, wq, "xq", "wq")
    M, K = xq.shape
    N = wq.shape[0]
    _mult128("K", K)
    _mult128("N", N)
    _dense(xq, "xq", (M, K), _U8)
    _dense(wq, "wq", (N, K), _U8)
    _dense(xs, "xs", (K // 128, M), _F32)
    _dense(ws, "ws", (N // 128, K // 128), _F32)
    y = _out(y, "y", (M, N), out_dtype, xq)
    yq, ys = _fused_out(fuse_quant, y, yq, ys, M, N, xq)
    return xq, wq, M, N, K, y, yq, ys


def _dgrad_args(dyq, dys, wqT, ws, dx, out_dtype):
    dyq, wqT = _operands(dyq, wqT, "dyq", "wqT")
    M, N = dyq.shape
    K = wqT.shape[0]
    _mult128("K", K)
    _mult128("N", N)
    _dense(dyq, "dyq", (M, N), _U8)
    _dense(wqT, "wqT", (K, N), _U8)
    _dense(dys, "dys", (N // 128, M), _F32)
    _dense(ws, "ws", (N // 128, K // 128), _F32)
    dx = _out(dx, "dx", (M, K), out_dtype, dyq)
    return dyq, wqT, M, N, K, dx


def _wgrad_args(dyqT, dysT, xqT, xsT, M, dw, out_dtype, accumulate):
    dyqT, xqT = _operands(dyqT, xqT, "dyqT", "xqT")
    M = int(M)
    if M < 0:
        raise ValueError("M must be >= 0")
    N, K = dyqT.shape[0], xqT.shape[0]
    _mult128("K", K)
    _mult128("N", N)
    Mp = -(-M // 128) * 128
    # the transposed operands hold exactly ceil(M/128)*128 token columns (their row stride)
    _dense(dyqT, "dyqT", (N, Mp), _U8)
    _dense(xqT, "xqT", (K, Mp), _U8)
    _dense(dysT, "dysT", (Mp // 128, N), _F32)
    _dense(xsT, "xsT", (Mp // 128, K), _F32)
    dw = _out(dw, "dw", (N, K), out_dtype, dyqT)
    if accumulate and dw.dtype != torch.float32:
        raise TypeError("accumulate needs a float32 dw")
    return dyqT, xqT, M, N, K, dw


def jet_fp8_linear_fwd(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                       yq=None, ys=None, workspace=None, stream=None):
    """Y = deq(xq) . deq(wq)^T.  Returns y, or (y, yq, ys) with fuse_quant."""
    xq, wq, M, N, K, y, yq, ys = _fwd_args(xq, xs, wq, ws, y, out_dtype, fuse_quant, yq, ys)
    workspace = _workspace(workspace, jet_workspace_bytes(JET_OP_FWD, M, N, K), xq, stream)
    _check("jet_fp8_linear_fwd", _lib.jet_fp8_linear_fwd(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype),
        _ptr(yq), _ptr(ys), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_fwd_batch_invariant(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                                       yq=None, ys=None, stream=None):
    """As jet_fp8_linear_fwd, with each output row bit-identical at every M
    (no workspace)."""
    xq, wq, M, N, K, y, yq, ys = _fwd_args(xq, xs, wq, ws, y, out_dtype, fuse_quant, yq, ys)
    _check("jet_fp8_linear_fwd_batch_invariant", _lib.jet_fp8_linear_fwd_batch_invariant(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype), _ptr(yq), _ptr(ys),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_fwd_noalloc(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                               yq=None, ys=None, stream=None):
    """As jet_fp8_linear_fwd, with the split-K partial sums in the library's
    static device scratch (the C call allocates nothing; pass y, and yq and
    ys when fusing, to allocate nothing here either).  Calls that overlap on
    one GPU race on the scratch."""
    xq, wq, M, N, K, y, yq, ys = _fwd_args(xq, xs, wq, ws, y, out_dtype, fuse_quant, yq, ys)
    _check("jet_fp8_linear_fwd_noalloc", _lib.jet_fp8_linear_fwd_noalloc(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype), _ptr(yq), _ptr(ys),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_dgrad(dyq, dys, wqT, ws, dx=None, out_dtype=torch.bfloat16, workspace=None,
                         stream=None):
    """dX = deq(dyq) . deq(W); wqT is the transposed weight codes [K, N]."""
    dyq, wqT, M, N, K, dx = _dgrad_args(dyq, dys, wqT, ws, dx, out_dtype)
    workspace = _workspace(workspace, jet_workspace_bytes(JET_OP_DGRAD, M, N, K), dyq, stream)
    _check("jet_fp8_linear_dgrad", _lib.jet_fp8_linear_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), M, N, K, _ptr(dx), _dtype_code(dx.dtype),
        _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return dx


def jet_fp8_linear_wgrad(dyqT, dysT, xqT, xsT, M, dw=None, out_dtype=torch.float32,
                         accumulate=False, workspace=None, stream=None):
    """dW (+)= deq(dyqT) . deq(xqT)^T over the M tokens (operands [N, Mp], [K, Mp],
    Mp = ceil(M/128)*128)."""
    dyqT, xqT, M, N, K, dw = _wgrad_args(dyqT, dysT, xqT, xsT, M, dw, out_dtype, accumulate)
    workspace = _workspace(workspace, jet_workspace_bytes(JET_OP_WGRAD, M, N, K), dyqT, stream)
    _check("jet_fp8_linear_wgrad", _lib.jet_fp8_linear_wgrad(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), M, N, K, _ptr(dw), _dtype_code(dw.dtype),
        1 if accumulate else 0, _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return dw


def jet_fp8_linear_fwd_pow2(xq, xs, wq, ws, y=None, out_dtype=torch.bfloat16, fuse_quant=False,
                            yq=None, ys=None, stream=None):
    """Forward on power-of-two-scaled operands (scales applied by the MFMA).
    Returns y, or (y, yq, ys) with the power-of-two 1x128 quantization of Y."""
    xq, wq, M, N, K, y, yq, ys = _fwd_args(xq, xs, wq, ws, y, out_dtype, fuse_quant, yq, ys)
    _check("jet_fp8_linear_fwd_pow2", _lib.jet_fp8_linear_fwd_pow2(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _dtype_code(y.dtype), _ptr(yq), _ptr(ys),
        _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_linear_dgrad_pow2(dyq, dys, wqT, ws, dx=None, out_dtype=torch.bfloat16, stream=None):
    """DGrad on power-of-two-scaled operands; wqT the transposed weight codes [K, N]."""
    dyq, wqT, M, N, K, dx = _dgrad_args(dyq, dys, wqT, ws, dx, out_dtype)
    _check("jet_fp8_linear_dgrad_pow2", _lib.jet_fp8_linear_dgrad_pow2(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), M, N, K, _ptr(dx), _dtype_code(dx.dtype), _stream(stream)))
    return dx


def jet_fp8_linear_wgrad_pow2(dyqT, dysT, xqT, xsT, M, dw=None, out_dtype=torch.float32, accumulate=False,
                              stream=None):
    """WGrad on power-of-two-scaled 128x1 operands ([N, Mp], [K, Mp])."""
    dyqT, xqT, M, N, K, dw = _wgrad_args(dyqT, dysT, xqT, xsT, M, dw, out_dtype, accumulate)
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
    _mult128("K", K)
    if src_s is None:
        if src.dtype != torch.bfloat16:
            raise TypeError("src must be bfloat16 when src_s is None")
        dt = JET_BF16
    else:
        src = _codes(src)
        _dense(src_s, "src_s", (K // 128, M), _F32)
        dt = JET_E4M3
    P = grouped_columns(M, E)
    qT = _codes_out(qT, "qT", K, P, src, min_ld=P)
    if K > 1 and qT.stride(0) % 128:
        raise ValueError("qT's row stride must be a multiple of 128")
    ld = qT.stride(0) if K > 1 else qT.shape[1]
    sT = _scales_out(sT, "sT", (ld // 128, K), src)
    _check(name, getattr(_lib, name)(
        _ptr(src), dt, _ptr(src_s), M, K, src.stride(0), _ptr(seg_off), E, _ptr(qT), qT.stride(0),
        _ptr(sT), _stream(stream)))
    return qT, sT


def _grouped_fwd_args(xq, xs, wq, ws, seg_off, y, out_dtype, fuse_quant, yq, ys):
    seg_off, E = _seg(seg_off)
    xq, wq = _codes(xq), _codes(wq)
    if xq.dim() != 2 or wq.dim() != 3:
        raise ValueError("xq must be 2-D [M, K] and wq 3-D [E, N, K]")
    M, K = xq.shape
    N = wq.shape[1]
    _mult128("K", K)
    _mult128("N", N)
    _dense(xq, "xq", (M, K), _U8)
    _dense(wq, "wq", (E, N, K), _U8)
    _dense(xs, "xs", (K // 128, M), _F32)
    _dense(ws, "ws", (E, N // 128, K // 128), _F32)
    y = _out(y, "y", (M, N), out_dtype, xq)
    yq, ys = _fused_out(fuse_quant, y, yq, ys, M, N, xq)
    return seg_off, E, xq, wq, M, N, K, y, yq, ys


def _grouped_dgrad_args(dyq, dys, wqT, ws, seg_off, dx, out_dtype):
    seg_off, E = _seg(seg_off)
    dyq, wqT = _operands(dyq, wqT, "dyq", "wqT")
    M, N = dyq.shape
    K = wqT.shape[0]
    _mult128("K", K)
    _mult128("N", N)
    _dense(dyq, "dyq", (M, N), _U8)
    _dense(wqT, "wqT", (K, E * N), _U8)
    _dense(dys, "dys", (N // 128, M), _F32)
    _dense(ws, "ws", (E, N // 128, K // 128), _F32)
    dx = _out(dx, "dx", (M, K), out_dtype, dyq)
    return seg_off, E, dyq, wqT, M, N, K, dx


def _grouped_wgrad_args(dyqT, dysT, xqT, xsT, seg_off, M, dw, out_dtype, accumulate):
    seg_off, E = _seg(seg_off)
    dyqT, xqT = _operands(dyqT, xqT, "dyqT", "xqT")
    M = int(M)
    if M < 0:
        raise ValueError("M must be >= 0")
    N, K = dyqT.shape[0], xqT.shape[0]
    _mult128("K", K)
    _mult128("N", N)
    _rowmajor(dyqT, "dyqT")
    _rowmajor(xqT, "xqT")
    ldT = dyqT.stride(0)
    if xqT.stride(0) != ldT:
        raise ValueError("dyqT and xqT need the same row stride")
    if ldT % 128 or ldT < grouped_columns(M, E) or dyqT.shape[1] > ldT or xqT.shape[1] > ldT:
        raise ValueError(f"the grouped transposed operands need a row stride that is a multiple of 128 "
                         f"and >= {grouped_columns(M, E)} (got {ldT})")
    _dense(dysT, "dysT", (ldT // 128, N), _F32)
    _dense(xsT, "xsT", (ldT // 128, K), _F32)
    dw = _out(dw, "dw", (E, N, K), out_dtype, dyqT)
    if accumulate and dw.dtype != torch.float32:
        raise TypeError("accumulate needs a float32 dw")
    return seg_off, E, dyqT, xqT, ldT, M, N, K, dw


def jet_fp8_grouped_fwd(xq, xs, wq, ws, seg_off, y=None, out_dtype=torch.bfloat16,
                        fuse_quant=False, yq=None, ys=None, workspace=None, stream=None):
    """Y rows of expert e = deq(xq_e) . deq(wq[e])^T; wq [E, N, K], ws [E, N/128, K/128]."""
    seg_off, E, xq, wq, M, N, K, y, yq, ys = _grouped_fwd_args(xq, xs, wq, ws, seg_off, y, out_dtype,
                                                               fuse_quant, yq, ys)
    # the grouped GEMMs need no workspace (a caller's buffer is passed through)
    _check("jet_fp8_grouped_fwd", _lib.jet_fp8_grouped_fwd(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(y),
        _dtype_code(y.dtype), _ptr(yq), _ptr(ys), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_grouped_dgrad(dyq, dys, wqT, ws, seg_off, dx=None, out_dtype=torch.bfloat16,
                          workspace=None, stream=None):
    """dX rows of expert e = deq(dyq_e) . deq(W_e); wqT [K, E*N] (stacked transposed codes)."""
    seg_off, E, dyq, wqT, M, N, K, dx = _grouped_dgrad_args(dyq, dys, wqT, ws, seg_off, dx, out_dtype)
    _check("jet_fp8_grouped_dgrad", _lib.jet_fp8_grouped_dgrad(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(dx),
        _dtype_code(dx.dtype), _ptr(workspace), _ws_bytes(workspace), _stream(stream)))
    return dx


def jet_fp8_grouped_wgrad(dyqT, dysT, xqT, xsT, seg_off, M, dw=None, out_dtype=torch.float32,
                          accumulate=False, workspace=None, stream=None):
    """dW_e (+)= deq(dyqT_e) . deq(xqT_e)^T; operands in the padded grouped layout [N, P], [K, P]."""
    seg_off, E, dyqT, xqT, ldT, M, N, K, dw = _grouped_wgrad_args(dyqT, dysT, xqT, xsT, seg_off, M, dw,
                                                                  out_dtype, accumulate)
    _check("jet_fp8_grouped_wgrad", _lib.jet_fp8_grouped_wgrad(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), ldT, _ptr(seg_off), E, M, N, K,
        _ptr(dw), _dtype_code(dw.dtype), 1 if accumulate else 0, _ptr(workspace), _ws_bytes(workspace),
        _stream(stream)))
    return dw


def jet_fp8_grouped_fwd_pow2(xq, xs, wq, ws, seg_off, y=None, out_dtype=torch.bfloat16,
                             fuse_quant=False, yq=None, ys=None, stream=None):
    """jet_fp8_grouped_fwd on power-of-two-scaled operands (scales applied by the MFMA)."""
    seg_off, E, xq, wq, M, N, K, y, yq, ys = _grouped_fwd_args(xq, xs, wq, ws, seg_off, y, out_dtype,
                                                               fuse_quant, yq, ys)
    _check("jet_fp8_grouped_fwd_pow2", _lib.jet_fp8_grouped_fwd_pow2(
        _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(y),
        _dtype_code(y.dtype), _ptr(yq), _ptr(ys), _stream(stream)))
    return (y, yq, ys) if fuse_quant else y


def jet_fp8_grouped_dgrad_pow2(dyq, dys, wqT, ws, seg_off, dx=None, out_dtype=torch.bfloat16, stream=None):
    """jet_fp8_grouped_dgrad on power-of-two-scaled operands."""
    seg_off, E, dyq, wqT, M, N, K, dx = _grouped_dgrad_args(dyq, dys, wqT, ws, seg_off, dx, out_dtype)
    _check("jet_fp8_grouped_dgrad_pow2", _lib.jet_fp8_grouped_dgrad_pow2(
        _ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), _ptr(seg_off), E, M, N, K, _ptr(dx),
        _dtype_code(dx.dtype), _stream(stream)))
    return dx


def jet_fp8_grouped_wgrad_pow2(dyqT, dysT, xqT, xsT, seg_off, M, dw=None, out_dtype=torch.float32,
                               accumulate=False, stream=None):
    """jet_fp8_grouped_wgrad on power-of-two-scaled operands."""
    seg_off, E, dyqT, xqT, ldT, M, N, K, dw = _grouped_wgrad_args(dyqT, dysT, xqT, xsT, seg_off, M, dw,
                                                                  out_dtype, accumulate)
    _check("jet_fp8_grouped_wgrad_pow2", _lib.jet_fp8_grouped_wgrad_pow2(
        _ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), ldT, _ptr(seg_off), E, M, N, K,
        _ptr(dw), _dtype_code(dw.dtype), 1 if accumulate else 0, _stream(stream)))
    return dw
