"""Python binding of the fused exact-attention library (``libattn127.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``.  torch supplies the
device memory and the current stream; there is no CPU or framework fallback,
and a missing library raises ``AttnLibraryMissing``.

The functions keep the C names:

    attn_fwd(q, k, v, o=None, lse=None, scale=None, causal=False)
    attn_fwd_simple(...)                       same contract, plain kernel
    attn_fp8_prepare(q, k, v, R)               -> (q8, k8, v8, sq, sk, sv)
    attn_fwd_fp8(q8, k8, v8, sq, sk, sv, ...)  -> (o, lse)
    attn_mxfp8_prepare(q, k, v, R)             -> (q8, k8, v8, sq, sk, sv)  E8M0 per 32 channels
    attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, ...) -> (o, lse)
    attn_bwd(q, k, v, o, dout, lse, ...)       -> (dq, dk, dv)
    attn_strerror(status)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loads the HIP runtime that the library then shares

__all__ = ["attn_fwd", "attn_fwd_simple", "attn_fp8_prepare", "attn_fwd_fp8",
           "attn_mxfp8_prepare", "attn_fwd_mxfp8", "attn_bwd", "MX_BLOCK",
           "attn_strerror", "AttnError", "AttnLibraryMissing", "lib", "LIB_PATH",
           "EXPORTED_SYMBOLS", "ATTN_F32", "ATTN_BF16", "FP8_TILE", "w4a16_gemm",
           "w4a16_dequantize", "W4A16_GROUP"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn127.so")
EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_simple", "attn_fp8_prepare", "attn_fwd_fp8",
                    "attn_mxfp8_prepare", "attn_fwd_mxfp8", "attn_bwd", "w4a16_gemm",
                    "w4a16_dequantize", "attn_strerror")
ATTN_F32, ATTN_BF16 = 0, 1
FP8_TILE = 128
MX_BLOCK = 32
W4A16_GROUP = 128
_STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_INVALID_ARG", -2: "ATTN_ERR_UNSUPPORTED",
           -3: "ATTN_ERR_HIP"}


class AttnLibraryMissing(RuntimeError):
    pass


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({attn_strerror(status)})")


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise AttnLibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -m exact_attention_127_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        fwd_args = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]
        for name in ("attn_fwd", "attn_fwd_simple"):
            fn = getattr(L, name)
            fn.argtypes = fwd_args
            fn.restype = _I
        L.attn_fp8_prepare.argtypes = [_P] * 10 + [_I, _I, _I, _I, _P]
        L.attn_fp8_prepare.restype = _I
        L.attn_fwd_fp8.argtypes = [_P] * 8 + [_I, _I, _I, _I, _F, _I, _P]
        L.attn_fwd_fp8.restype = _I
        L.attn_mxfp8_prepare.argtypes = [_P] * 10 + [_I, _I, _I, _I, _P]
        L.attn_mxfp8_prepare.restype = _I
        L.attn_fwd_mxfp8.argtypes = [_P] * 8 + [_I, _I, _I, _I, _F, _I, _P]
        L.attn_fwd_mxfp8.restype = _I
        L.attn_bwd.argtypes = [_P] * 10 + [_I, _I, _I, _I, _F, _I, _I, _P]
        L.attn_bwd.restype = _I
        L.w4a16_gemm.argtypes = [_P] * 5 + [_I, _I, _I, _I, _P]
        L.w4a16_gemm.restype = _I
        L.w4a16_dequantize.argtypes = [_P] * 4 + [_I, _I, _I, _P]
        L.w4a16_dequantize.restype = _I
        L.attn_strerror.argtypes = [_I]
        L.attn_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise AttnError(status, where)


def _fwd(name, q, k, v, o, lse, scale, causal, stream, with_lse):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t in (q, k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    if q.dtype == torch.bfloat16:
        dtype = ATTN_BF16
    elif q.dtype == torch.float32:
        dtype = ATTN_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                              float(scale), int(bool(causal)), dtype, _stream(stream))
    _check(st, name)
    return o, lse


def attn_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None, with_lse=True):
    """O (and LSE) of softmax(Q K^T * scale) V on matrix cores (bf16) or in float32."""
    return _fwd("attn_fwd", q, k, v, o, lse, scale, causal, stream, with_lse)


def attn_fwd_simple(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None,
                    with_lse=True):
    """The same operation on the plain float32-arithmetic kernel."""
    return _fwd("attn_fwd_simple", q, k, v, o, lse, scale, causal, stream, with_lse)


def attn_fp8_prepare(q, k, v, R, stream=None):
    """Rotate Q, K by R and quantise Q, K, V to e4m3 with one scale per 128-token tile."""
    B, H, N, d = q.shape
    for t in (q, k, v):
        if t.shape != q.shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous float32 [B, H, N, d]")
    if R.shape != (d, d) or R.dtype != torch.float32 or not R.is_contiguous():
        raise ValueError("R must be contiguous float32 [d, d]")
    nt = -(-N // FP8_TILE)
    codes = [torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device) for _ in range(3)]
    scales = [torch.empty((B, H, nt), dtype=torch.float32, device=q.device) for _ in range(3)]
    st = lib().attn_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(R), *map(_ptr, codes),
                                *map(_ptr, scales), B, H, N, d, _stream(stream))
    _check(st, "attn_fp8_prepare")
    return (*codes, *scales)


def attn_fwd_fp8(q8, k8, v8, sq, sk, sv, o=None, lse=None, scale=None, causal=False,
                 stream=None, with_lse=True):
    """Attention on e4m3 codes with per-tile scales; O is bf16."""
    B, H, N, d = q8.shape
    for t in (q8, k8, v8):
        if t.shape != q8.shape or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("q8, k8, v8 must be contiguous uint8 [B, H, N, d]")
    nt = -(-N // FP8_TILE)
    for s in (sq, sk, sv):
        if s.shape != (B, H, nt) or s.dtype != torch.float32 or not s.is_contiguous():
            raise ValueError("scales must be contiguous float32 [B, H, ceil(N/128)]")
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv),
                            _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                            _stream(stream))
    _check(st, "attn_fwd_fp8")
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, dq=None, dk=None, dv=None, delta=None, scale=None,
             causal=False, stream=None):
    """dQ, dK, dV of attn_fwd (bf16), from the forward's O and LSE and the
    output gradient dout.  ``delta`` is float32 [B, H, N] scratch (allocated
    here when not given)."""
    if q.dim() != 4:
        raise ValueError("q, k, v, o, dout must be [B, H, N, d]")
    B, H, N, d = q.shape
    for t in (q, k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, dout must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must be contiguous")
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_bwd takes bfloat16 tensors")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous bfloat16 like q")
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                        _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                        int(bool(causal)), ATTN_BF16, _stream(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv


def attn_mxfp8_prepare(q, k, v, R, stream=None):
    """MXFP8 codes and E8M0 scale bytes ([B, H, N, d/32] uint8) of q R, k R and v."""
    B, H, N, d = q.shape
    for t in (q, k, v):
        if t.shape != q.shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous float32 [B, H, N, d]")
    if R.shape != (d, d) or R.dtype != torch.float32 or not R.is_contiguous():
        raise ValueError("R must be contiguous float32 [d, d]")
    codes = [torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device) for _ in range(3)]
    scales = [torch.empty((B, H, N, d // MX_BLOCK), dtype=torch.uint8, device=q.device) for _ in range(3)]
    st = lib().attn_mxfp8_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(R), *(_ptr(c) for c in codes),
                                  *(_ptr(s) for s in scales), B, H, N, d, _stream(stream))
    _check(st, "attn_mxfp8_prepare")
    return (*codes, *scales)


def attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, o=None, lse=None, scale=None, causal=False,
                   stream=None, with_lse=True):
    """Attention on MXFP8 codes with E8M0 block scales; O is bf16."""
    B, H, N, d = q8.shape
    for t in (q8, k8, v8):
        if t.shape != q8.shape or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("q8, k8, v8 must be contiguous uint8 [B, H, N, d]")
    for s_ in (sq, sk, sv):
        if s_.shape != (B, H, N, d // MX_BLOCK) or s_.dtype != torch.uint8 or not s_.is_contiguous():
            raise ValueError("scales must be contiguous uint8 [B, H, N, d/32]")
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().attn_fwd_mxfp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv),
                              _ptr(o), _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                              _stream(stream))
    _check(st, "attn_fwd_mxfp8")
    return o, lse


def _w4_check(qweight, scales, zeros, K, group, device):
    N = qweight.shape[0]
    if qweight.dim() != 2 or qweight.element_size() != 4 or qweight.dtype.is_floating_point:
        raise ValueError("qweight must be a 2-D tensor of 32-bit words [N, K/8]")
    if tuple(qweight.shape) != (N, K // 8):
        raise ValueError(f"qweight must be [N, K/8] = [{N}, {K // 8}]")
    if scales.dtype != torch.float16 or tuple(scales.shape) != (N, K // group):
        raise ValueError(f"scales must be float16 [N, K/{group}]")
    if zeros.dtype != torch.uint8 or tuple(zeros.shape) != (N, K // group):
        raise ValueError(f"zeros must be uint8 [N, K/{group}]")
    for t in (qweight, scales, zeros):
        if not t.is_contiguous() or t.device != device:
            raise ValueError("qweight, scales, zeros must be contiguous and on the same device")
    return N


def w4a16_gemm(x, qweight, scales, zeros, y=None, group=W4A16_GROUP, stream=None):
    """Y = X W^T, fp16 [M, N], with W dequantised from packed 4-bit words in
    registers: w = fp16(s * (q - z)) per group of ``group`` k (M <= 16)."""
    if x.dim() != 2 or x.dtype != torch.float16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float16 [M, K] tensor")
    M, K = x.shape
    N = _w4_check(qweight, scales, zeros, K, group, x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    st = lib().w4a16_gemm(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), M, N, K,
                          int(group), _stream(stream))
    _check(st, "w4a16_gemm")
    return y


def w4a16_dequantize(qweight, scales, zeros, K, w=None, group=W4A16_GROUP, stream=None):
    """The fp16 weights [N, K] that w4a16_gemm feeds to the matrix cores."""
    N = _w4_check(qweight, scales, zeros, K, group, qweight.device)
    if w is None:
        w = torch.empty((N, K), dtype=torch.float16, device=qweight.device)
    st = lib().w4a16_dequantize(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(w), N, K,
                                int(group), _stream(stream))
    _check(st, "w4a16_dequantize")
    return w
