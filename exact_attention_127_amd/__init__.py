"""Python binding of the fused exact-attention library (``libattn127.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``.  torch supplies the
device memory and the current stream; there is no CPU or framework fallback,
and a missing library raises ``AttnLibraryMissing``.

The functions keep the C names:

    attn_fwd(q, k, v, o=None, lse=None, scale=None, causal=False)
    attn_fwd_launcher(q, k, v, o, lse, ...)    -> launch(): attn_fwd again, no checks
    attn_fwd_simple(...)                       same contract, plain kernel
    attn_fp8_prepare(q, k, v, R)               -> (q8, k8, v8, sq, sk, sv)
    attn_fwd_fp8(q8, k8, v8, sq, sk, sv, ...)  -> (o, lse)
    attn_mxfp8_prepare(q, k, v, R)             -> (q8, k8, v8, sq, sk, sv)  E8M0 per 32 channels
    attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, ...) -> (o, lse)
    attn_bwd(q, k, v, o, dout, lse, ...)       -> (dq, dk, dv)
    attn_bwd_static(q, k, v, o, dout, lse, ...) -> (dq, dk, dv)  no scratch argument
    w4a16_gemm(x, qweight, scales, zeros)      -> y
    w4a16_gemm_launcher(x, qweight, scales, zeros, y) -> launch(): w4a16_gemm again, no checks
    w4a16_dequantize(qweight, scales, zeros)   -> w
    attn_strerror(status)

Every wrapper checks the shape, dtype, contiguity and device of each tensor it
is given (outputs and scratch buffers included) and raises ValueError before
anything reaches the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library then shares

__all__ = ["attn_fwd", "attn_fwd_launcher", "attn_fwd_simple", "attn_fp8_prepare", "attn_fwd_fp8",
           "attn_mxfp8_prepare", "attn_fwd_mxfp8", "attn_bwd", "attn_bwd_static", "MX_BLOCK",
           "STATIC_SCRATCH_FLOATS",
           "attn_strerror", "AttnError", "AttnLibraryMissing", "lib", "LIB_PATH",
           "EXPORTED_SYMBOLS", "ATTN_F32", "ATTN_BF16", "FP8_TILE", "w4a16_gemm", "w4a16_gemm_launcher",
           "w4a16_dequantize", "W4A16_GROUP"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn127.so")
EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_simple", "attn_fp8_prepare", "attn_fwd_fp8",
                    "attn_mxfp8_prepare", "attn_fwd_mxfp8", "attn_bwd", "attn_bwd_static",
                    "w4a16_gemm", "w4a16_dequantize", "attn_strerror")
ATTN_F32, ATTN_BF16 = 0, 1
FP8_TILE = 128
MX_BLOCK = 32
W4A16_GROUP = 128
_STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_INVALID_ARG", -2: "ATTN_ERR_UNSUPPORTED",
           -3: "ATTN_ERR_HIP", -4: "ATTN_ERR_TOO_LARGE"}
STATIC_SCRATCH_FLOATS = 4194304


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
        L.attn_bwd_static.argtypes = [_P] * 9 + [_I, _I, _I, _I, _F, _I, _I, _P]
        L.attn_bwd_static.restype = _I
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


def _scale_arg(scale):
    """The scale passed to the C ABI: None selects the library's default,
    1/sqrt(d), which the C side applies when it receives 0."""
    return 0.0 if scale is None else float(scale)


def _want(t, name, shape, dtype):
    """A tensor argument must have exactly this shape and dtype and be
    contiguous (the C ABI sees only a pointer, so it cannot check sizes)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_gpu(**tensors):
    """Every tensor argument must live on one GPU: a host pointer handed to a
    kernel would fault the device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, not on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")


def _fwd(name, q, k, v, o, lse, scale, causal, stream, with_lse):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.dtype == torch.bfloat16:
        dtype = ATTN_BF16
    elif q.dtype == torch.float32:
        dtype = ATTN_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _want(t, nm, q.shape, q.dtype)
    if o is not None:
        _want(o, "o", q.shape, q.dtype)
    if lse is not None:
        _want(lse, "lse", (B, H, N), torch.float32)
    _same_gpu(q=q, k=k, v=v, o=o, lse=lse)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                              _scale_arg(scale), int(bool(causal)), dtype, _stream(stream))
    _check(st, name)
    return o, lse


def attn_fwd(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None, with_lse=True):
    """O (and LSE) of softmax(Q K^T * scale) V on matrix cores (bf16) or in float32."""
    return _fwd("attn_fwd", q, k, v, o, lse, scale, causal, stream, with_lse)


def attn_fwd_launcher(q, k, v, o, lse=None, scale=None, causal=False, stream=None):
    """Checks the arguments of attn_fwd once and returns a callable that
    launches it again on the same buffers and stream.  Each launch then costs
    one C call on the host, for loops whose kernels take less time than the
    per-call checks (short sequences); the buffers must stay alive."""
    _fwd("attn_fwd", q, k, v, o, lse, scale, causal, stream, lse is not None)
    B, H, N, d = q.shape
    dtype = ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_F32
    fn = lib().attn_fwd
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _scale_arg(scale),
            int(bool(causal)), dtype, _stream(stream))

    def launch():
        st = fn(*args)
        if st != 0:
            raise AttnError(st, "attn_fwd")
    return launch


def attn_fwd_simple(q, k, v, o=None, lse=None, scale=None, causal=False, stream=None,
                    with_lse=True):
    """The same operation on the plain float32-arithmetic kernel."""
    return _fwd("attn_fwd_simple", q, k, v, o, lse, scale, causal, stream, with_lse)


def attn_fp8_prepare(q, k, v, R, stream=None):
    """Rotate Q, K by R and quantise Q, K, V to e4m3 with one scale per 128-token tile."""
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _want(t, nm, q.shape, torch.float32)
    _want(R, "R", (d, d), torch.float32)
    _same_gpu(q=q, k=k, v=v, R=R)
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
    if q8.dim() != 4:
        raise ValueError("q8, k8, v8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    for nm, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _want(t, nm, q8.shape, torch.uint8)
    nt = -(-N // FP8_TILE)
    for nm, s_ in (("sq", sq), ("sk", sk), ("sv", sv)):
        _want(s_, nm, (B, H, nt), torch.float32)
    if o is not None:
        _want(o, "o", (B, H, N, d), torch.bfloat16)
    if lse is not None:
        _want(lse, "lse", (B, H, N), torch.float32)
    _same_gpu(q8=q8, k8=k8, v8=v8, sq=sq, sk=sk, sv=sv, o=o, lse=lse)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    st = lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv),
                            _ptr(o), _ptr(lse), B, H, N, d, _scale_arg(scale), int(bool(causal)),
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
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_bwd takes bfloat16 tensors")
    for nm, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, nm, q.shape, torch.bfloat16)
    _want(lse, "lse", (B, H, N), torch.float32)
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _want(t, nm, q.shape, torch.bfloat16)
    if delta is not None:
        _want(delta, "delta", (B, H, N), torch.float32)
    _same_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta),
                        _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale_arg(scale),
                        int(bool(causal)), ATTN_BF16, _stream(stream))
    _check(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_static(q, k, v, o, dout, lse, dq=None, dk=None, dv=None, scale=None, causal=False,
                    stream=None):
    """attn_bwd without the caller's scratch: the row statistic D lives in the
    library's fixed per-GPU array (B*H*N <= STATIC_SCRATCH_FLOATS).  The C
    call allocates nothing; pass dq, dk, dv to keep this wrapper from
    allocating them."""
    if q.dim() != 4:
        raise ValueError("q, k, v, o, dout must be [B, H, N, d]")
    B, H, N, d = q.shape
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_bwd_static takes bfloat16 tensors")
    for nm, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _want(t, nm, q.shape, torch.bfloat16)
    _want(lse, "lse", (B, H, N), torch.float32)
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _want(t, nm, q.shape, torch.bfloat16)
    _same_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    st = lib().attn_bwd_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale_arg(scale),
                               int(bool(causal)), ATTN_BF16, _stream(stream))
    _check(st, "attn_bwd_static")
    return dq, dk, dv


def attn_mxfp8_prepare(q, k, v, R, stream=None):
    """MXFP8 codes and E8M0 scale bytes ([B, H, N, d/32] uint8) of q R, k R and v."""
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _want(t, nm, q.shape, torch.float32)
    _want(R, "R", (d, d), torch.float32)
    _same_gpu(q=q, k=k, v=v, R=R)
    codes = [torch.empty((B, H, N, d), dtype=torch.uint8, device=q.device) for _ in range(3)]
    scales = [torch.empty((B, H, N, d // MX_BLOCK), dtype=torch.uint8, device=q.device) for _ in range(3)]
    st = lib().attn_mxfp8_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(R), *(_ptr(c) for c in codes),
                                  *(_ptr(s) for s in scales), B, H, N, d, _stream(stream))
    _check(st, "attn_mxfp8_prepare")
    return (*codes, *scales)


def attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, o=None, lse=None, scale=None, causal=False,
                   stream=None, with_lse=True):
    """Attention on MXFP8 codes with E8M0 block scales; O is bf16."""
    if q8.dim() != 4:
        raise ValueError("q8, k8, v8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    for nm, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _want(t, nm, q8.shape, torch.uint8)
    for nm, s_ in (("sq", sq), ("sk", sk), ("sv", sv)):
        _want(s_, nm, (B, H, N, d // MX_BLOCK), torch.uint8)
    if o is not None:
        _want(o, "o", (B, H, N, d), torch.bfloat16)
    if lse is not None:
        _want(lse, "lse", (B, H, N), torch.float32)
    _same_gpu(q8=q8, k8=k8, v8=v8, sq=sq, sk=sk, sv=sv, o=o, lse=lse)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    st = lib().attn_fwd_mxfp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv),
                              _ptr(o), _ptr(lse), B, H, N, d, _scale_arg(scale), int(bool(causal)),
                              _stream(stream))
    _check(st, "attn_fwd_mxfp8")
    return o, lse


def _w4_check(qweight, scales, zeros, K, group, device):
    if qweight.dim() != 2 or qweight.element_size() != 4 or qweight.dtype.is_floating_point:
        raise ValueError("qweight must be a 2-D tensor of 32-bit words [N, K/8]")
    N = qweight.shape[0]
    if tuple(qweight.shape) != (N, K // 8):
        raise ValueError(f"qweight must be [N, K/8] = [{N}, {K // 8}]")
    if not qweight.is_contiguous():
        raise ValueError("qweight must be contiguous")
    _want(scales, "scales", (N, K // group), torch.float16)
    _want(zeros, "zeros", (N, K // group), torch.uint8)
    for nm, t in (("qweight", qweight), ("scales", scales), ("zeros", zeros)):
        if t.device != device:
            raise ValueError(f"{nm} is on {t.device}, other arguments on {device}")
    return N


def w4a16_gemm(x, qweight, scales, zeros, y=None, group=W4A16_GROUP, stream=None):
    """Y = X W^T, fp16 [M, N], with W dequantised from packed 4-bit words in
    registers: w = fp16(s * (q - z)) per group of ``group`` k (M <= 16)."""
    if x.dim() != 2 or x.dtype != torch.float16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float16 [M, K] tensor")
    M, K = x.shape
    N = _w4_check(qweight, scales, zeros, K, group, x.device)
    if y is not None:
        _want(y, "y", (M, N), torch.float16)
    _same_gpu(x=x, qweight=qweight, scales=scales, zeros=zeros, y=y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    st = lib().w4a16_gemm(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), M, N, K,
                          int(group), _stream(stream))
    _check(st, "w4a16_gemm")
    return y


def w4a16_gemm_launcher(x, qweight, scales, zeros, y, group=W4A16_GROUP, stream=None):
    """Checks the arguments of w4a16_gemm once and returns a callable that
    launches it again on the same buffers and stream (one C call each)."""
    w4a16_gemm(x, qweight, scales, zeros, y=y, group=group, stream=stream)
    M, K = x.shape
    N = qweight.shape[0]
    fn = lib().w4a16_gemm
    args = (_ptr(x), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(y), M, N, K, int(group), _stream(stream))

    def launch():
        st = fn(*args)
        if st != 0:
            raise AttnError(st, "w4a16_gemm")
    return launch


def w4a16_dequantize(qweight, scales, zeros, K, w=None, group=W4A16_GROUP, stream=None):
    """The fp16 weights [N, K] that w4a16_gemm feeds to the matrix cores."""
    N = _w4_check(qweight, scales, zeros, K, group, qweight.device)
    if w is not None:
        _want(w, "w", (N, K), torch.float16)
    _same_gpu(qweight=qweight, scales=scales, zeros=zeros, w=w)
    if w is None:
        w = torch.empty((N, K), dtype=torch.float16, device=qweight.device)
    st = lib().w4a16_dequantize(_ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(w), N, K,
                                int(group), _stream(stream))
    _check(st, "w4a16_dequantize")
    return w
