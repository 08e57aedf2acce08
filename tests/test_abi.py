"""C-ABI checks that need no GPU: the library loads, exports every function
that include/attn.h declares, and rejects bad arguments before any HIP call
(so these calls are safe on a host without a device)."""
import ctypes
import os
import re

import pytest

import exact_attention_127_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?((?:attn|w4a16)_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(A.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = A.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror():
    assert A.attn_strerror(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert len(A.attn_strerror(s)) > 5
    assert A.attn_strerror(12345) == "unknown status"


FAKE = 0x10000          # 16-byte aligned, never dereferenced: checks fail first


def _fwd(fn, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=1, N=8, d=64, scale=0.125,
         causal=0, dtype=1):
    return getattr(A.lib(), fn)(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_simple"])
@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(q=FAKE + 2), dict(o=FAKE + 8), dict(lse=FAKE + 2),
    dict(d=32), dict(d=96), dict(d=0), dict(N=-1), dict(B=-1), dict(H=-2),
    dict(dtype=2), dict(dtype=-1), dict(scale=-1.0),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(N=1 << 30),
])
def test_invalid_arguments_rejected(fn, bad):
    assert _fwd(fn, **bad) == -1


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_simple"])
@pytest.mark.parametrize("empty", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_is_a_noop(fn, empty):
    # zero work: returns before any HIP call, so no device is needed
    assert _fwd(fn, **empty) == 0


def test_fp8_entry_points_validate():
    L = A.lib()
    args = [FAKE] * 10
    assert L.attn_fp8_prepare(*args, 1, 1, 8, 48, None) == -1
    assert L.attn_fp8_prepare(*([None] + args[1:]), 1, 1, 8, 64, None) == -1
    assert L.attn_fp8_prepare(*args, 0, 1, 8, 64, None) == 0
    f = [FAKE] * 7 + [None]
    assert L.attn_fwd_fp8(*f, 1, 1, 8, 128, -0.5, 0, None) == -1
    assert L.attn_fwd_fp8(*f, 1, 1, 8, 100, 0.1, 0, None) == -1
    assert L.attn_fwd_fp8(*f, 1, 0, 8, 128, 0.1, 0, None) == 0


def test_grid_limit_rejected():
    # B*H*ceil(N/64) would not fit a 1-D grid
    assert _fwd("attn_fwd", B=1 << 15, H=1 << 15, N=64 * 4) == -1


def _bwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, delta=FAKE, dq=FAKE, dk=FAKE,
         dv=FAKE, B=1, H=1, N=8, d=128, scale=0.125, causal=0, dtype=1):
    return A.lib().attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, B, H, N, d, scale, causal,
                            dtype, None)


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(do=None), dict(lse=None),
    dict(delta=None), dict(dq=None), dict(dk=None), dict(dv=None),
    dict(do=FAKE + 8), dict(dq=FAKE + 2), dict(lse=FAKE + 2), dict(delta=FAKE + 1),
    dict(d=96), dict(N=-1), dict(dtype=2), dict(scale=-0.5), dict(scale=float("nan")),
])
def test_bwd_invalid_arguments_rejected(bad):
    assert _bwd(**bad) == -1


def test_bwd_float32_is_unsupported_and_empty_is_a_noop():
    assert _bwd(dtype=0) == -2
    for empty in (dict(B=0), dict(H=0), dict(N=0)):
        assert _bwd(**empty) == 0


def test_mxfp8_entry_points_validate():
    L = A.lib()
    args = [FAKE] * 10
    assert L.attn_mxfp8_prepare(*args, 1, 1, 8, 48, None) == -1            # d not 64/128
    assert L.attn_mxfp8_prepare(*([None] + args[1:]), 1, 1, 8, 64, None) == -1
    assert L.attn_mxfp8_prepare(*(args[:7] + [FAKE + 1] + args[8:]), 1, 1, 8, 64, None) == -1  # scale rows: 2-byte aligned at d=64
    assert L.attn_mxfp8_prepare(*(args[:7] + [FAKE + 2] + args[8:]), 1, 1, 8, 128, None) == -1  # 4-byte at d=128
    assert L.attn_mxfp8_prepare(*args, 0, 1, 8, 64, None) == 0
    f = [FAKE] * 7 + [None]
    assert L.attn_fwd_mxfp8(*f, 1, 1, 8, 128, -0.5, 0, None) == -1
    assert L.attn_fwd_mxfp8(*f, 1, 1, 8, 100, 0.1, 0, None) == -1
    assert L.attn_fwd_mxfp8(*(f[:3] + [None] + f[4:]), 1, 1, 8, 128, 0.1, 0, None) == -1
    assert L.attn_fwd_mxfp8(*f, 1, 0, 8, 128, 0.1, 0, None) == 0


def test_w4a16_entry_points_validate():
    L = A.lib()
    g = lambda x=FAKE, q=FAKE, s=FAKE, z=FAKE, y=FAKE, M=1, N=32, K=256, group=128: \
        L.w4a16_gemm(x, q, s, z, y, M, N, K, group, None)
    assert g(M=17) == -1                      # more than 16 tokens
    assert g(M=-1) == -1 and g(N=-1) == -1
    assert g(K=100) == -1                     # not whole words
    assert g(K=136) == -1                     # not whole groups
    assert g(group=64) == -2                  # only groups of 128
    assert g(K=32768 + 128) == -2             # scales of 32 rows must fit 32 KB of LDS
    assert g(x=None) == -1 and g(y=None) == -1 and g(z=None) == -1
    assert g(q=FAKE + 4) == -1                # words: 16-byte aligned
    assert g(x=FAKE + 8) == -1                # activations: 16-byte aligned
    assert g(y=FAKE + 4) == -1                # output: 8-byte aligned
    assert g(s=FAKE + 1) == -1                # fp16 scales: 2-byte aligned
    assert g(M=0) == 0 and g(N=0) == 0 and g(K=0) == 0
    d = lambda q=FAKE, s=FAKE, z=FAKE, w=FAKE, N=32, K=256, group=128: \
        L.w4a16_dequantize(q, s, z, w, N, K, group, None)
    assert d(w=FAKE + 8) == -1 and d(K=120) == -1 and d(group=32) == -2
    assert d(N=0) == 0


# --- the Python binding checks every tensor before any pointer reaches the ABI


def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_host_tensors():
    import torch
    q = _t(1, 2, 8, 64)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd_simple(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd_launcher(q, q, q, q.clone())
    with pytest.raises(ValueError, match="GPU"):
        A.attn_bwd(q, q, q, q, q, _t(1, 2, 8, dtype=torch.float32))
    f = _t(1, 2, 8, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fp8_prepare(f, f, f, _t(64, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        A.attn_mxfp8_prepare(f, f, f, _t(64, 64, dtype=torch.float32))
    c = _t(1, 2, 8, 64, dtype=torch.uint8)
    s = _t(1, 2, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd_fp8(c, c, c, s, s, s)
    e = _t(1, 2, 8, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd_mxfp8(c, c, c, e, e, e)
    x = _t(1, 256, dtype=torch.float16)
    qw = _t(32, 32, dtype=torch.int32)
    sc = _t(32, 2, dtype=torch.float16)
    z = _t(32, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        A.w4a16_gemm(x, qw, sc, z)
    with pytest.raises(ValueError, match="GPU"):
        A.w4a16_gemm_launcher(x, qw, sc, z, _t(1, 32, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        A.w4a16_dequantize(qw, sc, z, 256)


@pytest.mark.parametrize("bad", ["o_shape", "o_dtype", "o_strided", "lse_shape", "lse_dtype",
                                 "k_shape", "v_dtype"])
def test_binding_rejects_mismatched_outputs(bad):
    import torch
    q = _t(1, 2, 8, 64)
    k, v = q.clone(), q.clone()
    o = _t(1, 2, 8, 64)
    lse = _t(1, 2, 8, dtype=torch.float32)
    if bad == "o_shape":
        o = _t(1, 2, 7, 64)
    elif bad == "o_dtype":
        o = _t(1, 2, 8, 64, dtype=torch.float32)
    elif bad == "o_strided":
        o = _t(1, 2, 64, 8).transpose(2, 3)
    elif bad == "lse_shape":
        lse = _t(1, 2, 4, dtype=torch.float32)
    elif bad == "lse_dtype":
        lse = _t(1, 2, 8)
    elif bad == "k_shape":
        k = _t(1, 2, 9, 64)
    elif bad == "v_dtype":
        v = _t(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        A.attn_fwd(q, k, v, o=o, lse=lse)
    with pytest.raises(ValueError):
        A.attn_fwd_launcher(q, k, v, o, lse)


def test_binding_rejects_mismatched_scratch_and_gradients():
    import torch
    q = _t(1, 2, 8, 64)
    lse = _t(1, 2, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="delta"):
        A.attn_bwd(q, q, q, q, q, lse, delta=_t(1, 2, 7, dtype=torch.float32))
    with pytest.raises(ValueError, match="dq"):
        A.attn_bwd(q, q, q, q, q, lse, dq=_t(1, 2, 8, 128))
    with pytest.raises(ValueError, match="lse"):
        A.attn_bwd(q, q, q, q, q, _t(1, 2, 8))
    c = _t(1, 2, 8, 64, dtype=torch.uint8)
    s = _t(1, 2, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="sk"):
        A.attn_fwd_fp8(c, c, c, s, _t(1, 2, 2, dtype=torch.float32), s)
    with pytest.raises(ValueError, match="o"):
        A.attn_fwd_fp8(c, c, c, s, s, s, o=_t(1, 2, 8, 64, dtype=torch.float32))
    x = _t(2, 256, dtype=torch.float16)
    qw = _t(32, 32, dtype=torch.int32)
    sc = _t(32, 2, dtype=torch.float16)
    z = _t(32, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="y"):
        A.w4a16_gemm(x, qw, sc, z, y=_t(1, 32, dtype=torch.float16))
    with pytest.raises(ValueError, match="scales"):
        A.w4a16_gemm(x, qw, _t(32, 3, dtype=torch.float16), z)


def test_bwd_static_validates_on_the_host():
    L = A.lib()
    f = [FAKE] * 9
    call = lambda ptrs=f, B=1, H=1, N=8, d=128, scale=0.125, dtype=1: \
        L.attn_bwd_static(*ptrs, B, H, N, d, scale, 0, dtype, None)
    assert call(N=A.STATIC_SCRATCH_FLOATS + 1) == -4          # beyond the fixed scratch array
    assert call(B=2, H=4, N=A.STATIC_SCRATCH_FLOATS // 8 + 1) == -4
    assert call(ptrs=[None] + f[1:]) == -1 and call(ptrs=f[:5] + [None] + f[6:]) == -1
    assert call(ptrs=f[:6] + [FAKE + 8] + f[7:]) == -1         # dq misaligned
    assert call(d=96) == -1 and call(scale=-1.0) == -1 and call(dtype=0) == -2
    assert call(B=0) == 0 and call(N=0) == 0
    assert "scratch" in A.attn_strerror(-4)
