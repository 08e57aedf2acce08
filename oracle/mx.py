"""MXFP8 preparation of Q, K, V -- TEST INFRASTRUCTURE ONLY.

The page "Efficient MoE training for biological foundation models" (the
section on memory and quantisation costs) describes MXFP8 as 8-bit values
with one scale for every block of 32 values.  Readings where it is silent:
  * a block is 32 consecutive channels of one token row (the contraction
    direction of Q K^T);
  * the scale is a power of two 2^e stored as an 8-bit biased exponent
    (byte = e + 127, the E8M0 layout the gfx950 block-scaled matrix
    instructions read);
  * e = ceil(log2(amax / 448)), clamped to [-127, 127], amax being the
    block's largest magnitude (amax = 0 gives e = -127 and zero codes): the
    smallest power of two that maps the block's largest value into the e4m3
    range without saturating -- the power-of-two counterpart of the per-tile
    rule s = amax / 448 of the fp8 path;
  * elements are e4m3 codes of x / 2^e (nearest-even; the division by a power
    of two is exact);
  * Q and K are first rotated by the same random orthogonal R as in the fp8
    path (incoherent processing); V is not rotated.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e4m3_encode
from .fp8 import rotate

MX_BLOCK = 32
E8M0_BIAS = 127


def mx_exponent(amax) -> np.ndarray:
    """e = ceil(log2(amax / 448)) clamped to [-127, 127]; -127 where amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    r = a / 448.0
    m, E = np.frexp(np.where(r > 0, r, 1.0))        # r = m * 2^E, m in [0.5, 1)
    e = np.where(m == 0.5, E - 1, E)                 # exact powers of two: log2 r = E - 1
    e = np.where(r > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize_mx(x) -> tuple[np.ndarray, np.ndarray]:
    """e4m3 codes (uint8, shape of x) and E8M0 scale bytes (uint8 ``[..., d/32]``)
    of a float32 array whose last axis (channels) is a multiple of 32."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    e = mx_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_encode(blocks / np.ldexp(1.0, e)[..., None])
    return codes.reshape(x.shape).astype(np.uint8), (e + E8M0_BIAS).astype(np.uint8)


def dequantize_mx(codes, scales) -> np.ndarray:
    """float64 values: decode(code) * 2^(scale byte - 127) of the code's block."""
    vals = e4m3_decode(codes)
    e = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    return vals * np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=-1)


def mxfp8_prepare(q, k, v, R):
    """((q8, q_scales), (k8, k_scales), (v8, v_scales)) for ``[B,H,N,d]`` float32 inputs."""
    return quantize_mx(rotate(q, R)), quantize_mx(rotate(k, R)), quantize_mx(v)
