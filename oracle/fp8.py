"""fp8 (e4m3) preparation of Q, K, V -- TEST INFRASTRUCTURE ONLY.

Follows the FP8 bullet of "FlashAttention scaling, multi-GPU training and
weight quantization", section 1, in its order:
  1. incoherent processing: Q' = Q R and K' = K R with one random orthogonal
     d x d matrix R (drawn by the input generator and passed in); V is not
     rotated.  Since R R^T = I, Q' K'^T = Q K^T, so the attention result is
     unchanged by this step.
  2. block quantisation: each tile of QUANT_TILE consecutive tokens x all d
     channels (d <= 128) of one (batch, head) gets its own float32 scale
     s = amax / 448 (amax = 0 gives s = 1), and each value is stored as the
     e4m3 code of x / s.
Readings where the page is silent: the rotated values are held in float32
(computed here in float64 and rounded once); s and x / s are IEEE float32
divisions; e4m3 rounding is to nearest-even with saturation.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode

QUANT_TILE = 128


def quantize_tiles(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-tile scale and e4m3 codes of a float32 ``[B,H,N,d]`` tensor."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nt = -(-N // QUANT_TILE)
    scales = np.empty((B, H, nt), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    for t in range(nt):
        blk = x[:, :, t * QUANT_TILE:(t + 1) * QUANT_TILE, :]
        amax = np.abs(blk).max(axis=(2, 3))
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, :, t] = s
        codes[:, :, t * QUANT_TILE:(t + 1) * QUANT_TILE, :] = e4m3_encode(
            (blk / s[:, :, None, None]).astype(np.float32))
    return codes, scales


def rotate(x, R) -> np.ndarray:
    """x R in float64, rounded once to float32."""
    return np.matmul(np.asarray(x, dtype=np.float64),
                     np.asarray(R, dtype=np.float64)).astype(np.float32)


def fp8_prepare(q, k, v, R):
    """Returns ((q8, sq), (k8, sk), (v8, sv)): e4m3 codes and per-tile scales."""
    return (quantize_tiles(rotate(q, R)), quantize_tiles(rotate(k, R)),
            quantize_tiles(v))


def fp8_dequantize(codes, scales) -> np.ndarray:
    """float64 values the codes stand for: decode(code) * s of the code's tile."""
    vals = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), QUANT_TILE, axis=2)
    return vals * s[:, :, :vals.shape[2], None]
