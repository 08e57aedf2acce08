"""W4A16 decode product -- TEST INFRASTRUCTURE ONLY.

Page "FlashAttention scaling, multi-GPU training and weight quantization",
section 3 (quantisation and on-the-fly dequantisation kernels): decoding one
token at a time is bound by reading the weights, so they are stored as 4-bit
integers, eight to a 32-bit word; the kernel reads the packed words, unpacks
them in registers with shifts and masks, applies the stored scale and zero
point to get FP16 values, and feeds those straight to the matrix units with
the FP16 activations, never writing the expanded weights back to memory.

This module computes what such a kernel computes, written out plainly:
unpack every weight, dequantise the whole matrix, then one matrix product in
float64.  Readings where the page is silent:
  * W is [N][K] (output features x input features, as a linear layer's
    weight); Y = X W^T with X fp16 [M][K] and Y [M][N];
  * packing: word (n, j) of qweight [N][K/8] (uint32) holds the integers of
    weights (n, 8j + i), i = 0..7, value i in bits 4i .. 4i+3;
  * scale and zero point per (output row n, group of G consecutive k):
    scales fp16 [N][K/G], zeros integers 0..15 as uint8 [N][K/G];
  * the FP16 weight fed to the matrix units is fp16(s * (q - z)), rounded
    once (q - z is an exact small integer);
  * products and sums as exact as float64 allows; the device accumulates in
    float32 and rounds Y to fp16, which the tests bound separately.
"""
from __future__ import annotations

import numpy as np

from .formats import fp16_round

PACK = 8          # 4-bit integers per 32-bit word


def unpack_int4(qweight, K: int) -> np.ndarray:
    """uint8 [N][K] integers 0..15 from packed words [N][K/8]."""
    words = np.asarray(qweight, dtype=np.uint32)
    N = words.shape[0]
    assert words.shape[1] * PACK == K
    out = np.empty((N, K // PACK, PACK), dtype=np.uint8)
    for i in range(PACK):
        out[:, :, i] = (words >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(N, K)


def pack_int4(q) -> np.ndarray:
    """Inverse of unpack_int4: integers 0..15 [N][K] -> uint32 words [N][K/8]."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    assert K % PACK == 0 and q.max(initial=0) < 16
    q = q.reshape(N, K // PACK, PACK)
    words = np.zeros((N, K // PACK), dtype=np.uint32)
    for i in range(PACK):
        words |= q[:, :, i] << np.uint32(4 * i)
    return words


def dequantize(qweight, scales, zeros, K: int, G: int) -> np.ndarray:
    """The fp16 weights the matrix units see, as float64 [N][K]."""
    q = unpack_int4(qweight, K).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), G, axis=1)
    z = np.repeat(np.asarray(zeros, dtype=np.float64), G, axis=1)
    assert s.shape == q.shape and z.shape == q.shape
    return fp16_round(s * (q - z))


def w4a16_gemm(x, qweight, scales, zeros, G: int) -> np.ndarray:
    """Y = X W^T in float64 [M][N] (before the output's fp16 rounding)."""
    x = np.asarray(x, dtype=np.float64)
    w = dequantize(qweight, scales, zeros, x.shape[1], G)
    return x @ w.T


def w4a16_rows(x, qweight, scales, zeros, G: int, cols) -> np.ndarray:
    """Y[:, cols] only: dequantises just the output rows ``cols`` of W."""
    cols = np.asarray(cols)
    return w4a16_gemm(x, np.asarray(qweight)[cols], np.asarray(scales)[cols],
                      np.asarray(zeros)[cols], G)


def w4a16_sum_abs(x, qweight, scales, zeros, G: int, cols=None) -> np.ndarray:
    """sum_k |X[m,k]| |W[n,k]| (float64 [M][N]): the scale of the rounding
    errors of any summation order of Y."""
    if cols is not None:
        qweight, scales, zeros = (np.asarray(a)[np.asarray(cols)] for a in (qweight, scales, zeros))
    x = np.abs(np.asarray(x, dtype=np.float64))
    w = np.abs(dequantize(qweight, scales, zeros, x.shape[1], G))
    return x @ w.T
