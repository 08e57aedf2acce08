"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 implementations of what the GPU path computes.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the library and its Python binding never do, and this package imports
nothing from them (the two sides share only the seeded input generator in
``seeded_inputs``).

Sources followed (page title, section):
  * "Self-Attention, CUDA kernels and FlashAttention", section 1 (the scaled
    dot-product scores, the row softmax whose rows sum to one, the product
    with V, heads in parallel) and section 3 (standard attention
    materialises the N x N score matrix -- which is exactly what this oracle
    does, one block of rows at a time; FlashAttention keeps only small
    normalisation statistics, read here as the natural-log log-sum-exp).
  * "FlashAttention scaling, multi-GPU training and weight quantization",
    section 1, FP8 bullet (block quantisation with an independent scale per
    small tile; incoherent processing: Q and K multiplied by a random
    orthogonal matrix before quantisation).
  * "Efficient MoE training for biological foundation models", the section
    on memory and quantisation costs (MXFP8: one scale per block of 32
    values): ``mx`` holds that block quantisation.
  * "FlashAttention scaling, multi-GPU training and weight quantization",
    section 3 (W4A16: packed 4-bit weights unpacked and dequantised to FP16
    in registers, fed to the matrix units): ``w4a16``.
  * The backward pass of the first page, section 3 (only small statistics
    are kept; tiles are recomputed): ``backward`` holds the gradients of the
    forward definition, written out by the chain rule.

Pins (tests/test_oracle*.py): high-precision brute force on tiny inputs,
hand-worked closed forms (tests/golden/), invariants (rows of P sum to one,
Q = 0 gives the mean of the visible V rows, causal row 0 equals V[0], a
dominant score selects one V row, invariance under a common orthogonal
rotation of Q and K, linearity in V), and the e4m3 / bf16 codecs against the
OCP 8-bit floating-point definition and torch's casts; the gradients against
central finite differences of the forward oracle and against invariants (the
dK rows sum to zero, the dV rows sum to the dO rows, identical keys give
dQ = 0).  Every function here is pinned; none is "parity unpinned".
"""
from .exact import attention, attention_rows, attention_probs
from .formats import (bf16_round, bf16_half_ulp, fp16_round, e4m3_decode, e4m3_encode,
                      E4M3_MAX, e4m3_table)
from .fp8 import fp8_prepare, fp8_dequantize, QUANT_TILE
from .backward import (attention_backward, attention_backward_head, row_delta,
                       dq_rows, dkdv_cols)
from .mx import mxfp8_prepare, quantize_mx, dequantize_mx, mx_exponent, MX_BLOCK
from .w4a16 import unpack_int4, pack_int4, dequantize, w4a16_gemm, w4a16_rows, w4a16_sum_abs

__all__ = ["attention", "attention_rows", "attention_probs",
           "bf16_round", "bf16_half_ulp", "e4m3_decode", "e4m3_encode",
           "E4M3_MAX", "e4m3_table", "fp8_prepare", "fp8_dequantize",
           "QUANT_TILE", "attention_backward", "attention_backward_head",
           "row_delta", "dq_rows", "dkdv_cols", "mxfp8_prepare", "quantize_mx",
           "dequantize_mx", "mx_exponent", "MX_BLOCK", "fp16_round", "unpack_int4",
           "pack_int4", "dequantize", "w4a16_gemm", "w4a16_rows", "w4a16_sum_abs"]
