"""Seeded synthetic inputs for the attention forward pass (and the W4A16
decode product at the end of this file).

This module is shared by the tests, the benchmark and the smoke check.  It
draws random tensors and nothing else: none of the attention arithmetic
(scores, softmax, products, fp8 quantisation) lives here.  Both the CPU
oracle and the GPU path consume exactly the arrays returned here.

Workload shapes follow the pages' own examples: a ViT-B/16 image of 224x224
pixels cut into 16x16 patches gives N = 196 tokens, with 12 heads and
d_k = 64 ("Self-Attention, CUDA kernels and FlashAttention", section 1); the
long-sequence, small-batch case is the one FlashAttention-2's sequence-length
parallelism targets ("FlashAttention scaling, multi-GPU training and weight
quantization", section 1, FlashAttention-2 bullets); the fp8 case follows
FlashAttention-3's block quantisation with incoherent processing (same page,
section 1, FP8 bullet).

Random-number recipe (numpy PCG64 via ``default_rng(seed)``), in draw order:
  1. per-head factors ``c = uniform(0.5, 2.0, size=H)`` if the workload has them;
  2. Q, K, V as float32 ``standard_normal((B, H, N, d))``, in that order;
  3. outlier channels ``integers(0, d, size=(3, n_out * H))`` (rows Q, K, V)
     and a float64 Gaussian ``G`` of shape (d, d) for the rotation, if the
     workload has them.
Per-head factors multiply both Q and K of head h before any rounding.  An
outlier channel is multiplied by ``outlier_mult`` for every batch and token.
bf16 workloads round the float32 draws to bf16 (round to nearest, ties to
even) and return them as float32 arrays whose values are exactly bf16.

The output gradient dO of the backward pass comes from its own stream,
``default_rng(SeedSequence([seed, 1]))``: float32 ``standard_normal((B, H, N,
d))``, rounded the same way for bf16 workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_output_grad", "random_inputs",
           "round_to_bf16_bits", "haar_orthogonal", "W4Workload", "W4_WORKLOADS",
           "make_w4a16_inputs"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32", "bf16" or "fp8" (fp8: f32 inputs quantised by the fp8 path)
    causal: bool
    seed: int
    head_factor: tuple | None = None      # (lo, hi) of the uniform per-head Q/K factor
    outlier_frac: float = 0.0             # fraction of channels per head made outliers
    outlier_mult: float = 1.0
    rotate: bool = False                  # draw a random orthogonal d x d matrix
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "vit_b16_single": Workload(
        "vit_b16_single", 1, 12, 196, 64, "f32", False, 1001,
        note="ViT-B/16 single 224x224 image, fp32"),
    "vit_b16_batch64": Workload(
        "vit_b16_batch64", 64, 12, 196, 64, "bf16", False, 1002,
        note="ViT-B/16 batch of 64, bf16, ragged last key tile"),
    "long_causal_16k": Workload(
        "long_causal_16k", 1, 16, 16384, 128, "bf16", True, 1003,
        note="long sequence, small batch, causal, bf16"),
    "llm_layer_4k": Workload(
        "llm_layer_4k", 8, 32, 4096, 128, "bf16", True, 1004,
        head_factor=(0.5, 2.0),
        note="LLM-style layer, per-head Q/K factor U(0.5,2), causal, bf16"),
    "fp8_outliers_8k": Workload(
        "fp8_outliers_8k", 4, 32, 8192, 128, "fp8", False, 1005,
        outlier_frac=0.005, outlier_mult=40.0, rotate=True,
        note="fp8 e4m3 path, 0.5% outlier channels x40, random rotation of Q and K"),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    # NaN stays NaN; the draws here are finite so this is only a guard.
    return np.where(np.isnan(x), x, out)


def haar_orthogonal(G: np.ndarray) -> np.ndarray:
    """Random orthogonal matrix from a Gaussian draw: QR with the sign of R's diagonal fixed."""
    qm, rm = np.linalg.qr(G)
    return qm * np.sign(np.diag(rm))[None, :]


def _draw(rng, B, H, N, d):
    return rng.standard_normal((B, H, N, d), dtype=np.float32)


def make_inputs(w: Workload | str, seed: int | None = None) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict with ``q, k, v`` (float32 numpy arrays ``[B,H,N,d]``; for
    bf16 workloads the values are exactly bf16), ``scale`` and ``causal``, and
    for rotating workloads ``R`` (float32 ``[d,d]``) plus the outlier channel
    indices ``outliers`` (int ``[3, n_out*H]``) and per-head factors ``c``.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out: dict = {"workload": w, "scale": w.scale, "causal": w.causal}
    c = None
    if w.head_factor is not None:
        c = rng.uniform(w.head_factor[0], w.head_factor[1], size=w.H).astype(np.float32)
        out["c"] = c
    q = _draw(rng, w.B, w.H, w.N, w.d)
    k = _draw(rng, w.B, w.H, w.N, w.d)
    v = _draw(rng, w.B, w.H, w.N, w.d)
    if c is not None:
        q *= c[None, :, None, None]
        k *= c[None, :, None, None]
    if w.outlier_frac > 0:
        n_out = max(1, int(round(w.outlier_frac * w.d)))
        ch = rng.integers(0, w.d, size=(3, n_out * w.H))
        out["outliers"] = ch
        for t, x in enumerate((q, k, v)):
            for h in range(w.H):
                for c_ in ch[t, h * n_out:(h + 1) * n_out]:
                    x[:, h, :, c_] *= np.float32(w.outlier_mult)
    if w.rotate:
        G = rng.standard_normal((w.d, w.d))
        out["R"] = haar_orthogonal(G).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = (round_to_bf16_bits(x) for x in (q, k, v))
    out["q"], out["k"], out["v"] = q, k, v
    return out


def make_output_grad(w: Workload | str, seed: int | None = None) -> np.ndarray:
    """dO for workload ``w``: float32 ``[B,H,N,d]``, exactly bf16 for bf16 workloads."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(np.random.SeedSequence([w.seed if seed is None else seed, 1]))
    do = _draw(rng, w.B, w.H, w.N, w.d)
    return round_to_bf16_bits(do) if w.dtype == "bf16" else do


def random_inputs(B, H, N, d, dtype="bf16", causal=False, seed=0, **kw) -> dict:
    """Small ad-hoc workload with the same recipe (used by parity sweeps)."""
    w = Workload(f"adhoc_{B}x{H}x{N}x{d}", B, H, N, d, dtype, causal, seed, **kw)
    return make_inputs(w)


# ---------------------------------------------------------------------------
# W4A16 decode product ("FlashAttention scaling, multi-GPU training and
# weight quantization", section 3: one token at a time, weights read as 4-bit
# integers).  The page gives no layer shapes; the workloads take the
# feed-forward projection of a 70B-class model (hidden size 8192, 28672
# feed-forward channels) for one token and for a batch of 16 tokens.
#
# Recipe (``default_rng(seed)``), in draw order:
#   1. X: float32 ``standard_normal((M, K))`` cast to fp16 (nearest);
#   2. packed weights: uint32 ``integers(0, 2**32, (N, K/8))`` -- eight
#      independent uniform 4-bit integers per word;
#   3. scales: ``uniform(0.002, 0.02, (N, K/G))`` cast to fp16;
#   4. zero points: ``integers(4, 12, (N, K/G))`` as uint8.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class W4Workload:
    name: str
    M: int
    N: int
    K: int
    G: int
    seed: int
    note: str = ""

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K

    @property
    def bytes(self) -> int:
        """Packed weights, scales (2 B) and zero points (1 B) read once, X read
        once, Y written once (fp16)."""
        return (self.N * self.K // 2 + 3 * self.N * (self.K // self.G)
                + 2 * self.M * self.K + 2 * self.M * self.N)

    def with_(self, **kw) -> "W4Workload":
        return replace(self, **kw)


W4_WORKLOADS = {
    "w4a16_decode_70b": W4Workload(
        "w4a16_decode_70b", 1, 28672, 8192, 128, 1101,
        note="one token through a 70B-class feed-forward projection, int4 groups of 128"),
    "w4a16_batch16_70b": W4Workload(
        "w4a16_batch16_70b", 16, 28672, 8192, 128, 1102,
        note="16 tokens through the same projection"),
    "w4a16_small": W4Workload(
        "w4a16_small", 3, 48, 384, 128, 1103, note="small parity case"),
}


def make_w4a16_inputs(w: W4Workload | str, seed: int | None = None) -> dict:
    """``x`` fp16 [M][K], ``qweight`` uint32 [N][K/8], ``scales`` fp16
    [N][K/G], ``zeros`` uint8 [N][K/G], and ``G``."""
    if isinstance(w, str):
        w = W4_WORKLOADS[w]
    assert w.K % w.G == 0 and w.K % 8 == 0
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = rng.standard_normal((w.M, w.K), dtype=np.float32).astype(np.float16)
    qweight = rng.integers(0, 2 ** 32, size=(w.N, w.K // 8), dtype=np.uint32)
    scales = rng.uniform(0.002, 0.02, size=(w.N, w.K // w.G)).astype(np.float16)
    zeros = rng.integers(4, 12, size=(w.N, w.K // w.G)).astype(np.uint8)
    return {"workload": w, "x": x, "qweight": qweight, "scales": scales, "zeros": zeros,
            "G": w.G}
