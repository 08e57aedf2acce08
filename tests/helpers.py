"""Shared test helpers: device copies of seeded inputs and error statistics.

Error statistics compare a device result with the float64 oracle; the
bf16 "excess" statistic subtracts the half-spacing of bf16 at each exact
value, i.e. the part of the error that rounding the exact answer to bf16
already forces.
"""
from __future__ import annotations

import numpy as np

import oracle


def to_device(x: np.ndarray, dtype, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device).to(dtype).contiguous()


def sample_rows(N: int, rng, extra: int = 24, block: int = 128) -> np.ndarray:
    """First/last rows, rows at block edges and a few random rows."""
    fixed = [0, 1, N - 1, N - 2]
    for b in range(block, N, block * max(1, (N // block) // 6)):
        fixed += [b - 1, b]
    rows = np.concatenate([np.array(fixed), rng.integers(0, N, extra)])
    return np.unique(rows[(rows >= 0) & (rows < N)])


def oracle_rows(inp: dict, heads, rows):
    """Oracle O [len(heads), len(rows), d] and LSE for selected (b, h) pairs and rows."""
    os_, ls_ = [], []
    for (b, h) in heads:
        o, l = oracle.attention_rows(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                                     inp["scale"], inp["causal"], rows)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def err_stats(o_dev: np.ndarray, lse_dev, o_ref: np.ndarray, lse_ref) -> dict:
    o_dev = np.asarray(o_dev, dtype=np.float64)
    diff = np.abs(o_dev - o_ref)
    st = {"max_abs": float(diff.max()) if diff.size else 0.0,
          "mean_abs": float(diff.mean()) if diff.size else 0.0,
          "excess_bf16": float(np.maximum(0.0, diff - oracle.bf16_half_ulp(o_ref)).max())
          if diff.size else 0.0,
          "floor_bf16": float(np.abs(oracle.bf16_round(o_ref) - o_ref).max()) if diff.size else 0.0,
          "floor_bf16_mean": float(np.abs(oracle.bf16_round(o_ref) - o_ref).mean())
          if diff.size else 0.0}
    if lse_dev is not None and lse_ref is not None:
        ld = np.abs(np.asarray(lse_dev, dtype=np.float64) - lse_ref)
        st["lse_max_abs"] = float(ld.max()) if ld.size else 0.0
    return st
