"""Shared test helpers: device copies of seeded inputs and error statistics.

Error statistics compare a device result with the float64 oracle; the
bf16 "excess" statistic subtracts the half-spacing of bf16 at each exact
value, i.e. the part of the error that rounding the exact answer to bf16
already forces.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os

import numpy as np

import oracle

# worker threads for whole-tensor oracle comparisons (numpy's BLAS and
# element-wise kernels release the GIL, so heads run in parallel; BLAS is
# held to one thread per worker meanwhile)
ORACLE_WORKERS = min(16, os.cpu_count() or 1)


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


def oracle_heads(inp: dict, heads, rows=None, q=None, k=None, v=None, workers=ORACLE_WORKERS):
    """Oracle O [len(heads), R, d] and LSE [len(heads), R] for (b, h) pairs,
    all rows unless ``rows`` is given, heads computed in parallel threads.
    ``q, k, v`` default to the inputs of ``inp``."""
    from threadpoolctl import threadpool_limits
    q = inp["q"] if q is None else q
    k = inp["k"] if k is None else k
    v = inp["v"] if v is None else v
    N = q.shape[2]
    rows = np.arange(N) if rows is None else np.asarray(rows)

    def one(bh):
        b, h = bh
        return oracle.attention_rows(q[b, h], k[b, h], v[b, h], inp["scale"], inp["causal"], rows)

    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one, list(heads)))
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def oracle_bwd_heads(inp: dict, do: np.ndarray, heads, workers=ORACLE_WORKERS):
    """Oracle dQ, dK, dV [len(heads), N, d] for (b, h) pairs, heads in parallel threads."""
    from threadpoolctl import threadpool_limits

    def one(bh):
        b, h = bh
        return oracle.attention_backward_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                                              do[b, h], inp["scale"], inp["causal"])

    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            res = list(ex.map(one, list(heads)))
    return tuple(np.stack([r[i] for r in res]) for i in range(3))


def record_parity(name: str, stats: dict, **extra) -> None:
    """Print the literal error figures of a parity case on one line and, when
    ATTN_PARITY_LOG names a file, append them to it as a JSON line."""
    rec = {"case": name, **{k_: (round(v_, 9) if isinstance(v_, float) else v_)
                             for k_, v_ in {**stats, **extra}.items()}}
    print("PARITY " + json.dumps(rec), flush=True)
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


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
