"""float64 gradients of exact attention -- TEST INFRASTRUCTURE ONLY.

The backward pass the page "Self-Attention, CUDA kernels and FlashAttention"
(section 3) describes keeps only the small per-row normalisation statistics
from the forward pass and recomputes the attention tiles.  What it computes is
the gradient of the forward definition (same page, section 1), written out
here by the chain rule.  With dO the gradient of a loss with respect to O and
the forward quantities of one head

    S = Q K^T * scale  (masked),   P = row-softmax(S),   O = P V,

the gradients are

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),   D_i = sum_j P_ij dP_ij     (softmax Jacobian, row i)
    dQ = scale * dS K
    dK = scale * dS^T Q

Masked entries have P_ij = 0 and therefore dS_ij = 0.  D_i equals
sum_c dO_ic O_ic, because O = P V; that second form is the one a kernel uses
with the stored O, and both appear in the pins.

Query rows are processed in blocks of ``ROW_CHUNK`` with the score block
materialised, as the forward oracle does; dK and dV sum the blocks'
contributions, which only changes the order of float64 additions.
"""
from __future__ import annotations

import numpy as np

from .exact import _scores, _softmax_stats

ROW_CHUNK = 1024


def attention_backward_head(q, k, v, do, scale, causal):
    """dQ, dK, dV (float64 ``[N, d]`` each) of one head."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    do64 = np.asarray(do, dtype=np.float64)
    n = q64.shape[0]
    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    for c0 in range(0, n, ROW_CHUNK):
        rows = np.arange(c0, min(n, c0 + ROW_CHUNK))
        s = _scores(q64, k64, rows, scale, causal)
        p, _ = _softmax_stats(s)
        dp = do64[rows] @ v64.T
        d_row = (p * dp).sum(axis=1)
        ds = p * (dp - d_row[:, None])
        dv += p.T @ do64[rows]
        dq[rows] = float(scale) * (ds @ k64)
        dk += float(scale) * (ds.T @ q64[rows])
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal):
    """Gradients for ``[B,H,N,d]`` inputs: (dQ, dK, dV), float64, same shape."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H, N, d))
    dv = np.zeros((B, H, N, np.asarray(v).shape[-1]))
    for b in range(B):
        for h in range(H):
            if N:
                dq[b, h], dk[b, h], dv[b, h] = attention_backward_head(
                    q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv


def row_delta(o, do):
    """D_i = sum_c dO_ic O_ic for every row of ``[..., N, d]`` inputs (float64)."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum(axis=-1)


def dq_rows(q, k, v, do, scale, causal, rows):
    """dQ of the selected query rows of one head (each row needs only its own
    scores, so large heads can be checked row by row)."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    do64 = np.asarray(do, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    s = _scores(q64, k64, rows, scale, causal)
    p, _ = _softmax_stats(s)
    dp = do64[rows] @ v64.T
    ds = p * (dp - (p * dp).sum(axis=1)[:, None])
    return float(scale) * (ds @ k64)


def dkdv_cols(q, k, v, do, scale, causal, cols):
    """dK and dV of the selected key rows of one head.  Every query row
    contributes, so the row statistics of the whole head are formed (one
    block of rows at a time); only the selected key columns are kept."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    do64 = np.asarray(do, dtype=np.float64)
    cols = np.asarray(cols, dtype=np.int64)
    n = q64.shape[0]
    dk = np.zeros((cols.size, k64.shape[1]))
    dv = np.zeros((cols.size, v64.shape[1]))
    for c0 in range(0, n, ROW_CHUNK):
        rows = np.arange(c0, min(n, c0 + ROW_CHUNK))
        s = _scores(q64, k64, rows, scale, causal)
        p, _ = _softmax_stats(s)
        dp = do64[rows] @ v64.T
        d_row = (p * dp).sum(axis=1)
        ds = p[:, cols] * (dp[:, cols] - d_row[:, None])
        dv += p[:, cols].T @ do64[rows]
        dk += float(scale) * (ds.T @ q64[rows])
    return dk, dv
