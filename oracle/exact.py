"""float64 exact attention, the plain definition -- TEST INFRASTRUCTURE ONLY.

Per head (page "Self-Attention, CUDA kernels and FlashAttention", section 1):

    S   = Q K^T * scale                       (scaled dot-product scores)
    S_ij = -inf for j > i when causal          (reading: square self-attention,
                                                row i sees keys 0..i)
    P   = row-softmax(S)                      (each row sums to one)
    O   = P V
    LSE_i = m_i + ln sum_j exp(S_ij - m_i),  m_i = max_j S_ij
                                              (the small per-row normalisation
                                               statistic kept instead of S,
                                               same page, section 3)

The score matrix is materialised exactly as the page's "standard attention"
does, one block of at most ``ROW_CHUNK`` query rows at a time; rows are
independent, so the chunking does not change any value.  Inputs of any float
dtype are upcast to float64 first, so the oracle sees exactly the values the
GPU sees.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


def _scores(q64: np.ndarray, k64: np.ndarray, rows: np.ndarray, scale: float,
            causal: bool) -> np.ndarray:
    """Scaled, masked scores of the given query rows against every key."""
    s = (q64[rows] @ k64.T) * float(scale)
    if causal:
        keys = np.arange(k64.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    return s


def _softmax_stats(s: np.ndarray):
    """Row max, row-softmax P and log-sum-exp of a block of scores."""
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe[:, None])
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(finite[:, None], e / denom[:, None], 0.0)
        lse = np.where(finite, m_safe + np.log(denom), -np.inf)
    return p, lse


def attention_rows(q, k, v, scale, causal, rows):
    """O (float64 ``[len(rows), d]``) and LSE (``[len(rows)]``) of one head.

    ``q, k, v`` are ``[N, d]`` arrays of one (batch, head); ``rows`` selects
    query rows.  A row that sees no key (only possible for an empty key set)
    gives O = 0 and LSE = -inf.
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v64.shape[1]))
    lse = np.empty(rows.size)
    for c0 in range(0, rows.size, ROW_CHUNK):
        r = rows[c0:c0 + ROW_CHUNK]
        if causal:
            # keys beyond the last visible one contribute exp(-inf) = 0
            kmax = int(r.max()) + 1
            s = _scores(q64, k64[:kmax], r, scale, causal)
            p, l_ = _softmax_stats(s)
            o[c0:c0 + r.size] = p @ v64[:kmax]
        else:
            s = _scores(q64, k64, r, scale, causal)
            p, l_ = _softmax_stats(s)
            o[c0:c0 + r.size] = p @ v64
        lse[c0:c0 + r.size] = l_
    return o, lse


def attention(q, k, v, scale, causal):
    """Full ``[B,H,N,d]`` attention: returns (O float64 ``[B,H,N,d]``, LSE ``[B,H,N]``)."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.zeros((B, H, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            if N:
                o[b, h], lse[b, h] = attention_rows(q[b, h], k[b, h], v[b, h],
                                                    scale, causal, rows)
    return o, lse


def attention_probs(q, k, scale, causal):
    """The full probability matrix P of one head (small inputs only)."""
    q64 = np.asarray(q, dtype=np.float64)
    rows = np.arange(q64.shape[0])
    s = _scores(q64, np.asarray(k, dtype=np.float64), rows, scale, causal)
    return _softmax_stats(s)[0]
