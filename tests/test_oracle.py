"""Pins of the float64 attention oracle (CPU only).

Each test fixes the oracle to something other than itself: a 50-digit
brute force, hand-worked closed forms, or an invariant that the definition
on "Self-Attention, CUDA kernels and FlashAttention", section 1, implies.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import attention, attention_rows, attention_probs
from seeded_inputs import WORKLOADS, make_inputs, haar_orthogonal
from tests.bruteforce import attention_bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_attention.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1), (3, 2), (5, 3), (8, 8), (7, 4), (2, 8)])
def test_matches_bruteforce(shape, causal):
    rng = np.random.default_rng(hash((shape, causal)) % 2**32)
    n, d = shape
    q, k, v = _rand(rng, n, d) * 2, _rand(rng, n, d) * 2, _rand(rng, n, d + 1)
    scale = 0.37
    o, lse = attention_rows(q, k, v, scale, causal, np.arange(n))
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lb))) < 1e-12


def test_non_square_keys_bruteforce():
    """More keys than queries and d != N: catches a transposed operand."""
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 3, 5), _rand(rng, 6, 5), _rand(rng, 6, 2)
    o, lse = attention_rows(q, k, v, 0.8, False, np.arange(3))
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.8, False)
    assert np.allclose(o, ob, atol=1e-12, rtol=0)
    assert np.allclose(lse, lb, atol=1e-12, rtol=0)


def test_handworked_golden():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = (np.array(c[x]) for x in ("q", "k", "v"))
        o, lse = attention_rows(q, k, v, c["scale"], c["causal"], np.arange(q.shape[0]))
        assert np.allclose(o, c["o"], atol=1e-12, rtol=0), c["name"]
        assert np.allclose(lse, c["lse"], atol=1e-12, rtol=0), c["name"]


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 64, 16) * 3, _rand(rng, 64, 16) * 3
    p = attention_probs(q, k, 0.25, causal)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)
    assert (p >= 0).all()
    if causal:
        assert np.all(np.triu(p, 1) == 0)
        assert np.all(np.diag(p) > 0)


@pytest.mark.parametrize("name", ["vit_b16_single", "long_causal_16k", "llm_layer_4k"])
def test_zero_query_closed_form(name):
    """Q = 0: every visible key scores 0, so O_i is the mean of the visible V
    rows and LSE_i = ln(#visible), at the workload's full sequence length."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(11)
    N, d = w.N, w.d
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    q = np.zeros((N, d))
    rows = np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 40)]))
    o, lse = attention_rows(q, k, v, w.scale, w.causal, rows)
    for r_i, r in enumerate(rows):
        nvis = r + 1 if w.causal else N
        assert np.allclose(o[r_i], v[:nvis].mean(axis=0), atol=1e-12, rtol=0)
        assert abs(lse[r_i] - np.log(nvis)) < 1e-12


def test_causal_row0_is_v0():
    inp = make_inputs(WORKLOADS["llm_layer_4k"].with_(B=1, H=2, N=300))
    o, lse = attention(inp["q"], inp["k"], inp["v"], inp["scale"], True)
    assert np.array_equal(o[:, :, 0], inp["v"][:, :, 0].astype(np.float64))
    s00 = np.einsum("bhd,bhd->bh", inp["q"][:, :, 0].astype(np.float64),
                    inp["k"][:, :, 0].astype(np.float64)) * inp["scale"]
    assert np.allclose(lse[:, :, 0], s00, atol=1e-12, rtol=0)


def test_dominant_score_selects_one_row():
    rng = np.random.default_rng(5)
    N, d = 50, 8
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    jstar = 17
    q = k[jstar:jstar + 1] * 40.0        # S_{0,j*} = 40|k_j*|^2 dominates
    o, _ = attention_rows(q, k, v, 1.0, False, [0])
    s = (q @ k.T)[0]
    gap = s[jstar] - np.max(np.delete(s, jstar))
    assert gap > 30
    bound = N * np.exp(-gap) * 2 * np.abs(v).max()
    assert np.max(np.abs(o[0] - v[jstar])) <= bound


def test_rotation_invariance():
    """A common orthogonal R leaves Q K^T, hence O and LSE, unchanged
    (the incoherent-processing step of the FP8 bullet)."""
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 2, 96, 32)) for _ in range(3))
    R = haar_orthogonal(rng.standard_normal((32, 32)))
    assert np.allclose(R @ R.T, np.eye(32), atol=1e-13)
    o1, l1 = attention(q, k, v, 0.3, False)
    o2, l2 = attention(q @ R, k @ R, v, 0.3, False)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_linearity_in_v():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, 1, 40, 16)) for _ in range(3))
    o1, _ = attention(q, k, v, 0.25, True)
    o2, _ = attention(q, k, 3.0 * v - 2.0, 0.25, True)
    assert np.max(np.abs(o2 - (3.0 * o1 - 2.0))) < 1e-12


def test_permutation_equivariance_noncausal():
    rng = np.random.default_rng(17)
    q, k, v = (rng.standard_normal((1, 1, 33, 8)) for _ in range(3))
    perm_k = rng.permutation(33)
    perm_q = rng.permutation(33)
    o1, l1 = attention(q, k, v, 0.5, False)
    o2, l2 = attention(q[:, :, perm_q], k[:, :, perm_k], v[:, :, perm_k], 0.5, False)
    assert np.max(np.abs(o2 - o1[:, :, perm_q])) < 1e-12
    assert np.max(np.abs(l2 - l1[:, :, perm_q])) < 1e-12


def test_scale_folds_into_q():
    rng = np.random.default_rng(19)
    q, k, v = (rng.standard_normal((1, 1, 20, 8)) for _ in range(3))
    o1, l1 = attention(q, k, v, 0.125, True)
    o2, l2 = attention(q * 4.0, k, v, 0.125 / 4.0, True)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


def test_full_equals_rows_subset():
    inp = make_inputs(WORKLOADS["vit_b16_single"])
    o, lse = attention(inp["q"], inp["k"], inp["v"], inp["scale"], False)
    rows = np.array([0, 5, 63, 64, 195])
    o2, l2 = attention_rows(inp["q"][0, 3], inp["k"][0, 3], inp["v"][0, 3], inp["scale"], False, rows)
    # BLAS may block the two products differently: equal to the last few ulps
    assert np.allclose(o[0, 3, rows], o2, atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 3, rows], l2, atol=1e-14, rtol=0)


def test_empty_sequence():
    z = np.zeros((1, 2, 0, 8))
    o, lse = attention(z, z, z, 1.0, True)
    assert o.shape == (1, 2, 0, 8) and lse.shape == (1, 2, 0)


# --- planted mistakes: each must be caught by one of the pins above --------

def _bruteforce_case(causal):
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 6, 4), _rand(rng, 6, 4), _rand(rng, 6, 3)
    ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
    return q, k, v, np.array(ob), np.array(lb)


@pytest.mark.parametrize("mistake", ["no_scale", "mask_diagonal", "transpose_k",
                                     "lse_without_max", "softmax_wrong_axis"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    import oracle.exact as A
    good_scores, good_stats = A._scores, A._softmax_stats

    def scores(q64, k64, rows, scale, causal):
        if mistake == "no_scale":
            return good_scores(q64, k64, rows, 1.0, causal)
        if mistake == "mask_diagonal":
            s = good_scores(q64, k64, rows, scale, False)
            if causal:
                keys = np.arange(k64.shape[0])
                s = np.where(keys[None, :] >= rows[:, None], -np.inf, s)
                s[rows == 0, 0] = 0.0   # keep row 0 finite
            return s
        if mistake == "transpose_k":
            return good_scores(q64, k64[::-1], rows, scale, causal)
        return good_scores(q64, k64, rows, scale, causal)

    def stats(s):
        p, lse = good_stats(s)
        if mistake == "lse_without_max":
            m = np.where(np.isfinite(s.max(axis=1)), s.max(axis=1), 0)
            lse = lse - m
        if mistake == "softmax_wrong_axis":
            e = np.exp(np.where(np.isfinite(s), s, -np.inf))
            p = e / e.sum(axis=0, keepdims=True)
        return p, lse

    monkeypatch.setattr(A, "_scores", scores)
    monkeypatch.setattr(A, "_softmax_stats", stats)
    caught = False
    for causal in (False, True):
        q, k, v, ob, lb = _bruteforce_case(causal)
        o, lse = A.attention_rows(q, k, v, 0.6, causal, np.arange(6))
        if np.max(np.abs(o - ob)) > 1e-9 or np.max(np.abs(lse - lb)) > 1e-9:
            caught = True
    assert caught, mistake
