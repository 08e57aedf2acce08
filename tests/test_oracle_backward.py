"""Pins for the float64 gradient oracle (oracle/backward.py).

The gradients are checked against central finite differences of the forward
oracle (itself pinned to 50-digit brute force), so the closed form is tested
against the forward definition rather than against a retyping of itself; and
against invariants that hold for any input:
  * sum over keys of dK = 0 (each row of dS sums to zero),
  * sum over keys of dV = sum over queries of dO (each row of P sums to one),
  * identical keys give dQ = 0,
  * D_i = sum_j P_ij dP_ij equals sum_c dO_ic O_ic.
"""
import numpy as np
import pytest

import oracle
import oracle.backward as ob


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_rows(q, k, v, scale, causal, np.arange(q.shape[0]))
    return float((o * do).sum())


def _fd_grad(q, k, v, do, scale, causal, which, eps=1e-5):
    args = {"q": q, "k": k, "v": v}
    x = args[which]
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy(); xp[idx] += eps
        xm = x.copy(); xm[idx] -= eps
        ap = dict(args, **{which: xp}); am = dict(args, **{which: xm})
        g[idx] = (_loss(ap["q"], ap["k"], ap["v"], do, scale, causal)
                  - _loss(am["q"], am["k"], am["v"], do, scale, causal)) / (2 * eps)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d,dv", [(6, 4, 4), (7, 3, 5)])
def test_gradients_match_finite_differences(causal, n, d, dv, monkeypatch):
    # blocks of 4 rows, so the accumulation of dK and dV across row blocks is exercised
    monkeypatch.setattr(ob, "ROW_CHUNK", 4)
    rng = np.random.default_rng(100 + n + 10 * causal)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    do = rng.standard_normal((n, dv))
    scale = 0.7
    dq, dk, dv_ = ob.attention_backward_head(q, k, v, do, scale, causal)
    for name, got in (("q", dq), ("k", dk), ("v", dv_)):
        ref = _fd_grad(q, k, v, do, scale, causal, name)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    rng = np.random.default_rng(7)
    n, d = 40, 16
    q, k, v, do = (rng.standard_normal((n, d)) * 1.5 for _ in range(4))
    dq, dk, dv = ob.attention_backward_head(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    # identical keys: every visible score of a row is equal, so dQ vanishes
    k_same = np.repeat(k[:1], n, axis=0)
    dq0, _, _ = ob.attention_backward_head(q, k_same, v, do, 0.3, causal)
    np.testing.assert_allclose(dq0, 0.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_row_delta_equals_softmax_jacobian_term(causal):
    rng = np.random.default_rng(11)
    n, d = 30, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, _ = oracle.attention_rows(q, k, v, 0.5, causal, np.arange(n))
    p = oracle.attention_probs(q, k, 0.5, causal)
    dp = do @ v.T
    np.testing.assert_allclose(ob.row_delta(o, do), (p * dp).sum(axis=1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_columns_match_the_full_gradient(causal, monkeypatch):
    monkeypatch.setattr(ob, "ROW_CHUNK", 16)
    rng = np.random.default_rng(5)
    n, d = 50, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = ob.attention_backward_head(q, k, v, do, 0.4, causal)
    rows = np.array([0, 3, 17, 49])
    np.testing.assert_allclose(ob.dq_rows(q, k, v, do, 0.4, causal, rows), dq[rows], rtol=1e-12, atol=1e-12)
    cols = np.array([0, 1, 30, 49])
    dkc, dvc = ob.dkdv_cols(q, k, v, do, 0.4, causal, cols)
    np.testing.assert_allclose(dkc, dk[cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dvc, dv[cols], rtol=1e-12, atol=1e-12)


def test_causal_last_key_sees_only_the_last_row():
    # with causal masking, key N-1 is visible to row N-1 only, where it is one of N keys
    rng = np.random.default_rng(3)
    n, d = 9, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    _, _, dv = ob.attention_backward_head(q, k, v, do, 1.0, True)
    p_last = oracle.attention_probs(q, k, 1.0, True)[n - 1, n - 1]
    np.testing.assert_allclose(dv[n - 1], p_last * do[n - 1], rtol=1e-12)
