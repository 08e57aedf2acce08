"""Parity of the backward pass (attn_bwd) with the float64 gradient oracle.

The GPU side runs attn_fwd (for O and LSE) and then attn_bwd on the same
seeded bf16 inputs; the oracle computes the exact gradients of those inputs.
Errors are measured relative to the size of each gradient tensor:
    rel_max  = max |G - R| / max |R|,     rel_mean = mean |G - R| / mean |R|.
Where the tolerances come from:
  * P and dS enter the products rounded to bf16 and the outputs are rounded
    to bf16 (unit roundoff 2^-8 each): about 2.3e-3 mean on short rows, as
    measured, and up to ~4e-3 where dQ is mostly cancellation (N = 2).
  * D = rowsum(dO * O) is formed from the stored bf16 O, as the method keeps
    O and the row statistic rather than S.  Its error does not average out
    over a long row while dQ shrinks (diffuse attention): on the 16k
    workload the oracle alone, with D taken from bf16-rounded exact O, is
    already 1.9e-2 (max) / 2.2e-3 (mean) away from the exact dQ; the device's
    O also carries the forward pass's own error.  Long rows therefore get
    twice that allowance.
"""
import numpy as np
import pytest

import oracle
from helpers import oracle_bwd_heads, to_device
from seeded_inputs import WORKLOADS, make_inputs, make_output_grad, random_inputs

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 1e-2, 5e-3              # rows of at most a few hundred keys
REL_MAX_LONG, REL_MEAN_LONG = 5e-2, 1e-2     # 4k and 16k rows


def _run(inp, do_np, device):
    import torch
    import exact_attention_127_amd as A
    q, k, v, do = (to_device(x, torch.bfloat16, device) for x in (inp["q"], inp["k"], inp["v"], do_np))
    o, lse = A.attn_fwd(q, k, v, scale=inp["scale"], causal=inp["causal"])
    dq, dk, dv = A.attn_bwd(q, k, v, o, do, lse, scale=inp["scale"], causal=inp["causal"])
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def _rel(g, r):
    d = np.abs(g - r)
    big = max(float(np.abs(r).max()), 1e-3)
    mean_ref = max(float(np.abs(r).mean()), 1e-6)
    return float(d.max()) / big, float(d.mean()) / mean_ref


def _check(name, g, r, max_tol=REL_MAX, mean_tol=REL_MEAN):
    rm, rmean = _rel(g, r)
    print(f"{name}: rel_max {rm:.3e} rel_mean {rmean:.3e}")
    assert np.isfinite(g).all(), name
    assert rm <= max_tol and rmean <= mean_tol, (name, rm, rmean)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [2, 31, 64, 65, 127, 129, 200, 300, 449, 700])
def test_small_shapes_match_the_oracle(gpu, N, d, causal):
    inp = random_inputs(1, 2, N, d, "bf16", causal, seed=300 + N + d + causal)
    do = make_output_grad(inp["workload"])
    dq, dk, dv = _run(inp, do, gpu)
    rq, rk, rv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
    _check(f"N={N} d={d} causal={causal} dq", dq, rq)
    _check(f"N={N} d={d} causal={causal} dk", dk, rk)
    _check(f"N={N} d={d} causal={causal} dv", dv, rv)


# B*H a multiple of 8: the dK/dV and dQ grids give each XCD whole heads and,
# when causal, walk chunks of heads; all gradients are compared
@pytest.mark.parametrize("causal", [False, True])
def test_head_grouped_grid(gpu, causal):
    inp = random_inputs(2, 8, 300, 128, "bf16", causal, seed=500 + causal)
    do = make_output_grad(inp["workload"])
    dq, dk, dv = _run(inp, do, gpu)
    rq, rk, rv = oracle.attention_backward(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
    _check(f"B*H=16 causal={causal} dq", dq, rq)
    _check(f"B*H=16 causal={causal} dk", dk, rk)
    _check(f"B*H=16 causal={causal} dv", dv, rv)


@pytest.mark.parametrize("d", [64, 128])
def test_single_token_gradients(gpu, d):
    # one key: P = 1, so dS = 0 (dQ = dK = 0 up to float32 rounding of D) and dV = dO
    inp = random_inputs(1, 3, 1, d, "bf16", True, seed=7)
    do = make_output_grad(inp["workload"])
    dq, dk, dv = _run(inp, do, gpu)
    assert np.abs(dq).max() < 1e-3 and np.abs(dk).max() < 1e-3
    np.testing.assert_array_equal(dv, do.astype(np.float64))


def test_backward_is_deterministic(gpu):
    inp = random_inputs(2, 3, 777, 128, "bf16", True, seed=11)
    do = make_output_grad(inp["workload"])
    a = _run(inp, do, gpu)
    b = _run(inp, do, gpu)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# B*H = 128 causal with per-head Q/dO (dQ kernel) and K/V (dK/dV kernel)
# bytes above 1 MiB: each XCD walks its 16 heads in two chunks of 8; every
# element of every gradient is compared
def test_two_head_chunks_per_xcd(gpu):
    inp = random_inputs(16, 8, 2112, 128, "bf16", True, seed=510)
    do = make_output_grad(inp["workload"])
    dq, dk, dv = _run(inp, do, gpu)
    heads = [(b, h) for b in range(16) for h in range(8)]
    rq, rk, rv = oracle_bwd_heads(inp, do, heads)
    _check("two chunks dq", dq.reshape(rq.shape), rq, REL_MAX_LONG, REL_MEAN_LONG)
    _check("two chunks dk", dk.reshape(rk.shape), rk, REL_MAX_LONG, REL_MEAN_LONG)
    _check("two chunks dv", dv.reshape(rv.shape), rv, REL_MAX_LONG, REL_MEAN_LONG)


def test_guard_bands_untouched(gpu):
    """attn_bwd writes dQ, dK, dV and D and nothing around them."""
    import torch
    import exact_attention_127_amd as A
    B, H, N, d = 1, 3, 777, 128
    inp = random_inputs(B, H, N, d, "bf16", True, seed=12)
    do_np = make_output_grad(inp["workload"])
    q, k, v, do = (to_device(x, torch.bfloat16, gpu) for x in (inp["q"], inp["k"], inp["v"], do_np))
    o, lse = A.attn_fwd(q, k, v, scale=inp["scale"], causal=True)
    G, n, m = 4096, B * H * N * d, B * H * N
    bigs = [torch.full((n + 2 * G,), 7.0, dtype=torch.bfloat16, device=gpu) for _ in range(3)]
    dbig = torch.full((m + 2 * G,), 7.0, dtype=torch.float32, device=gpu)
    dq, dk, dv = (x[G:G + n].view(B, H, N, d) for x in bigs)
    delta = dbig[G:G + m].view(B, H, N)
    A.attn_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, delta=delta, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    for x in bigs:
        assert (x[:G] == 7).all() and (x[G + n:] == 7).all()
    assert (dbig[:G] == 7).all() and (dbig[G + m:] == 7).all()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def _sampled(inp, do, dev_grads, heads, rows, cols):
    dq, dk, dv = dev_grads
    for (b, h) in heads:
        args = (inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], do[b, h], inp["scale"], inp["causal"])
        rq = oracle.dq_rows(*args, rows)
        _check(f"head {b},{h} dq rows", dq[b, h][rows], rq, REL_MAX_LONG, REL_MEAN_LONG)
        if cols is not None:
            rk, rv = oracle.dkdv_cols(*args, cols)
            _check(f"head {b},{h} dk cols", dk[b, h][cols], rk, REL_MAX_LONG, REL_MEAN_LONG)
            _check(f"head {b},{h} dv cols", dv[b, h][cols], rv, REL_MAX_LONG, REL_MEAN_LONG)


def test_llm_layer_4k_sampled(gpu):
    # the 4k-token LLM layer (B=8, H=32, per-head Q/K factor, causal) at full size;
    # dQ rows and dK/dV columns of two heads against the oracle
    w = WORKLOADS["llm_layer_4k"]
    inp = make_inputs(w)
    do = make_output_grad(w)
    grads = _run(inp, do, gpu)
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 4095], rng.integers(0, 4096, 27)]))
    cols = np.unique(np.concatenate([[0, 127, 128, 4094, 4095], rng.integers(0, 4096, 11)]))
    _sampled(inp, do, grads, [(0, 0), (7, 31)], rows, cols)


def test_long_causal_16k_sampled(gpu):
    # B=1 H=16 N=16384 d=128 causal at full size: dQ rows of two heads
    w = WORKLOADS["long_causal_16k"]
    inp = make_inputs(w)
    do = make_output_grad(w)
    grads = _run(inp, do, gpu)
    rng = np.random.default_rng(43)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 8191, 16383], rng.integers(0, 16384, 18)]))
    _sampled(inp, do, grads, [(0, 0), (0, 15)], rows, None)
    dq, dk, dv = grads
    # dV summed over keys equals dO summed over queries (rows of P sum to one)
    for h in (3, 9):
        s_dv = dv[0, h].sum(axis=0)
        s_do = do[0, h].astype(np.float64).sum(axis=0)
        assert np.abs(s_dv - s_do).max() <= 2e-2 * np.abs(dv[0, h]).sum(axis=0).max() / 128
