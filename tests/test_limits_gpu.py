"""The bf16 forward far past the benchmark sizes (GPU).

* One causal sequence of 131 109 keys (2^17 + 37: a ragged last block), at
  d = 64 and d = 128: sampled rows -- the first and last, rows on both sides
  of block edges and random ones -- against the float64 oracle.
* 4224 heads of 4096 tokens at d = 128, causal: each of Q, K, V, O holds
  more than 2^31 elements, so the last heads start past element 2^31, and
  the grid has 67 584 workgroups.
  Five whole heads (the first, the last and three drawn at random) against
  the oracle.  The inputs are drawn on the device with a seeded torch
  generator, one batch entry at a time; the oracle reads those bf16 values
  back for the heads it checks, so both sides see the same numbers.

Gates as for the workloads: O max-abs <= 1e-2, mean-abs <= 1e-3, LSE
max-abs <= 1e-3.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
from seeded_inputs import random_inputs
from tests.helpers import err_stats, oracle_heads, record_parity, sample_rows, to_device

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN, TOL_LSE = 1e-2, 1e-3, 1e-3


@pytest.mark.parametrize("d", [64, 128])
def test_long_sequence_sampled_rows(gpu, d):
    import torch
    N = (1 << 17) + 37
    inp = random_inputs(1, 1, N, d, "bf16", True, seed=5000 + d)
    q, k, v = (to_device(inp[x], torch.bfloat16, gpu) for x in "qkv")
    o, lse = A.attn_fwd(q, k, v, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(N, np.random.default_rng(d), extra=16, block=256)
    rows = np.unique(np.concatenate([rows, np.arange(N - 37, N)]))
    o_ref, l_ref = oracle_heads(inp, [(0, 0)], rows)
    od = o[0, 0].float().cpu().numpy()[rows][None]
    ld = lse[0, 0].cpu().numpy()[rows][None]
    st = err_stats(od, ld, o_ref, l_ref)
    record_parity(f"long_causal_N{N}_d{d}_sampled", st, rows=int(rows.size))
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    assert st["max_abs"] <= TOL_MAX, st
    assert st["mean_abs"] <= TOL_MEAN, st
    assert st["lse_max_abs"] <= TOL_LSE, st


def test_many_heads_past_2_31_elements(gpu):
    import torch
    B, H, N, d = 66, 64, 4096, 128
    g = torch.Generator(device=gpu)
    g.manual_seed(5100)
    q, k, v = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device=gpu) for _ in range(3))
    for t in (q, k, v):
        for b in range(B):
            t[b] = torch.randn((H, N, d), generator=g, device=gpu).to(torch.bfloat16)
    assert q.numel() > 1 << 31 and (B * H - 1) * N * d > 1 << 31
    scale = d ** -0.5
    o, lse = A.attn_fwd(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(51)
    heads = sorted({0, B * H - 1, *(int(x) for x in rng.integers(0, B * H, 3))})
    pairs = [divmod(i, H) for i in heads]
    host = {name: np.stack([t[b, h].float().cpu().numpy() for (b, h) in pairs])[:, None]
            for name, t in (("q", q), ("k", k), ("v", v))}
    inp = {**host, "scale": scale, "causal": True}
    o_ref, l_ref = oracle_heads(inp, [(i, 0) for i in range(len(pairs))])
    od = np.stack([o[b, h].float().cpu().numpy() for (b, h) in pairs])
    ld = np.stack([lse[b, h].cpu().numpy() for (b, h) in pairs])
    st = err_stats(od, ld, o_ref, l_ref)
    record_parity("heads_4224_N4096_d128_causal", st, heads=len(pairs))
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    assert st["max_abs"] <= TOL_MAX, st
    assert st["mean_abs"] <= TOL_MEAN, st
    assert st["lse_max_abs"] <= TOL_LSE, st
