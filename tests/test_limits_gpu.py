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

* The backward pass on the same 4224 heads: dQ, dK, dV of three whole
  heads against the float64 gradient oracle.
* The fp8 and MXFP8 paths on 4224 heads of float32 tokens: codes and scales
  of three whole heads bit-exact under a signed-permutation rotation, and
  the forward on them against float64 attention on the dequantised codes.

Forward gates as for the workloads: O max-abs <= 1e-2, mean-abs <= 1e-3,
LSE max-abs <= 1e-3.  Backward gates as for the long-row workloads:
max |G - R| / max |R| <= 5e-2 and mean |G - R| / mean |R| <= 1e-2 per
gradient tensor.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
import oracle
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


BIG = (66, 64, 4096, 128)          # B, H, N, d: more than 2^31 elements per tensor


def _device_normal(shape, n, seed, gpu):
    """n bf16 tensors of standard normal draws from one seeded device
    generator, filled one batch entry at a time."""
    import torch
    g = torch.Generator(device=gpu)
    g.manual_seed(seed)
    out = [torch.empty(shape, dtype=torch.bfloat16, device=gpu) for _ in range(n)]
    for t in out:
        for b in range(shape[0]):
            t[b] = torch.randn(shape[1:], generator=g, device=gpu).to(torch.bfloat16)
    return out


def test_many_heads_past_2_31_elements(gpu):
    import torch
    B, H, N, d = BIG
    q, k, v = _device_normal(BIG, 3, 5100, gpu)
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


def test_backward_many_heads_past_2_31_elements(gpu):
    import torch
    B, H, N, d = BIG
    q, k, v, do = _device_normal(BIG, 4, 5200, gpu)
    scale = d ** -0.5
    o, lse = A.attn_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = A.attn_bwd(q, k, v, o, do, lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(52)
    heads = sorted({0, B * H - 1, int(rng.integers(0, B * H))})
    for i in heads:
        b, h = divmod(i, H)
        x = [t[b, h].float().cpu().numpy().astype(np.float64) for t in (q, k, v, do)]
        ref = oracle.attention_backward_head(*x, scale, True)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            gv = got[b, h].float().cpu().numpy().astype(np.float64)
            diff = np.abs(gv - r)
            rel_max = float(diff.max()) / max(float(np.abs(r).max()), 1e-3)
            rel_mean = float(diff.mean()) / max(float(np.abs(r).mean()), 1e-6)
            record_parity(f"bwd_heads_4224_N4096_d128_causal_head{i}_{name}",
                          {"rel_max": rel_max, "rel_mean": rel_mean})
            assert np.isfinite(gv).all(), (i, name)
            assert rel_max <= 5e-2 and rel_mean <= 1e-2, (i, name, rel_max, rel_mean)


def test_fp8_many_heads_past_2_31_elements(gpu):
    """attn_fp8_prepare then attn_fwd_fp8 on 4224 heads of 4096 float32
    tokens.  With a signed permutation as the rotation (exact in float32)
    the sampled heads' e4m3 codes and tile scales equal the oracle's bit for
    bit; the forward on them is held to the small-shape fp8 gates against
    float64 attention on the dequantised codes."""
    import torch
    B, H, N, d = BIG
    g = torch.Generator(device=gpu)
    g.manual_seed(5300)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device=gpu) for _ in range(3))
    rng = np.random.default_rng(53)
    R = np.zeros((d, d), np.float32)
    R[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d)
    q8, k8, v8, sq, sk, sv = A.attn_fp8_prepare(q, k, v, torch.from_numpy(R).to(gpu))
    o, lse = A.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale=d ** -0.5, causal=True)
    torch.cuda.synchronize()
    heads = sorted({0, B * H - 1, int(rng.integers(0, B * H))})
    pairs = [divmod(i, H) for i in heads]
    pick = lambda t: np.stack([t[b, h].cpu().numpy() for (b, h) in pairs])[None]
    (oq, osq), (ok, osk), (ov, osv) = oracle.fp8_prepare(pick(q), pick(k), pick(v), R)
    for got, want in ((q8, oq), (k8, ok), (v8, ov), (sq, osq), (sk, osk), (sv, osv)):
        assert np.array_equal(pick(got), want)
    qd, kd, vd = (oracle.fp8_dequantize(c, s) for c, s in ((oq, osq), (ok, osk), (ov, osv)))
    inp = {"q": qd[0][:, None], "k": kd[0][:, None], "v": vd[0][:, None], "scale": d ** -0.5, "causal": True}
    o_ref, l_ref = oracle_heads(inp, [(i, 0) for i in range(len(pairs))])
    od = pick(o.float())[0]
    ld = pick(lse)[0]
    st = err_stats(od, ld, o_ref, l_ref)
    record_parity("fp8_heads_4224_N4096_d128_causal", st, heads=len(pairs))
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    assert np.all(np.abs(od - o_ref) <= 6e-2 * np.maximum(1.0, np.abs(o_ref)))
    assert st["mean_abs"] < 5e-3 and st["lse_max_abs"] < 2e-2, st


def test_mxfp8_many_heads_past_2_31_elements(gpu):
    """attn_mxfp8_prepare then attn_fwd_mxfp8 on the same 4224 heads: codes and
    E8M0 scale bytes of three whole heads bit-exact under a signed-permutation
    rotation; the forward within the element-wise bound of the MXFP8 tests
    (bf16 rounding of P and O, float32 score sums) of float64 attention on
    the dequantised codes."""
    import torch
    from tests.test_mxfp8_gpu import _acc_delta
    B, H, N, d = BIG
    g = torch.Generator(device=gpu)
    g.manual_seed(5400)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device=gpu) for _ in range(3))
    rng = np.random.default_rng(54)
    R = np.zeros((d, d), np.float32)
    R[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d)
    q8, k8, v8, sq, sk, sv = A.attn_mxfp8_prepare(q, k, v, torch.from_numpy(R).to(gpu))
    scale = d ** -0.5
    o, lse = A.attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, scale=scale, causal=True)
    torch.cuda.synchronize()
    heads = sorted({0, B * H - 1, int(rng.integers(0, B * H))})
    pairs = [divmod(i, H) for i in heads]
    pick = lambda t: np.stack([t[b, h].cpu().numpy() for (b, h) in pairs])[None]
    (oq, osq), (ok, osk), (ov, osv) = oracle.mxfp8_prepare(pick(q), pick(k), pick(v), R)
    for got, want in ((q8, oq), (k8, ok), (v8, ov), (sq, osq), (sk, osk), (sv, osv)):
        assert np.array_equal(pick(got), want)
    qd, kd, vd = (oracle.dequantize_mx(c, s)[0][:, None] for c, s in ((oq, osq), (ok, osk), (ov, osv)))
    inp = {"q": qd, "k": kd, "v": vd, "scale": scale, "causal": True}
    hs = [(i, 0) for i in range(len(pairs))]
    o_ref, l_ref = oracle_heads(inp, hs)
    pv, _ = oracle_heads(inp, hs, v=np.abs(vd))
    od = pick(o.float())[0]
    ld = pick(lse)[0]
    st = err_stats(od, ld, o_ref, l_ref)
    record_parity("mxfp8_heads_4224_N4096_d128_causal", st, heads=len(pairs))
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    for i in range(len(pairs)):
        dl = _acc_delta(qd[i, 0], kd[i, 0], scale)
        bound = (2.0 ** -8 + 2 * np.expm1(dl)) * pv[i] + 2.0 ** -8 * np.abs(o_ref[i]) + 1e-6
        assert np.all(np.abs(od[i] - o_ref[i]) <= bound), i
        assert np.abs(ld[i] - l_ref[i]).max() <= 1e-3 + dl, i
