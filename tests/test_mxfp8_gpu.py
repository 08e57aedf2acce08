"""MXFP8 path (one E8M0 scale per 32 channels of a token) on the GPU against
the float64 oracle.

* attn_mxfp8_prepare: with an exactly representable rotation (a signed
  permutation) codes and scale bytes equal the oracle's bit for bit; with a
  random orthogonal R the rotated values differ from the oracle's only by
  float32 summation order, so a scale byte may differ only where the block
  maximum sits at a power-of-two boundary, and a code only next to a
  rounding midpoint.
* attn_fwd_mxfp8 on oracle-made codes against float64 attention on exactly
  the dequantised inputs ("oracle B").  Widening V to bf16 is exact, so the
  remaining error is the bf16 rounding of P (at most u = 2^-8, bf16's unit
  roundoff, of each weight, i.e. <= u (P|V|) per output) and of O (<= u |O|),
  plus the float32 sums inside the score instruction: a sum of d exact
  products rounded faithfully at every step (any rounding mode) errs by at
  most d 2^-23 sum|q_c k_c| <= d 2^-23 |q| |k|, which moves each weight p by
  a factor within exp(+-delta), delta = scale d 2^-23 max|q| max|k|, and O by
  at most 2 (e^delta - 1) (P|V|) (numerator and normaliser).  Element by
  element, with P|V| from the oracle.
* the full pipeline (prepare + forward) on the fp8 workload without outlier
  channels against the unquantised oracle, under the fp8 tolerance 6e-2; with
  the x40 outliers the scores reach thousands, e4m3's 2^-4 relative spacing
  moves them by tens and the softmax can select another key, so that
  comparison is printed beside the input-quantisation floor, and the kernel
  is gated against oracle B on the same inputs instead.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
import oracle
from seeded_inputs import WORKLOADS, haar_orthogonal, make_inputs, random_inputs
from tests.helpers import oracle_heads, record_parity

pytestmark = pytest.mark.gpu
TOL8 = 6e-2


def _dev(x, gpu):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(gpu)


def _gpu_prepare(inp, R, gpu):
    import torch
    outs = A.attn_mxfp8_prepare(*(_dev(inp[x].astype(np.float32), gpu) for x in "qkv"),
                                _dev(np.asarray(R, np.float32), gpu))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in outs]


def _signed_permutation(d, rng):
    P = np.zeros((d, d), np.float32)
    P[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d)
    return P


@pytest.mark.parametrize("N", [1, 128, 300])
@pytest.mark.parametrize("d", [64, 128])
def test_prepare_exact_rotation_bit_exact(gpu, N, d):
    rng = np.random.default_rng(N + d)
    inp = random_inputs(2, 3, N, d, "f32", False, seed=N * 5 + d)
    inp["q"][0, 1, :, 3] *= 40.0                       # an outlier channel
    inp["v"][1, 2, :, 37 % d] *= 1e-3                  # a small channel
    inp["k"][1, 0, :min(N, 5), :32] = 0.0              # all-zero blocks
    R = _signed_permutation(d, rng)
    q8, k8, v8, sq, sk, sv = _gpu_prepare(inp, R, gpu)
    (oq, osq), (ok, osk), (ov, osv) = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], R)
    for got, want in ((q8, oq), (k8, ok), (v8, ov), (sq, osq), (sk, osk), (sv, osv)):
        assert got.shape == want.shape and got.dtype == want.dtype
        assert np.array_equal(got, want)


def test_prepare_random_rotation(gpu):
    w = WORKLOADS["fp8_outliers_8k"].with_(B=1, H=3, N=1000)
    inp = make_inputs(w)
    q8, k8, v8, sq, sk, sv = _gpu_prepare(inp, inp["R"], gpu)
    (oq, osq), (ok, osk), (ov, osv) = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], inp["R"])
    assert np.array_equal(v8, ov) and np.array_equal(sv, osv)
    for got, want, gs, ws in ((q8, oq, sq, osq), (k8, ok, sk, osk)):
        assert (gs != ws).mean() < 1e-3               # block maxima on a power-of-two boundary only
        same = np.repeat(gs == ws, 32, axis=-1)
        diff = (got != want) & same
        assert diff.mean() < 1e-3
        # where the codes differ, the two decoded values are neighbours (a midpoint case)
        a = oracle.e4m3_decode(got[diff] & 0x7F)
        b = oracle.e4m3_decode(want[diff] & 0x7F)
        tab = np.sort(np.unique(oracle.e4m3_table()[:127]))
        ia, ib = np.searchsorted(tab, a), np.searchsorted(tab, b)
        assert np.all(np.abs(ia - ib) <= 1)


def _fwd_on_codes(cs, gpu, scale, causal):
    import torch
    (q8, sq), (k8, sk), (v8, sv) = cs
    o, lse = A.attn_fwd_mxfp8(*(_dev(x, gpu) for x in (q8, k8, v8, sq, sk, sv)),
                              scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _oracle_b(cs, heads, rows, scale, causal):
    (q8, sq), (k8, sk), (v8, sv) = cs
    qd, kd, vd = (oracle.dequantize_mx(c, s) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    os_, ls_ = [], []
    for b, h in heads:
        o, l = oracle.attention_rows(qd[b, h], kd[b, h], vd[b, h], scale, causal, rows)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def _acc_delta(qd, kd, scale):
    """delta = scale d 2^-23 max|q| max|k| of one head (float32 score sums)."""
    d = qd.shape[-1]
    return scale * d * 2.0 ** -23 * np.linalg.norm(qd, axis=-1).max() * np.linalg.norm(kd, axis=-1).max()


def _bound(cs, heads, rows, scale, causal):
    """2^-8 (P|V|) + 2^-8 |O_B| + 2 (e^delta - 1) (P|V|): the bf16 rounding
    (unit roundoff 2^-8) of P and of O, and the float32 sums of the scores."""
    (q8, sq), (k8, sk), (v8, sv) = cs
    qd, kd, vd = (oracle.dequantize_mx(c, s) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    bs = []
    for b, h in heads:
        pv, _ = oracle.attention_rows(qd[b, h], kd[b, h], np.abs(vd[b, h]), scale, causal, rows)
        ob, _ = oracle.attention_rows(qd[b, h], kd[b, h], vd[b, h], scale, causal, rows)
        dl = _acc_delta(qd[b, h], kd[b, h], scale)
        bs.append((2.0 ** -8 + 2 * np.expm1(dl)) * pv + 2.0 ** -8 * np.abs(ob) + 1e-6)
    return np.stack(bs)


# N = 777 = 3*256 + 9 = 6*128 + 9: several full query blocks of 256 or 128
# rows and a ragged last one, whose waves past the end hold no rows
@pytest.mark.parametrize("N", [1, 64, 129, 300, 777])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_mxfp8_vs_dequantised_oracle(gpu, N, d, causal):
    inp = random_inputs(2, 2, N, d, "f32", causal, seed=37 * N + d + causal)
    inp["v"][0, 1, :, 5] *= 40.0                       # an outlier channel of V
    R = haar_orthogonal(np.random.default_rng(N + 1).standard_normal((d, d))).astype(np.float32)
    cs = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    heads = [(b, h) for b in range(2) for h in range(2)]
    rows = np.arange(N)
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    bound = _bound(cs, heads, rows, inp["scale"], causal)
    print(f"N={N} d={d} causal={causal}: max err/bound {(np.abs(od - ob) / bound).max():.3f} "
          f"lse {np.abs(ld - lb).max():.2e}")
    assert np.all(np.abs(od - ob) <= bound)
    assert np.abs(ld - lb).max() <= 1e-3


# B*H a multiple of 8: whole heads per XCD, causal head chunks (every row compared)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_mxfp8_head_grouped_grid(gpu, d, causal):
    N = 777
    inp = random_inputs(2, 8, N, d, "f32", causal, seed=4300 + d + causal)
    R = haar_orthogonal(np.random.default_rng(79).standard_normal((d, d))).astype(np.float32)
    cs = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    heads = [(b, h) for b in range(2) for h in range(8)]
    rows = np.arange(N)
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    bound = _bound(cs, heads, rows, inp["scale"], causal)
    assert np.all(np.abs(od - ob) <= bound)
    assert np.abs(ld - lb).max() <= 1e-3


def _sample_heads(w, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(n)} | {(0, 0)})


def test_fp8_workload_no_outliers_full_pipeline(gpu):
    """The fp8 workload's shapes and rotation without the outlier channels,
    attn_mxfp8_prepare + attn_fwd_mxfp8 at full size, sampled heads and rows
    against the unquantised oracle, under 6e-2."""
    import torch
    w = WORKLOADS["fp8_outliers_8k"].with_(outlier_frac=0.0, outlier_mult=1.0)
    inp = make_inputs(w)
    q8, k8, v8, sq, sk, sv = A.attn_mxfp8_prepare(*(_dev(inp[x], gpu) for x in "qkv"), _dev(inp["R"], gpu))
    o, _ = A.attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    rows = np.unique(np.concatenate([[0, w.N - 1], np.random.default_rng(6).integers(0, w.N, 48)]))
    err = 0.0
    for b, h in _sample_heads(w, 4, 5):
        oa, _ = oracle.attention_rows(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], w.scale, False, rows)
        err = max(err, float(np.abs(o[b, h][rows] - oa).max()))
    print(f"mxfp8 without outliers, full pipeline vs unquantised oracle: max-abs {err:.4f}")
    assert err <= TOL8


def test_fp8_workload_literal(gpu):
    """The literal fp8 workload (x40 outlier channels): the kernel on
    oracle-made codes of 4 heads at the full sequence length against oracle
    B, every row, under the element-wise bf16 bound; the full GPU pipeline
    against the unquantised oracle recorded beside the input-quantisation
    floor."""
    import torch
    w = WORKLOADS["fp8_outliers_8k"]
    inp = make_inputs(w)
    heads = sorted({(0, 0), (w.B - 1, w.H - 1), (1, 7), (2, 20)})
    sl = {x: np.ascontiguousarray(np.stack([inp[x][b, h] for b, h in heads])[None]) for x in "qkv"}
    cs = oracle.mxfp8_prepare(sl["q"], sl["k"], sl["v"], inp["R"])
    o, _ = _fwd_on_codes(cs, gpu, w.scale, False)
    local = [(0, i) for i in range(len(heads))]
    (q8, sq), (k8, sk), (v8, sv) = cs
    qd, kd, vd = (oracle.dequantize_mx(c, s_) for c, s_ in ((q8, sq), (k8, sk), (v8, sv)))
    ob, _ = oracle_heads(inp, local, q=qd, k=kd, v=vd)
    pv, _ = oracle_heads(inp, local, q=qd, k=kd, v=np.abs(vd))
    dl = np.array([_acc_delta(qd[0, i], kd[0, i], w.scale) for i in range(len(heads))])[:, None, None]
    bound = (2.0 ** -8 + 2 * np.expm1(dl)) * pv + 2.0 ** -8 * np.abs(ob) + 1e-6
    od = o[0]
    assert np.all(np.abs(od - ob) <= bound)

    q8, k8, v8, sq, sk, sv = A.attn_mxfp8_prepare(*(_dev(inp[x], gpu) for x in "qkv"), _dev(inp["R"], gpu))
    of, _ = A.attn_fwd_mxfp8(q8, k8, v8, sq, sk, sv, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    of = np.stack([of[b, h].float().cpu().numpy() for b, h in heads])
    oa, _ = oracle_heads(inp, local, q=sl["q"], k=sl["k"], v=sl["v"])
    record_parity("mxfp8 fp8_outliers_8k kernel on oracle codes vs dequantised oracle",
                  {"max_err_over_bound": float((np.abs(od - ob) / bound).max()),
                   "max_abs": float(np.abs(od - ob).max())}, heads=len(heads), rows=w.N)
    record_parity("mxfp8 fp8_outliers_8k full pipeline vs unquantised oracle (literal, not gated)",
                  {"max_abs": float(np.abs(of - oa).max()), "mean_abs": float(np.abs(of - oa).mean()),
                   "floor_input_quant_max": float(np.abs(ob - oa).max())}, gate_max_abs=TOL8,
                  heads=len(heads), rows=w.N)


def test_fwd_mxfp8_deterministic_and_guard_bands(gpu):
    """Two launches give identical bits, and nothing outside O and LSE is written."""
    import torch
    B, H, N, d = 2, 3, 777, 128
    inp = random_inputs(B, H, N, d, "f32", True, seed=78)
    R = haar_orthogonal(np.random.default_rng(10).standard_normal((d, d))).astype(np.float32)
    cs = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], R)
    (q8, sq), (k8, sk), (v8, sv) = cs
    args = [_dev(x, gpu) for x in (q8, k8, v8, sq, sk, sv)]
    G, n, m = 4096, B * H * N * d, B * H * N
    big = torch.full((n + 2 * G,), 7.0, dtype=torch.bfloat16, device=gpu)
    lbig = torch.full((m + 2 * G,), 7.0, dtype=torch.float32, device=gpu)
    o = big[G:G + n].view(B, H, N, d)
    lse = lbig[G:G + m].view(B, H, N)
    A.attn_fwd_mxfp8(*args, o=o, lse=lse, scale=inp["scale"], causal=True)
    o2, l2 = A.attn_fwd_mxfp8(*args, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    assert (big[:G] == 7).all() and (big[G + n:] == 7).all()
    assert (lbig[:G] == 7).all() and (lbig[G + m:] == 7).all()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("rise", [3.0, 20.0, 100.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_mxfp8_rising_scores(gpu, rise, causal):
    """Scores that grow along the keys (3, 20 and 100 per 64 keys): the
    exponent reference has to move to each new tile's maximum."""
    from tests.test_parity_gpu import _rising_inputs
    d, N = 128, 300
    inp = _rising_inputs(N, d, causal, rise, seed=int(rise) + 11 * causal)
    R = haar_orthogonal(np.random.default_rng(6).standard_normal((d, d))).astype(np.float32)
    cs = oracle.mxfp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    heads = [(0, h) for h in range(2)]
    rows = np.arange(N)
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    bound = _bound(cs, heads, rows, inp["scale"], causal)
    # LSE: scores reach ~1e3 before scaling here, so the float32 sum of the
    # d exact code products inside the block-scaled matrix core joins the
    # 1e-3.  A sum of d terms whose every partial sum is rounded faithfully
    # (to either neighbouring float, whatever the rounding mode) errs by at
    # most d u sum|q_c k_c| with u = 2^-23, one unit in the last place; the
    # instruction's internal rounding mode is not documented, so that
    # mode-independent bound is the gate.  (Round-to-nearest would give
    # u = 2^-24; a first gate at that value failed by 1.5x at rise 100.)
    (q8, sq), (k8, sk), _ = cs
    qd, kd = oracle.dequantize_mx(q8, sq), oracle.dequantize_mx(k8, sk)
    acc = max(float((np.abs(qd[b, h]) @ np.abs(kd[b, h]).T).max()) for b, h in heads)
    lse_gate = 1e-3 + d * 2.0 ** -23 * inp["scale"] * acc
    print(f"rise={rise} causal={causal}: max err/bound {(np.abs(od - ob) / bound).max():.3f} "
          f"lse {np.abs(ld - lb).max():.2e} (gate {lse_gate:.2e})")
    assert np.all(np.abs(od - ob) <= bound)
    assert np.abs(ld - lb).max() <= lse_gate
