"""fp8 (e4m3) path on the GPU against the float64 oracle.

* attn_fp8_prepare: with an exactly representable rotation (a signed
  permutation) the codes and tile scales must equal the oracle's bit for bit;
  with a random orthogonal R the rotated values differ from the oracle's only
  by float32 summation order, so codes may differ only next to a rounding
  midpoint.
* attn_fwd_fp8: compared with "oracle B" -- float64 attention on exactly the
  dequantised inputs the kernel consumes (codes made by the oracle) -- under
  |O - O_B| <= 6e-2 * max(1, |O_B|) (6e-2 ~ 2^-4, e4m3's relative spacing,
  taken as relative once |O| > 1), and, for the fp8 workload without
  outliers, with the unquantised oracle under max-abs <= 6e-2 (gate G1).
  The literal outlier workload is gated against oracle B (gate G2) on 8 heads
  at every row; against the unquantised oracle its literal 6e-2 gate fails,
  recorded as a strict expected failure with the measured value beside the
  input-quantisation floor |O_B - O_A|: quantising the x40 channels alone
  moves O far beyond 6e-2.
"""
import numpy as np
import pytest

import exact_attention_127_amd as A
import oracle
from seeded_inputs import WORKLOADS, haar_orthogonal, make_inputs, random_inputs
from tests.helpers import oracle_heads, record_parity

pytestmark = pytest.mark.gpu
TOL8 = 6e-2


def _dev(x, gpu, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(gpu) if dtype is None else t.to(gpu).to(dtype)


def _gpu_prepare(inp, R, gpu):
    import torch
    outs = A.attn_fp8_prepare(*(_dev(inp[x].astype(np.float32), gpu) for x in "qkv"),
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
    inp = random_inputs(2, 3, N, d, "f32", False, seed=N * 7 + d)
    inp["q"][0, 1, :, 3] *= 40.0                     # an outlier channel
    R = _signed_permutation(d, rng)
    q8, k8, v8, sq, sk, sv = _gpu_prepare(inp, R, gpu)
    (oq, osq), (ok, osk), (ov, osv) = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    for got, want in ((q8, oq), (k8, ok), (v8, ov), (sq, osq), (sk, osk), (sv, osv)):
        assert got.shape == want.shape
        assert np.array_equal(got, want)


def test_prepare_codec_edge_values(gpu):
    """A V tile whose largest magnitude is 448 has scale 1, so its codes are
    the e4m3 codes of the values themselves: midpoints (ties to even),
    subnormals, the subnormal/normal boundary, saturation and signed zero."""
    table = oracle.e4m3_table()
    pos = table[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([pos, -pos, mids, -mids, [0.0, -0.0, 447.9, 448.0, -448.0,
                                                    2.0 ** -10, 2.0 ** -9 * 1.5, 15 / 1024]])
    d, N = 64, 128
    v = np.zeros((1, 1, N, d), np.float32)
    flat = v.reshape(-1)
    flat[:vals.size] = vals.astype(np.float32)
    flat[vals.size] = 448.0
    inp = {"q": v.copy(), "k": v.copy(), "v": v}
    _, _, v8, _, _, sv = _gpu_prepare(inp, np.eye(d, dtype=np.float32), gpu)
    (ov, osv) = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], np.eye(d))[2]
    assert sv.item() == 1.0 == osv.item()
    assert np.array_equal(v8, ov)


@pytest.mark.parametrize("amax", [761.6, 1.0e-3, 3.0e5])
def test_prepare_quotients_near_code_midpoints(gpu, amax):
    """Values x whose quotient x/s lands on, or a few float32 ulps beside,
    the midpoint between two adjacent e4m3 codes, for a scale s = amax/448
    that is not a power of two: the codes follow the float32 quotient
    rounded to nearest, as the oracle computes it."""
    table = oracle.e4m3_table()
    pos = table[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    am = np.float32(amax)
    s = np.float32(am / np.float32(448.0))
    vals = []
    for m in mids:                         # x = fl(m s) and its neighbours up to 3 ulps away
        x0 = np.float32(m * s)
        up = dn = x0
        vals.append(x0)
        for _ in range(3):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(-np.inf))
            vals += [up, dn]
    vals = np.asarray(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    d = 64
    N = 128 * (-(-(vals.size + 1) // (128 * d)))
    v = np.zeros((1, 1, N, d), np.float32)
    flat = v.reshape(-1)
    flat[:vals.size] = vals
    for t in range(N // 128):              # every tile's largest magnitude is amax
        flat[t * 128 * d + 128 * d - 1] = am
    inp = {"q": v.copy(), "k": v.copy(), "v": v}
    _, _, v8, _, _, sv = _gpu_prepare(inp, np.eye(d, dtype=np.float32), gpu)
    (ov, osv) = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], np.eye(d))[2]
    assert np.array_equal(sv, osv) and sv.reshape(-1)[0] == s
    assert np.array_equal(v8, ov)


def test_prepare_random_rotation(gpu):
    w = WORKLOADS["fp8_outliers_8k"].with_(B=1, H=3, N=1000)
    inp = make_inputs(w)
    q8, k8, v8, sq, sk, sv = _gpu_prepare(inp, inp["R"], gpu)
    (oq, osq), (ok, osk), (ov, osv) = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], inp["R"])
    assert np.array_equal(v8, ov) and np.array_equal(sv, osv)
    for got, want, gs, ws, x in ((q8, oq, sq, osq, inp["q"]), (k8, ok, sk, osk, inp["k"])):
        assert np.allclose(gs, ws, rtol=2e-6, atol=0)
        diff = got != want
        # a code may differ only where the exact rotated value is within the
        # float32 summation error bound (gamma_d * sum |x_i R_ic|, plus the
        # scale's own rounding) of the midpoint between the two codes
        x64 = x.astype(np.float64)
        R64 = inp["R"].astype(np.float64)
        y = np.matmul(x64, R64)
        ysum = np.matmul(np.abs(x64), np.abs(R64))
        dd = x.shape[-1]
        gamma = dd * 2.0 ** -24 / (1 - dd * 2.0 ** -24)
        s = np.repeat(ws.astype(np.float64), 128, axis=2)[:, :, :y.shape[2], None]
        z = np.abs(y / s)
        bound = (gamma * ysum + 2.0 ** -24 * np.abs(y)) / s + 4e-6 * z
        lo = oracle.e4m3_decode(want & 0x7F)
        hi = oracle.e4m3_decode(got & 0x7F)
        mid = (lo + hi) / 2
        assert np.all(np.abs(z[diff] - mid[diff]) <= bound[diff])
        assert diff.mean() < 1e-3


def _oracle_b(codes_scales, heads, rows, scale, causal):
    (q8, sq), (k8, sk), (v8, sv) = codes_scales
    qd, kd, vd = (oracle.fp8_dequantize(c, s) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    os_, ls_ = [], []
    for b, h in heads:
        o, l = oracle.attention_rows(qd[b, h], kd[b, h], vd[b, h], scale, causal, rows)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def _fwd_on_codes(cs, gpu, scale, causal):
    import torch
    (q8, sq), (k8, sk), (v8, sv) = cs
    o, lse = A.attn_fwd_fp8(*(_dev(x, gpu) for x in (q8, k8, v8, sq, sk, sv)),
                            scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


# N = 777 = 3*256 + 9 = 6*128 + 9: several full query blocks of 256 or 128
# rows and a ragged last one, whose waves past the end hold no rows
@pytest.mark.parametrize("N", [1, 64, 129, 300, 777])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_vs_dequantised_oracle(gpu, N, d, causal):
    inp = random_inputs(2, 2, N, d, "f32", causal, seed=31 * N + d + causal)
    R = haar_orthogonal(np.random.default_rng(N).standard_normal((d, d))).astype(np.float32)
    cs = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    rows = np.arange(N)
    heads = [(b, h) for b in range(2) for h in range(2)]
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    assert np.all(np.abs(od - ob) <= TOL8 * np.maximum(1.0, np.abs(ob)))
    assert np.abs(od - ob).mean() < 5e-3
    assert np.max(np.abs(ld - lb)) < 2e-2


# B*H a multiple of 8: whole heads per XCD, causal head chunks (every row compared)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_head_grouped_grid(gpu, d, causal):
    N = 777
    inp = random_inputs(2, 8, N, d, "f32", causal, seed=4100 + d + causal)
    R = haar_orthogonal(np.random.default_rng(77).standard_normal((d, d))).astype(np.float32)
    cs = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    rows = np.arange(N)
    heads = [(b, h) for b in range(2) for h in range(8)]
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    assert np.all(np.abs(od - ob) <= TOL8 * np.maximum(1.0, np.abs(ob)))
    assert np.abs(od - ob).mean() < 5e-3
    assert np.max(np.abs(ld - lb)) < 2e-2


def _sample_heads(w, n, seed):
    """n distinct (b, h) pairs, always including the first and the last head."""
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < n:
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    return sorted(heads)


def _full_pipeline(inp, gpu):
    """attn_fp8_prepare + attn_fwd_fp8 on the GPU over the whole workload."""
    import torch
    w = inp["workload"]
    q8, k8, v8, sq, sk, sv = A.attn_fp8_prepare(*(_dev(inp[x], gpu) for x in "qkv"), _dev(inp["R"], gpu))
    o, lse = A.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def test_fp8_workload_no_outliers_vs_unquantised(gpu):
    """Gate G1: the fp8 workload's shapes, rotation and tile scales without the
    outlier channels, full pipeline on the GPU, against the unquantised oracle
    on 8 heads at every row."""
    w = WORKLOADS["fp8_outliers_8k"].with_(outlier_frac=0.0, outlier_mult=1.0)
    inp = make_inputs(w)
    o, _ = _full_pipeline(inp, gpu)
    heads = _sample_heads(w, 8, 1)
    oa, _ = oracle_heads(inp, heads)
    err = np.abs(np.stack([o[b, h] for b, h in heads]) - oa)
    record_parity("fp8_no_outliers_vs_unquantised (G1)", {"max_abs": float(err.max()),
                  "mean_abs": float(err.mean())}, gate_max_abs=TOL8, heads=len(heads), rows=w.N)
    assert err.max() <= TOL8


_C5 = {}


def _literal_fp8(gpu):
    """The literal fp8 workload (x40 outlier channels in Q, K and V), once per
    session: the full GPU pipeline on every head; the kernel on oracle-made
    codes of 8 heads at the full sequence length (heads are independent, so a
    slice of heads is the same work per head); oracle B (float64 attention on
    exactly those dequantised codes) and oracle A (the unquantised inputs) on
    those 8 heads at every row."""
    if not _C5:
        w = WORKLOADS["fp8_outliers_8k"]
        inp = make_inputs(w)
        heads = _sample_heads(w, 8, 3)
        o_full, _ = _full_pipeline(inp, gpu)
        sl = {x: np.ascontiguousarray(np.stack([inp[x][b, h] for b, h in heads])[None]) for x in "qkv"}
        cs = oracle.fp8_prepare(sl["q"], sl["k"], sl["v"], inp["R"])
        o_codes, l_codes = _fwd_on_codes(cs, gpu, w.scale, False)
        (q8, sq), (k8, sk), (v8, sv) = cs
        deq = {"q": oracle.fp8_dequantize(q8, sq), "k": oracle.fp8_dequantize(k8, sk),
               "v": oracle.fp8_dequantize(v8, sv)}
        sl_heads = [(0, i) for i in range(len(heads))]
        ob, lb = oracle_heads(inp, sl_heads, q=deq["q"], k=deq["k"], v=deq["v"])
        oa, la = oracle_heads(inp, sl_heads, q=sl["q"], k=sl["k"], v=sl["v"])
        o_full_h = np.stack([o_full[b, h] for b, h in heads])
        _C5.update(dict(o_codes=o_codes[0], l_codes=l_codes[0], ob=ob, lb=lb, oa=oa, la=la,
                        o_full=o_full_h, heads=heads, N=w.N))
    return _C5


def test_fp8_workload_literal(gpu):
    """Gate G2 on the literal fp8 workload: the kernel on oracle-made codes
    against oracle B, |O - O_B| <= 6e-2 * max(1, |O_B|) at every element of 8
    heads (every row)."""
    c = _literal_fp8(gpu)
    rel = np.abs(c["o_codes"] - c["ob"]) / np.maximum(1.0, np.abs(c["ob"]))
    record_parity("fp8_outliers_8k kernel vs dequantised-input oracle (G2)",
                  {"max_rel": float(rel.max()), "max_abs": float(np.abs(c["o_codes"] - c["ob"]).max()),
                   "mean_abs": float(np.abs(c["o_codes"] - c["ob"]).mean()),
                   "lse_max_abs": float(np.abs(c["l_codes"] - c["lb"]).max())},
                  gate_max_rel=TOL8, heads=len(c["heads"]), rows=c["N"])
    assert np.isfinite(c["o_codes"]).all()
    assert rel.max() <= TOL8


@pytest.mark.xfail(strict=True, reason="literal fp8 gate (max-abs <= 6e-2 against the unquantised "
                   "float64 oracle) fails: quantising the x40 outlier channels to e4m3 alone moves O "
                   "by tens (the input-quantisation floor |O_B - O_A| is recorded beside it)")
def test_fp8_workload_literal_vs_unquantised(gpu):
    c = _literal_fp8(gpu)
    err = np.abs(c["o_full"] - c["oa"])
    floor = np.abs(c["ob"] - c["oa"])
    record_parity("fp8_outliers_8k full pipeline vs unquantised oracle (literal)",
                  {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
                   "floor_input_quant_max": float(floor.max()),
                   "floor_input_quant_mean": float(floor.mean())},
                  gate_max_abs=TOL8, heads=len(c["heads"]), rows=c["N"])
    assert err.max() <= TOL8


def test_fwd_fp8_deterministic_and_guard_bands(gpu):
    """Two launches give identical bits, and nothing outside O and LSE is written."""
    import torch
    B, H, N, d = 2, 3, 777, 128
    inp = random_inputs(B, H, N, d, "f32", True, seed=77)
    R = haar_orthogonal(np.random.default_rng(9).standard_normal((d, d))).astype(np.float32)
    cs = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    (q8, sq), (k8, sk), (v8, sv) = cs
    args = [_dev(x, gpu) for x in (q8, k8, v8, sq, sk, sv)]
    G, n, m = 4096, B * H * N * d, B * H * N
    big = torch.full((n + 2 * G,), 7.0, dtype=torch.bfloat16, device=gpu)
    lbig = torch.full((m + 2 * G,), 7.0, dtype=torch.float32, device=gpu)
    o = big[G:G + n].view(B, H, N, d)
    lse = lbig[G:G + m].view(B, H, N)
    A.attn_fwd_fp8(*args, o=o, lse=lse, scale=inp["scale"], causal=True)
    o2, l2 = A.attn_fwd_fp8(*args, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    assert (big[:G] == 7).all() and (big[G + n:] == 7).all()
    assert (lbig[:G] == 7).all() and (lbig[G + m:] == 7).all()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# B*H = 128 causal with fp8 K/V bytes above 1 MiB per head: each XCD walks
# its 16 heads in two chunks of 8; every row of every head is compared
def test_fwd_fp8_two_head_chunks_per_xcd(gpu):
    B, H, N, d = 16, 8, 4160, 128
    inp = random_inputs(B, H, N, d, "f32", True, seed=4300)
    R = haar_orthogonal(np.random.default_rng(78).standard_normal((d, d))).astype(np.float32)
    cs = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], True)
    (q8, sq), (k8, sk), (v8, sv) = cs
    heads = [(b, h) for b in range(B) for h in range(H)]
    ob, lb = oracle_heads(inp, heads, q=oracle.fp8_dequantize(q8, sq), k=oracle.fp8_dequantize(k8, sk),
                          v=oracle.fp8_dequantize(v8, sv))
    od = o.reshape(ob.shape)
    ld = lse.reshape(lb.shape)
    assert np.all(np.abs(od - ob) <= TOL8 * np.maximum(1.0, np.abs(ob)))
    assert np.abs(od - ob).mean() < 5e-3
    assert np.max(np.abs(ld - lb)) < 2e-2


@pytest.mark.parametrize("rise", [3.0, 20.0, 100.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_rising_scores(gpu, rise, causal):
    """Scores that grow along the keys (3, 20 and 100 per 64 keys): each key
    tile's numerators outgrow the exponent reference of earlier tiles, so the
    kernel must move it to the tile's own maximum again and again."""
    from tests.test_parity_gpu import _rising_inputs
    d, N = 128, 300
    inp = _rising_inputs(N, d, causal, rise, seed=int(rise) + 7 * causal)
    R = haar_orthogonal(np.random.default_rng(5).standard_normal((d, d))).astype(np.float32)
    cs = oracle.fp8_prepare(inp["q"], inp["k"], inp["v"], R)
    o, lse = _fwd_on_codes(cs, gpu, inp["scale"], causal)
    heads = [(0, h) for h in range(2)]
    rows = np.arange(N)
    ob, lb = _oracle_b(cs, heads, rows, inp["scale"], causal)
    od = np.stack([o[b, h] for b, h in heads])
    ld = np.stack([lse[b, h] for b, h in heads])
    assert np.isfinite(od).all() and np.isfinite(ld).all()
    assert np.all(np.abs(od - ob) <= TOL8 * np.maximum(1.0, np.abs(ob)))
    assert np.abs(od - ob).mean() < 5e-3
    assert np.max(np.abs(ld - lb)) < 2e-2
