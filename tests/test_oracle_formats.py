"""Pins of the oracle's number formats and fp8 preparation (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import (E4M3_MAX, bf16_half_ulp, bf16_round, e4m3_decode, e4m3_encode,
                    e4m3_table, fp8_dequantize, fp8_prepare, attention)
from oracle.fp8 import QUANT_TILE, quantize_tiles
from seeded_inputs import WORKLOADS, make_inputs, round_to_bf16_bits


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])


def test_e4m3_definition_landmarks():
    t = e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x38] == 1.0                                   # exponent field 7 = bias
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.all(np.diff(t[:127]) > 0)


def test_e4m3_encode_roundtrip_all_codes():
    t = e4m3_table()
    for code in range(256):
        if np.isnan(t[code]):
            continue
        c = int(e4m3_encode(t[code]))
        assert t[c] == t[code]
        if t[code] != 0:
            assert c == code


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    x = x[np.abs(x) < E4M3_MAX].astype(np.float32)
    # every midpoint between neighbouring finite values (ties go to even)
    pos = e4m3_table()[:127]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = e4m3_encode(x)
    # torch keeps -0 for values rounding to zero from below, as does the encoder here
    assert np.array_equal(ref, mine)


def test_e4m3_saturates():
    assert e4m3_encode(1e6) == 0x7E and e4m3_encode(-1e6) == 0xFE
    assert e4m3_encode(464.0) == 0x7E          # beyond the 448/480 midpoint, still 448
    assert e4m3_encode(np.nan) == 0x7F


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * s for s in (1e-30, 1e-3, 1, 1e3, 1e30)])
    # exact ties: bf16 value plus half its spacing
    base = round_to_bf16_bits(rng.standard_normal(2000).astype(np.float32)).astype(np.float64)
    ties = base + bf16_half_ulp(base) * np.sign(base)
    x = np.concatenate([x, ties]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_half_ulp():
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_half_ulp(3.9) == 2.0 ** -7
    assert bf16_half_ulp(4.0) == 2.0 ** -6
    x = np.random.default_rng(2).standard_normal(10000) * 5
    assert np.all(np.abs(bf16_round(x) - x) <= bf16_half_ulp(x))


def test_generator_bf16_matches_torch():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_to_bf16_bits(x), ref)


def test_generator_is_deterministic_and_shaped():
    w = WORKLOADS["llm_layer_4k"].with_(B=2, H=4, N=70)
    a, b = make_inputs(w), make_inputs(w)
    for key in ("q", "k", "v", "c"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (2, 4, 70, 128) and a["q"].dtype == np.float32
    assert np.all((a["c"] >= 0.5) & (a["c"] <= 2.0))
    assert np.array_equal(round_to_bf16_bits(a["q"]), a["q"])


def test_generator_outliers_and_rotation():
    w = WORKLOADS["fp8_outliers_8k"].with_(B=1, H=3, N=256)
    inp = make_inputs(w)
    R = inp["R"].astype(np.float64)
    assert np.max(np.abs(R @ R.T - np.eye(w.d))) < 1e-5
    ch = inp["outliers"]
    assert ch.shape == (3, 3)
    for t, x in enumerate((inp["q"], inp["k"], inp["v"])):
        for h in range(3):
            col = np.abs(x[0, h, :, ch[t, h]]).mean()
            rest = np.abs(np.delete(x[0, h], ch[t, h], axis=1)).mean()
            assert col > 20 * rest


def test_quantize_tiles_properties():
    """Per-tile scale amax/448; every value within half an e4m3 spacing
    (relative 2^-4, or 2^-10 * s near zero) of its dequantised value; the
    tile's largest magnitude lands exactly on +-448."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((2, 3, 300, 64)) * rng.uniform(0.1, 50, (2, 3, 1, 1))).astype(np.float32)
    codes, s = quantize_tiles(x)
    assert s.shape == (2, 3, 3)
    deq = fp8_dequantize(codes, s)
    srep = np.repeat(s.astype(np.float64), QUANT_TILE, axis=2)[:, :, :300, None]
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, srep * 2.0 ** -10) * 1.0000001)
    for t in range(3):
        blk = x[:, :, t * 128:(t + 1) * 128]
        amax = np.abs(blk).max(axis=(2, 3))
        assert np.array_equal(s[:, :, t], (amax / np.float32(448)).astype(np.float32))
        top = np.abs(e4m3_decode(codes[:, :, t * 128:(t + 1) * 128])).max(axis=(2, 3))
        assert np.all(top == 448.0)


def test_quantize_zero_tile_scale_one():
    codes, s = quantize_tiles(np.zeros((1, 1, 130, 8), np.float32))
    assert np.all(s == 1.0) and np.all(codes == 0)


def test_fp8_prepare_preserves_attention_without_outliers():
    """Rotation + quantisation of outlier-free inputs keeps attention close to
    the unquantised oracle (e4m3 keeps 3 mantissa bits, so each input moves by
    up to 2^-4 relative; a scrambled scale or a rotation of only one of Q, K
    gives errors of order one)."""
    w = WORKLOADS["fp8_outliers_8k"].with_(B=1, H=2, N=256, outlier_frac=0.0)
    inp = make_inputs(w)
    (q8, sq), (k8, sk), (v8, sv) = fp8_prepare(inp["q"], inp["k"], inp["v"], inp["R"])
    oa, _ = attention(inp["q"], inp["k"], inp["v"], w.scale, False)
    ob, _ = attention(fp8_dequantize(q8, sq), fp8_dequantize(k8, sk),
                      fp8_dequantize(v8, sv), w.scale, False)
    assert np.max(np.abs(oa - ob)) < 0.1
    assert np.mean(np.abs(oa - ob)) < 0.01
