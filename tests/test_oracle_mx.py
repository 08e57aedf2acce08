"""Pins for the MXFP8 oracle (oracle/mx.py).

* the scale exponent at closed-form points (powers of two times 448, just
  above and below them, zero, subnormal and huge amax);
* no saturation and full use of the top binade: for every block with
  amax > 0, amax / 2^e lies in (224, 448];
* element codes against torch's float8_e4m3fn cast of x / 2^e (an
  independent encoder; no value exceeds 448, so its out-of-range rule never
  applies);
* the round-trip error bound of e4m3 (2^-4 relative in the normal range, half
  a subnormal step 2^-10 * 2^e below it);
* blocks run along channels of one token (a block-per-token reading would
  fail the per-block exponent check), and the rotated Q K^T is unchanged.
"""
import numpy as np
import pytest

import oracle
import oracle.fp8
from oracle import mx


@pytest.mark.parametrize("amax,e", [
    (448.0, 0), (449.0, 1), (447.0, 0), (224.0, -1), (224.5, 0), (896.0, 1), (896.5, 2),
    (1.0, -8), (0.875, -9), (0.875 * 1.0001, -8), (0.0, -127), (1e-45, -127),
    (3.0e38, 120), (448.0 * 2.0 ** -130, -127),
])
def test_exponent_closed_forms(amax, e):
    assert int(mx.mx_exponent(np.float32(amax))) == e


def test_every_block_fills_the_top_binade_without_saturating():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((3, 5, 64)) * np.exp(rng.uniform(-20, 20, (3, 5, 1)))).astype(np.float32)
    codes, sc = mx.quantize_mx(x)
    e = sc.astype(np.int64) - mx.E8M0_BIAS
    blocks = np.abs(x.reshape(3, 5, 2, 32).astype(np.float64))
    ratio = blocks.max(axis=-1) / np.ldexp(1.0, e)
    assert (ratio > 224).all() and (ratio <= 448).all()
    assert (codes & 0x7F).max() <= 0x7E          # never the NaN code


def test_codes_match_torch_e4m3_cast():
    import torch
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((4, 7, 128)) * rng.uniform(0.01, 50, (4, 7, 1))).astype(np.float32)
    x[0, 0, :32] = 0.0                           # an all-zero block
    x[1, 1, 40] = 1e-30                          # a tiny value next to ordinary ones
    codes, sc = mx.quantize_mx(x)
    e = np.repeat(sc.astype(np.int64) - mx.E8M0_BIAS, 32, axis=-1)
    scaled = torch.from_numpy((x.astype(np.float64) / np.ldexp(1.0, e)).astype(np.float32))
    ref = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)


def test_round_trip_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 256)) * 3).astype(np.float32)
    x[2, 5] = 80.0                               # an outlier inside one block
    codes, sc = mx.quantize_mx(x)
    deq = mx.dequantize_mx(codes, sc)
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - mx.E8M0_BIAS), 32, axis=-1)
    ax = np.abs(x.astype(np.float64))
    normal = ax / X >= 2.0 ** -6
    err = np.abs(deq - x)
    assert (err[normal] <= 2.0 ** -4 * ax[normal] * (1 + 1e-12)).all()
    assert (err[~normal] <= 2.0 ** -10 * X[~normal] * (1 + 1e-12)).all()
    # the outlier's block is coarse, the other blocks of that row are not
    blk = 5 // 32
    assert sc[2, blk] > sc[2, blk + 1]


def test_blocks_are_along_channels():
    x = np.ones((2, 64), dtype=np.float32)
    x[0, :32] *= 100.0                           # token 0, first block only
    _, sc = mx.quantize_mx(x)
    assert sc[0, 0] != sc[0, 1] and sc[0, 1] == sc[1, 0] == sc[1, 1]


def test_prepare_rotates_q_and_k_only():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2, 40, 64)).astype(np.float32) for _ in range(3))
    G = rng.standard_normal((64, 64))
    from seeded_inputs import haar_orthogonal
    R = haar_orthogonal(G).astype(np.float32)
    (q8, qs), (k8, ks), (v8, vs) = mx.mxfp8_prepare(q, k, v, R)
    np.testing.assert_array_equal(v8, mx.quantize_mx(v)[0])
    qd, kd = mx.dequantize_mx(q8, qs), mx.dequantize_mx(k8, ks)
    qr, kr = (oracle.fp8.rotate(x, R).astype(np.float64) for x in (q, k))
    # rotation leaves Q K^T unchanged (up to the float32 rounding of x R)
    s_ref = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    s_rot = np.einsum("bhid,bhjd->bhij", qr, kr)
    assert np.abs(s_rot - s_ref).max() < 1e-4 * np.abs(s_ref).max()
    # quantised scores within the element-wise e4m3 bound of both factors
    def emax(x, sc):
        X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - mx.E8M0_BIAS), 32, axis=-1)
        return 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * X
    dq_, dk_ = emax(qr, qs), emax(kr, ks)
    bound = (np.einsum("bhid,bhjd->bhij", dq_, np.abs(kr)) + np.einsum("bhid,bhjd->bhij", np.abs(qr), dk_)
             + np.einsum("bhid,bhjd->bhij", dq_, dk_))
    s_q = np.einsum("bhid,bhjd->bhij", qd, kd)
    assert (np.abs(s_q - s_rot) <= bound * (1 + 1e-9) + 1e-12).all()
