"""Pins for the W4A16 oracle (oracle/w4a16.py) and fp16 rounding.

* fp16_round against numpy's float16 cast (an independent rounding routine),
  including ties, subnormals and overflow;
* the nibble order of a packed word against hand-built words, with a round
  trip on random data;
* dequantisation: closed forms (q = z gives 0; per-group scales land on
  exactly their group's k and their row's n), and the single rounding of
  s (q - z) against numpy's float16 product (fp16 x fp16 is exact in float32,
  then rounded once);
* the product against a pure-Python exact sum (math.fsum) on tiny shapes and
  against a one-hot activation, which must select one weight column.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import w4a16
from seeded_inputs import make_w4a16_inputs


def test_fp16_round_matches_numpy_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000)),
        np.array([65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25,
                  2.0 ** -14, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0, -0.0]),
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    got = oracle.fp16_round(x)
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(want[fin]))


def test_nibble_order_closed_form():
    words = np.array([[0x87654321, 0xF0000000, 0x0000000A]], dtype=np.uint32)
    q = w4a16.unpack_int4(words, 24)
    assert q[0, :8].tolist() == [1, 2, 3, 4, 5, 6, 7, 8]
    assert q[0, 8:16].tolist() == [0] * 7 + [15]
    assert q[0, 16:24].tolist() == [10] + [0] * 7


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    words = w4a16.pack_int4(q)
    assert words.dtype == np.uint32 and words.shape == (5, 8)
    assert np.array_equal(w4a16.unpack_int4(words, 64), q)
    # value i of a word sits in bits 4i..4i+3: read back with Python integers
    for n in range(5):
        for j in range(8):
            hexs = format(int(words[n, j]), "08x")[::-1]
            assert [int(c, 16) for c in hexs] == q[n, 8 * j:8 * j + 8].tolist()


def test_dequantize_closed_forms():
    N, K, G = 3, 32, 8
    rng = np.random.default_rng(2)
    z = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    s = (np.arange(N * (K // G)).reshape(N, K // G) + 1).astype(np.float16) / np.float16(64)
    # q = z everywhere -> all weights exactly zero
    qz = np.repeat(z, G, axis=1)
    assert not np.any(w4a16.dequantize(w4a16.pack_int4(qz), s, z, K, G))
    # q = z + 1 (z < 15) -> every weight equals its own (row, group) scale
    z1 = np.minimum(z, 14).astype(np.uint8)
    q1 = np.repeat(z1 + 1, G, axis=1)
    w = w4a16.dequantize(w4a16.pack_int4(q1), s, z1, K, G)
    for n in range(N):
        for k in range(K):
            assert w[n, k] == float(s[n, k // G])
    # a negative difference: s = 1.5, q - z = -3 -> -4.5
    assert w4a16.dequantize(w4a16.pack_int4(np.full((1, 8), 2, np.uint8)),
                            np.array([[1.5]], np.float16), np.array([[5]], np.uint8), 8, 8)[0, 0] == -4.5


def test_dequantize_rounds_once_like_fp16_product():
    inp = make_w4a16_inputs("w4a16_small")
    q = w4a16.unpack_int4(inp["qweight"], 384)
    diff = (q.astype(np.int16) - np.repeat(inp["zeros"], 128, axis=1).astype(np.int16)).astype(np.float16)
    want = (np.repeat(inp["scales"], 128, axis=1) * diff).astype(np.float64)   # numpy float16 product
    got = w4a16.dequantize(inp["qweight"], inp["scales"], inp["zeros"], 384, 128)
    assert np.array_equal(got, want)
    # scales with long mantissas make the rounding visible
    s = np.array([[1 + 2.0 ** -10, 1.0009765625 + 2.0 ** -9]], dtype=np.float16)
    qq = w4a16.pack_int4(np.array([[15] * 8 + [13] * 8], np.uint8))
    zz = np.array([[0, 2]], np.uint8)
    got = w4a16.dequantize(qq, s, zz, 16, 8)
    want = (np.repeat(s, 8, axis=1) * np.array([[15.0] * 8 + [11.0] * 8], np.float16)).astype(np.float64)
    assert np.array_equal(got, want)
    assert got[0, 0] != float(s[0, 0]) * 15          # the exact product is not an fp16 value


def test_product_against_exact_python_sum():
    rng = np.random.default_rng(3)
    M, N, K, G = 2, 3, 32, 16
    x = rng.standard_normal((M, K)).astype(np.float16)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = rng.uniform(0.01, 0.1, size=(N, K // G)).astype(np.float16)
    z = rng.integers(0, 16, size=(N, K // G)).astype(np.uint8)
    y = w4a16.w4a16_gemm(x, w4a16.pack_int4(q), s, z, G)
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                wk = float(np.float16(float(s[n, k // G]) * (int(q[n, k]) - int(z[n, k // G]))))
                terms.append(float(x[m, k]) * wk)            # exact: fp16 x fp16 fits float64
            exact = math.fsum(terms)
            assert abs(y[m, n] - exact) <= 1e-14 * max(1.0, sum(abs(t) for t in terms))


def test_one_hot_activation_selects_a_weight_column():
    inp = make_w4a16_inputs("w4a16_small")
    K = 384
    w = w4a16.dequantize(inp["qweight"], inp["scales"], inp["zeros"], K, 128)
    for k in (0, 7, 8, 127, 128, 383):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        y = w4a16.w4a16_gemm(x, inp["qweight"], inp["scales"], inp["zeros"], 128)
        assert np.array_equal(y[0], w[:, k])


def test_sampled_rows_and_error_scale():
    inp = make_w4a16_inputs("w4a16_small")
    args = (inp["x"], inp["qweight"], inp["scales"], inp["zeros"], 128)
    y = w4a16.w4a16_gemm(*args)
    cols = np.array([0, 5, 47])
    assert np.array_equal(w4a16.w4a16_rows(*args, cols), y[:, cols])
    sa = w4a16.w4a16_sum_abs(*args)
    assert np.all(np.abs(y) <= sa) and np.all(sa > 0)
    assert np.array_equal(w4a16.w4a16_sum_abs(*args, cols=cols), sa[:, cols])
