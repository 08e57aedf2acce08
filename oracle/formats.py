"""Number formats written from their definitions -- TEST INFRASTRUCTURE ONLY.

* bf16: 1 sign, 8 exponent, 7 fraction bits (float32's exponent range);
  rounding to nearest, ties to the even significand.
* fp16 (IEEE binary16): 1 sign, 5 exponent bits with bias 15, 10 fraction
  bits; subnormals m * 2^-24; largest finite value 65504; rounding to
  nearest, ties to even; magnitudes that round above 65504 become infinite.
* e4m3 ("E4M3FN" of the OCP 8-bit floating-point specification, the format
  the FP8 bullet of "FlashAttention scaling, multi-GPU training and weight
  quantization", section 1, quantises to): 1 sign, 4 exponent bits with bias
  7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; there are
  no infinities; S.1111.111 is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448.  Encoding rounds to nearest, ties to even, and saturates
  magnitudes above 448 to 448 (the reading taken for out-of-range values).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value of x (float64 in, float64 out), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    _, E = np.frexp(ax)                     # ax in [2^(E-1), 2^E)
    e = np.maximum(E - 1, -126)             # below 2^-126 the spacing stays 2^-133
    spacing = np.ldexp(1.0, e - 7)
    r = np.rint(ax / spacing) * spacing     # rint: half-way cases go to the even integer
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    return out


def fp16_round(x) -> np.ndarray:
    """Nearest fp16 value of x (float64 in, float64 out), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    _, E = np.frexp(ax)                     # ax in [2^(E-1), 2^E)
    e = np.maximum(E - 1, -14)              # below 2^-14 the spacing stays 2^-24
    spacing = np.ldexp(1.0, e - 10)
    r = np.rint(ax / spacing) * spacing     # rint: half-way cases go to the even integer
    r = np.where(r > 65504.0, np.inf, r)
    out[fin] = np.copysign(r, x[fin])
    return out


def bf16_half_ulp(x) -> np.ndarray:
    """Half the bf16 spacing in the binade of |x| (the largest rounding error there)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(np.where(ax > 0, ax, 1.0))
    e = np.maximum(E - 1, -126)
    return np.where(ax > 0, np.ldexp(1.0, e - 8), np.ldexp(1.0, -134))


def e4m3_table() -> np.ndarray:
    """Value of every e4m3 code 0..255 (NaN for the two NaN codes)."""
    vals = np.empty(256)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_table()
_POS = _TABLE[:127]                 # codes 0..126: the finite non-negative values, ascending


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of x, ties to even, saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    hi = np.clip(np.searchsorted(_POS, ax, side="left"), 1, 126)
    lo = hi - 1
    d_lo = ax - _POS[lo]
    d_hi = _POS[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(ax >= E4M3_MAX, 126, mag)          # saturate
    mag = np.where(ax <= 0.0, 0, mag)
    code = mag.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
