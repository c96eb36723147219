"""fp8 per-token-head KV encoding (test infrastructure only).

The format holds, for every stored token and KV head, D 8-bit floating-point
codes plus one 4-byte float scale, separately for K and for V: the sibling of
the int8 per-token-head format, with the same D + 4 bytes per row (FreeToken
PR #898: the description bullet on the per-token-head formats, and "End to
end", where the E2B unit bytes with either 8-bit format go to 3096 / 6240 and
fp8 raises the page count 2.38x).  The pages print neither the code format nor
the recipe.  This oracle's reading:

* Codes are OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3
  mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no
  infinities; S.1111.111 is NaN, so the largest finite value is 448.
* Per row x (D bf16 values, exact in float32): amax = max_d |x_d|,
  scale = fl32(amax / 448), one IEEE float32 division.  amax == 0: scale 0,
  every code +0.  Otherwise y_d = fl32(x_d / scale) (IEEE float32 division),
  rounded to the nearest E4M3 value with ties to even mantissa; a result
  beyond 448 in magnitude becomes +-448 (saturation; with this scale only a
  rounding of amax itself can get there).
* A code decodes to its E4M3 value times the scale, exactly in float64.

The rounding is written out from the E4M3 definition (exponent and mantissa
grid), not taken from a library; the tests check it against torch's own
float8_e4m3fn conversion over the values where both are defined.
"""

import numpy as np

FP8_MAX = 448.0


def e4m3_value(codes):
    """Exact value of E4M3 codes (uint8), as float64; NaN for the NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = m * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = s * np.where(e == 0, sub, nor)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(y):
    """Nearest E4M3 code of each float (ties to even mantissa), saturating at
    +-448.  y: float32 (or float64) array; NaN is not expected."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    sign = (np.signbit(np.asarray(y, dtype=np.float64))).astype(np.int64) << 7
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range (|y| < 2^-6): multiples of 2^-9; m = 8 is the first normal
    sub = a < 2.0 ** -6
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)
    # normal range: a = f * 2^e with f in [1, 2); the 3-bit mantissa is
    # rint((f - 1) * 8), carrying into the exponent at 8
    mant, ex = np.frexp(np.where(sub, 1.0, a))
    e = ex - 1
    f = mant * 2.0
    q = np.rint((f - 1.0) * 8.0).astype(np.int64)
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    big = (e > 8) | ((e == 8) & (q > 6))
    e = np.where(big, 8, e)
    q = np.where(big, 6, q)
    nor = ((e + 7) << 3) | q
    code = np.where(sub, code, nor)
    # a negative zero keeps its sign bit only for negative inputs that round to 0
    return (code | sign).astype(np.uint8)


def quantise_rows(x):
    """x: [..., D] float32 (bf16 values) -> (codes uint8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.divide(amax, np.float32(FP8_MAX), dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), scale).astype(np.float32)
    y = np.divide(x, safe[..., None], dtype=np.float32)
    codes = e4m3_encode(y)
    codes[zero] = 0
    return codes, scale.astype(np.float32)


def dequantise_rows(codes, scale):
    """Exact float64 value of each stored element: e4m3(code) * scale."""
    return e4m3_value(codes) * np.asarray(scale, dtype=np.float64)[..., None]
