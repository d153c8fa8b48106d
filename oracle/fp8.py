"""OCP 8-bit floating point, E4M3FN flavour — oracle codec (test infrastructure).

The pages keep the projected scoring cache in "FP8" (paper summary, §3.4
Projected Scoring Cache) without naming the flavour.  The reading taken here is
the OCP E4M3FN format that gfx950 converts natively (OCP 8-bit Floating Point
Specification v1.0):

  * 1 sign, 4 exponent (bias 7), 3 mantissa bits;
  * normals (1 + m/8) * 2^(e-7) for e in 1..15 (e = 15, m = 7 is NaN);
  * subnormals m * 2^-9 for e = 0;
  * no infinities; largest finite magnitude 448 (S.1111.110);
  * encoding rounds to nearest, ties to even; magnitudes above 448 saturate
    to 448 (saturating conversion mode); NaN in gives NaN out (0x7F/0xFF).
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    out = sign * mag
    out = np.where((e == 15) & ((c & 7) == 7), np.nan, out)
    return out


def encode(x: np.ndarray) -> np.ndarray:
    """fp64 values -> uint8 codes: round to nearest even, saturate to +-448."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.abs(np.where(nan, 0.0, x))
    a = np.minimum(a, MAX_FINITE)  # saturation (448 is representable, so clamp-then-round is exact)
    # exponent of the binade: a = f * 2^ex with f in [0.5, 1) -> unbiased exponent ex-1
    _, ex = np.frexp(a)
    unb = ex - 1
    sub = (a < 2.0 ** -6)
    # subnormal/zero: quantum 2^-9
    q_sub = np.rint(a * 2.0 ** 9)                       # exact scaling, rint = ties-to-even
    # normal: quantum 2^(unb-3)
    unb_n = np.where(sub, 0, unb)
    q_nrm = np.rint(np.ldexp(a, -(unb_n - 3)))          # in [8, 16]
    carry = q_nrm >= 16
    unb_n = np.where(carry, unb_n + 1, unb_n)
    q_nrm = np.where(carry, 8, q_nrm)
    code_n = ((unb_n + 7) << 3) | (q_nrm.astype(np.int64) - 8)
    code_s = q_sub.astype(np.int64)                     # 8 -> 0x08, the smallest normal: correct
    code = np.where(sub, code_s, code_n)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, NAN_CODE, code)
    return code.astype(np.uint8)


def signed_magnitude(codes: np.ndarray) -> np.ndarray:
    """Integer position of a code on the number line (+0 and -0 both map to 0).

    Adjacent representable values differ by exactly 1, so |sm(a) - sm(b)| is the
    distance in units in the last place."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)
