"""OCP E4M3 ("FN" variant) codec by bit manipulation.  Test infrastructure only.

Format (OCP 8-bit floating point specification; the surveyed pages only name
"E4M3" next to "E5M2" in page 4's section "Was ist fp8?"): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits.  There are no infinities; codes
0x7F and 0xFF are NaN, so the largest finite magnitude is 0x7E = 1.75 * 2^8 =
448.  Exponent field 0 holds subnormals m * 2^-9.

Reading taken where the pages are silent: encoding rounds to nearest with ties
to even (RNE) and saturates finite overflow (and +-inf) to +-448 ("satfinite");
the sign is kept for zero and for values that underflow to zero; NaN maps to
the NaN code of the same sign.
"""

import numpy as np

E4M3_MAX = 448.0


def decode(codes) -> np.ndarray:
    """E4M3 code bytes -> float64 values (exact).  NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c >> 7) == 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    subnormal = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(neg, -mag, mag)


def encode(y) -> np.ndarray:
    """binary32 values -> E4M3 code bytes (RNE, satfinite), on the float's bits.

    Normal range (|y| >= 2^-6): rebias the binary32 exponent (127 -> 7) and
    round the 23-bit mantissa to 3 bits, ties to even; a carry out of the
    mantissa moves into the exponent.  Subnormal range: |y| * 2^9 rounded to an
    integer, ties to even (that integer is the code, and 8 is the smallest
    normal code).  Anything that rounds past 0x7E saturates to 0x7E.
    """
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    bits = y.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) << 7
    a = bits & 0x7FFFFFFF
    exp32 = a >> 23
    man = a & 0x7FFFFF

    keep = man >> 20
    rem = man & 0xFFFFF
    half = 0x80000
    up = (rem > half) | ((rem == half) & ((keep & 1) == 1))
    code_normal = ((exp32 - 120) << 3) + keep + up.astype(np.int64)

    # Only subnormal-range inputs are widened: a signalling NaN would raise
    # the invalid flag in the float32 -> float64 conversion.
    small = np.where(exp32 < 121, y, np.float32(0.0))
    scaled = np.abs(small.astype(np.float64)) * 512.0      # exact
    code_sub = np.rint(scaled).astype(np.int64)

    code = np.where(exp32 >= 121, code_normal, code_sub)
    code = np.minimum(code, 0x7E)                          # satfinite, +-inf
    code = np.where(a > 0x7F800000, 0x7F, code)            # NaN
    return (code | sign).astype(np.uint8)
