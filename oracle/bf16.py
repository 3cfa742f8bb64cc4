"""BF16 helpers for the oracle.  Test infrastructure only.

BF16 is binary32 with the low 16 mantissa bits dropped: 1 sign, 8 exponent,
7 stored mantissa bits.  Arrays of BF16 are carried as uint16 bit patterns.
Page 1 (the uniondaocoop.com post on FP8 mixed-precision training) names BF16
as one of the two output precisions of the FP8 GEMMs; the reading taken for
the rounding is round-to-nearest, ties to even, applied once to the exact
(float64) result.
"""

import numpy as np


def to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def from_f64_rne(x) -> np.ndarray:
    """float64 values -> BF16 bit patterns, one rounding, ties to even.

    Normal range: write x = f * 2^e with 0.5 <= |f| < 1 (frexp), round
    f * 2^8 to an integer (8 significant bits), scale back.  Below 2^-126 the
    BF16 spacing is 2^-133.  Results that round beyond the largest finite BF16
    become infinity.  NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)
    tiny = np.abs(x) < 2.0 ** -126
    r = np.where(tiny, np.ldexp(np.rint(np.ldexp(x, 133)), -133), r)
    r = np.where(np.isnan(x), np.nan, r)
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)                         # exact: r fits BF16
    return (np.ascontiguousarray(r32).view(np.uint32) >> 16).astype(np.uint16)
