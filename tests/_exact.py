"""Exact-arithmetic helpers for oracle pins (Fractions; no oracle code)."""

from fractions import Fraction

import numpy as np
import torch


def ilog2(a: Fraction) -> int:
    """floor(log2(a)) for a positive Fraction, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    r = q - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2):
        fl += 1
    return fl


def rn32(q: Fraction) -> float:
    """Nearest binary32 to the exact rational q (ties to even), as a float."""
    if q == 0:
        return 0.0
    a = abs(q)
    e = max(ilog2(a), -126)
    ulp = Fraction(2) ** (e - 23)
    v = round_half_even(a / ulp) * ulp
    return float(v) if q > 0 else -float(v)


def e4m3_table() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0..0x7E (torch's decoder)."""
    return torch.from_numpy(np.arange(0, 0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def nearest_code(y: float, table=None) -> int:
    """Nearest E4M3 code to float y, same sign, ties to the even code,
    magnitudes above 448 saturate to 448."""
    tab = e4m3_table() if table is None else table
    m = abs(y)
    if m > 448.0:
        c = 0x7E
    else:
        d = np.abs(tab - m)
        c = int(np.argmin(d))
        if c + 1 <= 0x7E and d[c + 1] == d[c] and c % 2 == 1:
            c += 1
    return c | (0x80 if np.signbit(y) else 0)


def tile_scale_exact(amax: float, pow2: bool) -> float:
    """Scale of a tile from exact arithmetic: nearest float32 to amax/448
    (1 for a zero tile, at least 2^-149 for a nonzero one), rounded up to a
    power of two on request."""
    if amax == 0:
        return 1.0
    s = max(rn32(Fraction(amax) / 448), 2.0 ** -149)
    if pow2:
        e = ilog2(Fraction(s))
        if Fraction(2) ** e != Fraction(s):
            e += 1
        s = float(Fraction(2) ** e)
    return s
