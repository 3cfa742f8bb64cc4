"""Pins for the oracle's E4M3 and BF16 codecs (CPU only).

Independent sources: torch's own float8_e4m3fn and bfloat16 casts (library
routines), a value table enumerated here from the OCP E4M3 definition with
exact Fractions, and brute-force nearest-code searches.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3

ALL = np.arange(256, dtype=np.uint8)
NAN_CODES = {0x7F, 0xFF}
FINITE = np.array([c for c in range(256) if c not in NAN_CODES], dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(x_f32):
    return torch.from_numpy(np.asarray(x_f32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fraction_table():
    """Value of every finite code from the OCP E4M3 definition, as Fractions."""
    out = {}
    for c in FINITE.tolist():
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out[c] = -mag if s else mag
    return out


def test_decode_matches_torch_all_codes():
    ours = e4m3.decode(ALL)
    ref = torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert set(np.flatnonzero(np.isnan(ours)).tolist()) == NAN_CODES
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_matches_fraction_table():
    tab = fraction_table()
    ours = e4m3.decode(FINITE)
    for c, v in zip(FINITE.tolist(), ours.tolist()):
        assert Fraction(v) == tab[c], hex(c)


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6),
                                        (0x01, 2.0 ** -9), (0x38, 1.0), (0x07, 7 * 2.0 ** -9),
                                        (0x00, 0.0), (0x77, 240.0)])
def test_decode_named_codes(code, value):
    assert e4m3.decode(np.array([code], np.uint8))[0] == value


def test_decode_negative_zero():
    v = e4m3.decode(np.array([0x80], np.uint8))[0]
    assert v == 0.0 and np.signbit(v)


def test_encode_roundtrips_every_finite_code():
    vals = e4m3.decode(FINITE).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), FINITE)


def _brute_force_encode(x64):
    """Nearest finite code of the same sign (ties -> even code), |x| > 448 -> 448."""
    tab = torch_decode(np.arange(0, 0x7F, dtype=np.uint8))  # non-negative finite codes, library values
    mag = np.abs(x64)
    dist = np.abs(mag[:, None] - tab[None, :])
    best = np.argmin(dist, axis=1)                            # first (smaller) code on ties
    dmin = dist[np.arange(len(mag)), best]
    nxt = np.minimum(best + 1, 0x7E)
    tie = (nxt != best) & (dist[np.arange(len(mag)), nxt] == dmin)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    best = np.where(mag > 448.0, 0x7E, best)
    return (best | (np.signbit(x64).astype(np.int64) << 7)).astype(np.uint8)


def test_encode_exhaustive_bf16_vs_brute_force():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16.to_f32(bits)
    fin = np.isfinite(x)
    ours = e4m3.encode(x[fin])
    ref = _brute_force_encode(x[fin].astype(np.float64))
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, [(float(x[fin][i]), ours[i], ref[i]) for i in bad[:5]]


def test_encode_midpoints_and_neighbours():
    vals = torch_decode(np.arange(0, 0x7F, dtype=np.uint8))
    lo, hi = vals[:-1], vals[1:]
    mid = ((lo + hi) / 2).astype(np.float32)                  # exact in float32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    codes = np.arange(0, 0x7E)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(e4m3.encode(mid), even.astype(np.uint8))
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(e4m3.encode(up), (codes + 1).astype(np.uint8))
    assert np.array_equal(e4m3.encode(dn), codes.astype(np.uint8))
    assert np.array_equal(e4m3.encode(-mid), (even | 0x80).astype(np.uint8))


def test_encode_matches_torch_below_overflow():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464.0)]
    # add many values in the interesting range [2^-12, 464)
    y = (rng.random(2_000_000) * 2.0 ** rng.integers(-12, 9, 2_000_000)).astype(np.float32)
    y = np.concatenate([x, y, -y])
    assert np.array_equal(e4m3.encode(y), torch_encode(y))


@pytest.mark.parametrize("v,code", [(448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E),
                                    (1e9, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE), (-1e30, 0xFE),
                                    (2.0 ** -10, 0x00), (-2.0 ** -10, 0x80), (3 * 2.0 ** -10, 0x02),
                                    (-0.0, 0x80), (2.0 ** -30, 0x00), (np.nan, 0x7F)])
def test_encode_special_values(v, code):
    assert e4m3.encode(np.array([v], np.float32))[0] == code


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16.to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_rne_matches_torch_on_float32_inputs():
    # For float32-representable inputs torch's float32 -> bfloat16 cast is one RNE rounding.
    rng = np.random.default_rng(2)
    x = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16.from_f64_rne(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_rne_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-40 lies just above a BF16 midpoint; rounding it to float32
    # first would drop the 2^-40 and tie to even (down).  One rounding goes up.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)])
    got = bf16.to_f32(bf16.from_f64_rne(x)).astype(np.float64)
    assert got.tolist() == [1 + 2.0 ** -7, 1.0, 1 + 2 * 2.0 ** -7, -(1 + 2.0 ** -7)]
    # brute force over Fractions on random doubles: nearest BF16, ties to even
    rng = np.random.default_rng(3)
    v = rng.standard_normal(2000) * 2.0 ** rng.integers(-20, 20, 2000)
    out = bf16.to_f32(bf16.from_f64_rne(v)).astype(np.float64)
    for xi, oi in zip(v.tolist(), out.tolist()):
        f, e = np.frexp(xi)
        ulp = Fraction(2) ** (int(e) - 8)
        q = Fraction(xi) / ulp
        fl = q.numerator // q.denominator
        r = q - fl
        n = fl + (1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2) else 0)
        assert Fraction(oi) == n * ulp
