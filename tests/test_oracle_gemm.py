"""Pins for the oracle's GEMM references (CPU only).

Independent of the oracle's own arithmetic: Python-integer and Fraction sums,
torch's E4M3 decoder, a closed form (identity weights), and a second exact
path (int64 chunk sums) cross-checked against the float64 definition.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import synth
from oracle import bf16, gemm, quantize
from tests._exact import ilog2, round_half_even


def tdec(q):
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def rn_bf16(q: Fraction) -> float:
    """Nearest BF16 to the exact rational q (ties to even)."""
    if q == 0:
        return 0.0
    a = abs(q)
    e = max(ilog2(a), -126)
    ulp = Fraction(2) ** (e - 7)
    v = float(round_half_even(a / ulp) * ulp)
    return v if q > 0 else -v


def integer_codes():
    """E4M3 codes whose values are the integers -16..16 (torch's decoder)."""
    vals = tdec(np.arange(256, dtype=np.uint8))
    keep = [c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
            and abs(vals[c]) <= 16 and c != 0x80]
    assert len(keep) == 33
    return np.array(keep, np.uint8)


def test_exact_integer_gemm_bit_exact():
    rng = np.random.default_rng(0)
    M, N, K = 8, 136, 512
    codes = integer_codes()
    a = rng.choice(codes, (M, K))
    b = rng.choice(codes, (N, K))
    # |sum| <= 4 chunks * 128 * 16 * 16 * 4 = 2^19 on a 2^-1 grid: 20 bits, exact in FP32
    sa = (2.0 ** rng.integers(-1, 2, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(0, 2, (2, K // 128))).astype(np.float32)
    got = gemm.gemm_ref(a, sa, b, sb, "bf16")
    got32 = gemm.gemm_ref(a, sa, b, sb, "f32")
    av = tdec(a).astype(np.int64)
    bv = tdec(b).astype(np.int64)
    for m in range(M):
        for n in range(0, N, 5):
            tot = Fraction(0)
            for kb in range(K // 128):
                sl = slice(kb * 128, kb * 128 + 128)
                p = int(np.dot(av[m, sl], bv[n, sl]))        # exact Python/int64 integer
                tot += p * Fraction(float(sa[kb, m])) * Fraction(float(sb[n // 128, kb]))
            assert bf16.to_f32(got[m, n]) == np.float32(rn_bf16(tot))
            assert float(got32[m, n]) == float(tot)


def test_identity_weights_give_dequantized_activation():
    x = synth.activation(64, 256, seed=3)["a"]
    a, sa = quantize.quantize_1x128(x)
    b = np.zeros((256, 256), np.uint8)
    b[np.arange(256), np.arange(256)] = 0x38                  # 1.0
    sb = np.ones((2, 2), np.float32)
    got = gemm.gemm_ref(a, sa, b, sb, "bf16")
    deq = tdec(a)
    for m in range(0, 64, 3):
        for k in range(0, 256, 11):
            want = rn_bf16(Fraction(float(deq[m, k])) * Fraction(float(sa[k // 128, m])))
            assert float(bf16.to_f32(got[m, k])) == want


def test_fraction_brute_force_small():
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    a = rng.choice(finite, (2, 256))
    b = rng.choice(finite, (2, 256))
    sa = rng.uniform(1e-3, 2.0, (2, 2)).astype(np.float32)
    sb = rng.uniform(1e-3, 2.0, (1, 2)).astype(np.float32)
    got = gemm.gemm_ref(a, sa, b, sb, "bf16")
    got32 = gemm.gemm_ref(a, sa, b, sb, "f32")
    exact2 = gemm.chunk_sums_exact(a, sa, b, sb)
    av, bv = tdec(a), tdec(b)
    for m in range(2):
        for n in range(2):
            tot = sum(Fraction(float(av[m, k])) * Fraction(float(sa[k // 128, m]))
                      * Fraction(float(bv[n, k])) * Fraction(float(sb[0, k // 128])) for k in range(256))
            assert float(bf16.to_f32(got[m, n])) == rn_bf16(tot)
            assert abs(Fraction(float(got32[m, n])) - tot) <= abs(tot) * Fraction(1, 2 ** 24)
            assert abs(Fraction(float(exact2[m, n])) - tot) <= abs(tot) * Fraction(1, 2 ** 50)


def test_two_exact_paths_agree_on_workload_recipe():
    w = synth.dense(64, 200, 512, seed=6)
    a, sa = quantize.quantize_1x128(w["a"])
    b, sb = quantize.quantize_128x128(w["b"])
    d1 = gemm.gemm_f64(a, sa, b, sb)
    d2 = gemm.chunk_sums_exact(a, sa, b, sb)
    assert np.max(np.abs(d1 - d2)) <= 1e-12 * np.max(np.abs(d1))
    rows = np.array([0, 5, 63, 17])
    cols = np.array([199, 0, 128, 127])
    assert np.allclose(gemm.gemm_sample_f64(a, sa, b, sb, rows, cols), d1[rows, cols], rtol=1e-14, atol=0)
    blk = gemm.gemm_block_f64(a, sa, b, sb, rows, cols)
    assert np.allclose(blk, d1[np.ix_(rows, cols)], rtol=1e-14, atol=0)


def test_grouped_contiguous_is_dense_per_group():
    w = synth.contiguous(4, 512, 96, 256, seed=8)
    offs = w["m_offsets"]
    a, sa = quantize.quantize_1x128(w["a"])
    b, sb = quantize.quantize_128x128(w["b"])
    d = gemm.grouped_contiguous_f64(a, sa, b, sb, offs)
    assert offs[0] == 0 and offs[-1] == 512 and np.all(np.diff(offs) % 128 == 0)
    for g in range(4):
        lo, hi = offs[g], offs[g + 1]
        if hi > lo:
            np.testing.assert_array_equal(d[lo:hi], gemm.gemm_f64(a[lo:hi], sa[:, lo:hi], b[g], sb[g]))
    # zero-size groups and rows past the last offset
    offs2 = np.array([0, 0, 256, 256, 384], np.int32)
    d2 = gemm.grouped_contiguous_f64(a, sa, b, sb, offs2)
    np.testing.assert_array_equal(d2[:256], gemm.gemm_f64(a[:256], sa[:, :256], b[1], sb[1]))
    np.testing.assert_array_equal(d2[256:384], gemm.gemm_f64(a[256:384], sa[:, 256:384], b[3], sb[3]))
    assert np.isnan(d2[384:]).all()


def test_grouped_masked_counts():
    w = synth.masked(3, 256, 64, 256, seed=10)
    G, cap, K = w["a"].shape
    a, sa = quantize.quantize_1x128(w["a"].reshape(G * cap, K))
    a = a.reshape(G, cap, K)
    sa = np.stack([sa[:, g * cap:(g + 1) * cap] for g in range(G)])
    b, sb = quantize.quantize_128x128(w["b"])
    counts = np.array([0, 256, 77], np.int32)
    d = gemm.grouped_masked_f64(a, sa, b, sb, counts)
    assert np.isnan(d[0]).all()
    np.testing.assert_array_equal(d[1], gemm.gemm_f64(a[1], sa[1], b[1], sb[1]))
    np.testing.assert_array_equal(d[2, :77], gemm.gemm_f64(a[2, :77], sa[2][:, :77], b[2], sb[2]))
    assert np.isnan(d[2, 77:]).all()


# ---- weight-gradient reference ---------------------------------------------

def test_wgrad_fraction_brute_force_small():
    # both operands scaled per row and per 128 K; exact rational sums
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, N, K = 3, 2, 384
    a = rng.choice(finite, (M, K))
    b = rng.choice(finite, (N, K))
    sa = rng.uniform(1e-3, 2.0, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(1e-3, 2.0, (K // 128, N)).astype(np.float32)
    d_in = rng.standard_normal((M, N)).astype(np.float32)
    got = gemm.wgrad_ref(a, sa, b, sb)
    got_acc = gemm.wgrad_ref(a, sa, b, sb, d_in)
    av, bv = tdec(a), tdec(b)
    for m in range(M):
        for n in range(N):
            tot = sum(Fraction(float(av[m, k])) * Fraction(float(sa[k // 128, m]))
                      * Fraction(float(bv[n, k])) * Fraction(float(sb[k // 128, n])) for k in range(K))
            assert abs(Fraction(float(got[m, n])) - tot) <= abs(tot) * Fraction(1, 2 ** 24)
            tot_acc = tot + Fraction(float(d_in[m, n]))
            assert abs(Fraction(float(got_acc[m, n])) - tot_acc) <= abs(tot_acc) * Fraction(1, 2 ** 24)


def test_wgrad_exact_integer_sums():
    # integer-valued codes, power-of-two scales: Python-integer sums are exact
    rng = np.random.default_rng(12)
    ints = integer_codes()
    M, N, K = 5, 7, 256
    a = rng.choice(ints, (M, K))
    b = rng.choice(ints, (N, K))
    sa = (2.0 ** rng.integers(-3, 3, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-3, 3, (K // 128, N))).astype(np.float32)
    av, bv = tdec(a).astype(np.int64), tdec(b).astype(np.int64)
    got = gemm.wgrad_ref(a, sa, b, sb)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // 128):
                chunk = int(sum(int(av[m, k]) * int(bv[n, k]) for k in range(kb * 128, kb * 128 + 128)))
                tot += chunk * Fraction(float(sa[kb, m])) * Fraction(float(sb[kb, n]))
            assert Fraction(float(got[m, n])) == tot          # |sum| < 2^24: exact in FP32


def test_wgrad_transposed_scale_layout_is_distinct():
    # a transposed sB (the [rows][K/128] layout) changes the result: the
    # reference reads sB as [K/128][N]
    rng = np.random.default_rng(13)
    ints = integer_codes()
    a = rng.choice(ints, (4, 256))
    b = rng.choice(ints, (2, 256))
    sa = np.ones((2, 4), np.float32)
    sb = np.array([[1.0, 2.0], [4.0, 8.0]], np.float32)     # [K/128][N]
    ref = gemm.wgrad_f64(a, sa, b, sb)
    av, bv = tdec(a), tdec(b)
    expect = np.zeros((4, 2))
    for kb in range(2):
        sl = slice(kb * 128, kb * 128 + 128)
        expect += (av[:, sl] @ bv[:, sl].T) * sb[kb][None, :]
    assert np.array_equal(ref, expect)
    assert not np.array_equal(gemm.wgrad_f64(a, sa, b, sb.T.copy()), expect)
