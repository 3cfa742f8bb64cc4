"""Pins for the limited-accumulation emulator (CPU only).

What fixes these values: page 1's claim that ~14-bit accumulation gives a
maximum relative error near 2% at K = 4096 and grows with K, and that
promotion to FP32 fixes it; plus hand-worked cases of the truncation rule.
"""

import json
import os

import numpy as np

from oracle import accum_emu, e4m3, quantize

CLAIMS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_claims.json")))["accumulation"]


def per_tensor_fp8(x32):
    s = quantize.tile_scale(np.max(np.abs(x32)), False)
    q = quantize.quantize_values(x32, s)
    return e4m3.decode(q), float(s)


def emulated_errors(K, seed=0, MN=32):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((MN, K)).astype(np.float32)
    b = rng.standard_normal((MN, K)).astype(np.float32)
    av, _ = per_tensor_fp8(a)
    bv, _ = per_tensor_fp8(b)
    p = accum_emu.products(av, bv)
    exact = np.sum(p, axis=-1)
    nop = accum_emu.limited_accumulate(p, bits=CLAIMS["bits_retained"], promote_every=None)
    pro = accum_emu.limited_accumulate(p, bits=CLAIMS["bits_retained"], promote_every=128)
    return accum_emu.max_relative_error(nop, exact), accum_emu.max_relative_error(pro, exact)


def test_no_promotion_error_is_of_the_reported_order_and_promotion_removes_it():
    K, claimed = CLAIMS["at_K"], CLAIMS["max_relative_error_without_promotion"]
    nop4096, pro4096 = emulated_errors(K)
    nop512, _ = emulated_errors(512)
    assert claimed / 4 <= nop4096 <= claimed * 5   # same order as the pages' figure
    assert nop512 < nop4096                    # grows with K
    assert pro4096 * 10 <= nop4096             # promotion every 128 removes it


def test_truncation_rule_by_hand():
    # largest term 2^14 + 1 -> leading bit 14 -> lsb 1: -0.75 truncates to -1, 0.75 to 0
    p = np.array([[2.0 ** 14 + 1, -0.75] + [0.0] * 30])
    assert accum_emu.limited_accumulate(p)[0] == 2.0 ** 14
    p = np.array([[2.0 ** 14 + 1, 0.75] + [0.0] * 30])
    assert accum_emu.limited_accumulate(p)[0] == 2.0 ** 14 + 1
    # the accumulator takes part in the alignment: a big running sum swallows small terms
    p = np.array([[2.0 ** 20] + [0.0] * 31 + [1.0] * 32])
    assert accum_emu.limited_accumulate(p)[0] == 2.0 ** 20   # lsb = 2^6 in group 2
    # with a fresh chain every 32 (promotion) they survive
    assert accum_emu.limited_accumulate(p, promote_every=32)[0] == 2.0 ** 20 + 32


def test_small_integer_sums_are_unaffected():
    rng = np.random.default_rng(1)
    p = rng.integers(-8, 9, (16, 1024)).astype(np.float64)
    assert np.max(np.abs(np.cumsum(p, axis=1))) < 2 ** 14
    np.testing.assert_array_equal(accum_emu.limited_accumulate(p), p.sum(axis=1))
    np.testing.assert_array_equal(accum_emu.limited_accumulate(p, promote_every=128), p.sum(axis=1))
