"""Exhaustive GPU parity sweeps of the quantizers' arithmetic against the CPU
oracle (bit-exact):

- one 1x128 tile for every positive finite BF16 amax (and the zero tile),
  through the 1x128 and the dual quantizer, with FP32 and power-of-two
  scales.  The scale s = fl32(amax / 448) rounds down for about half of the
  amax values, which puts the tile maximum's quotient just above 448: the
  encoder must still give 448 there.  The tiles' other values span
  [-amax, amax] down to the BF16 subnormals, so the kernels' division (one
  reciprocal per tile, a product and one correction step, tiles below 2^-60
  scaled by 2^64) meets every amax with small and large quotients.
- the elementwise E4M3 cast on every one of the 2^32 FP32 bit patterns
  (the encoding: page 4, "Deepseek veroeffentlicht Deepgemm", section
  "Was ist fp8?", names E4M3; OCP format, round to nearest even, saturating).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs
from oracle import e4m3, quantize
from tests.gpu_util import assert_codes_equal, bf16_dev, codes_host, f32_bits_host, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def bf16_of_f32(v):
    """float32 values -> BF16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def amax_sweep_tiles():
    """[4096, 1024] BF16 bits: 32768 tiles of 128; tile i < 32639 has amax
    BF16 bits i + 1, tile 32639 is all zeros, the rest are random."""
    rng = np.random.default_rng(21)
    n_amax = 0x7F7F
    tiles = np.zeros((32768, 128), np.uint16)
    a_bits = np.arange(1, n_amax + 1, dtype=np.uint16)
    a = (a_bits.astype(np.uint32) << 16).view(np.float32)
    # random magnitudes at most amax, uniform over the bit patterns (every
    # exponent down to the subnormals), random signs
    mag = (rng.random((n_amax, 128)) * (a_bits[:, None].astype(np.float64) + 1)).astype(np.uint16)
    mag = np.minimum(mag, a_bits[:, None])
    sign = rng.integers(0, 2, (n_amax, 128)).astype(np.uint16) << 15
    t = mag | sign
    # fixed members: amax at a position that moves with the tile, -amax,
    # +-amax/2, +-amax * 3/7 (a quotient near 192), the smallest subnormals
    idx = np.arange(n_amax)
    pos = idx % 128
    t[idx, pos] = a_bits
    others = np.stack([bf16_of_f32(-a), bf16_of_f32(a * 0.5), bf16_of_f32(-a * 0.5),
                       bf16_of_f32(a * (3.0 / 7.0)), np.ones(n_amax, np.uint16), np.full(n_amax, 0x8001, np.uint16)],
                      axis=1)
    # keep them at most amax in magnitude (the rounding of amax * 3/7 or of
    # the subnormal 1 can exceed a tiny amax)
    others_mag = others & 0x7FFF
    others = np.where(others_mag <= a_bits[:, None], others, others & 0x8000)
    for j in range(others.shape[1]):
        p = (pos + 1 + j) % 128
        t[idx, p] = others[:, j]
    tiles[:n_amax] = t
    # tile n_amax: zeros (amax = 0, s = 1); the remaining tiles: random values
    tiles[n_amax + 1:] = bf16_of_f32(rng.standard_normal((32768 - n_amax - 1, 128)).astype(np.float32))
    return tiles.reshape(4096, 1024), a


@pytest.mark.parametrize("pow2", [False, True])
def test_every_bf16_amax_1x128_and_dual(pow2):
    print(f"amax sweep pow2={pow2}", flush=True)
    x, a = amax_sweep_tiles()
    if not pow2:
        # the sweep reaches quotients above 448: scales that rounded down
        s = (a / np.float32(448.0)).astype(np.float32)
        assert np.count_nonzero(a.astype(np.float64) / s.astype(np.float64) > 448.0) > 10000
    q, s = fp8bs.quantize_1x128(bf16_dev(x), pow2)
    torch.cuda.synchronize()
    q_ref, s_ref = quantize.quantize_1x128(x, pow2)
    assert_codes_equal(codes_host(q), q_ref, "amax sweep 1x128 codes")
    assert_codes_equal(f32_bits_host(s), s_ref.view(np.uint32), "amax sweep 1x128 scales")
    # the dual quantizer: the same 1x128 tiles, and 128x1 tiles of the same values
    q2, s2, qt, st = fp8bs.quantize_dual(bf16_dev(x), pow2)
    torch.cuda.synchronize()
    rq, rs, rqt, rst = quantize.quantize_dual(x, pow2)
    assert_codes_equal(codes_host(q2), rq, "amax sweep dual 1x128 codes")
    assert_codes_equal(f32_bits_host(s2), rs.view(np.uint32), "amax sweep dual 1x128 scales")
    assert_codes_equal(codes_host(qt), rqt, "amax sweep dual 128x1 codes")
    assert_codes_equal(f32_bits_host(st), rst.view(np.uint32), "amax sweep dual 128x1 scales")


CHUNK = 1 << 28
SUB = 1 << 22


def encode_range(start, n):
    """oracle codes of the FP32 bit patterns start .. start+n-1, threaded"""
    def one(i):
        lo = start + i * SUB
        bits = np.arange(lo, lo + SUB, dtype=np.uint64).astype(np.uint32)
        return e4m3.encode(bits.view(np.float32))
    workers = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        return np.concatenate(list(ex.map(one, range(n // SUB))))


@pytest.mark.slow
@pytest.mark.parametrize("chunk", range(16))
def test_cast_every_fp32_bit_pattern(chunk):
    start = chunk * CHUNK
    print(f"cast sweep bits {start:#010x} .. {start + CHUNK - 1:#010x}", flush=True)
    v = torch.arange(start, start + CHUNK, dtype=torch.int64, device="cuda")
    v = torch.where(v >= 2 ** 31, v - 2 ** 32, v).to(torch.int32).view(torch.float32)
    q = codes_host(fp8bs.cast_to_e4m3(v))
    del v
    torch.cuda.synchronize()
    ref = encode_range(start, CHUNK)
    assert_codes_equal(q, ref, f"cast chunk {chunk}")
