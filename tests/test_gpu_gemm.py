"""GPU parity of the dense block-scaled GEMM against the CPU oracle.

Inputs: the seeded workload recipe quantized by the oracle (the same bytes go
to both sides).  Bar: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) elementwise,
ref = float64 definition rounded once to the output dtype; bit-exact when the
exact result is representable in FP32 at every step (exact-integer inputs).
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import bf16, e4m3, gemm, quantize
from tests.gpu_util import (assert_codes_equal, assert_gemm_close, codes_dev, dense_allowance, f32_dev, out_host_f64,
                            require_gpu)

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def operands(M, N, K, seed, pow2=False):
    w = synth.dense(M, N, K, seed=seed)
    a, sa = quantize.quantize_1x128(w["a"], pow2)
    b, sb = quantize.quantize_128x128(w["b"], pow2)
    return a, sa, b, sb


def run(a, sa, b, sb, out_dtype=torch.bfloat16):
    d = fp8bs.gemm(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 16, 128), (37, 48, 384), (130, 2112, 256),
                                   (256, 272, 1024), (64, 4096, 128), (300, 400, 640), (513, 144, 1152),
                                   # enough 256x256 tiles for the large-tile path; ragged edges,
                                   # then ragged rows (4000 = 15.6 tiles) on it
                                   (4096, 4096, 256), (4000, 7168, 256),
                                   # the 192x192 tile (ragged edges), then the 256x160 tile
                                   (4000, 4112, 384), (2304, 4096, 256), (2560, 3584, 384),
                                   # few rows: the 64x64 tile (two row tiles, the second ragged;
                                   # ragged columns), then 128x96 (ragged rows and columns)
                                   (100, 208, 1152), (100, 13328, 384),
                                   # the 64x64 tile up to 512 rows, at its 512-tile limit
                                   (384, 4096, 7168), (512, 4096, 2048)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_workload_recipe(M, N, K, out_dtype):
    print(f"gemm M={M} N={N} K={K} out={out_dtype}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + 7 * N + K)
    d = run(a, sa, b, sb, out_dtype)
    ref = gemm.gemm_f64(a, sa, b, sb)
    ref = (bf16.to_f32(gemm.round_out(ref, "bf16")) if out_dtype == torch.bfloat16
           else gemm.round_out(ref, "f32")).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, f"gemm {M}x{N}x{K}", dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N,K", [(256, 272, 1024),
                                   # 192x192 and 256x160 tiles: a wave's columns straddle two
                                   # weight blocks
                                   (4000, 4112, 256), (2560, 3584, 256),
                                   # the 64x64 and 128x96 tiles of few-row shapes, then the
                                   # 128x128 tile (past 512 rows) and 64x64 with ragged rows
                                   (100, 208, 640), (100, 13328, 256), (513, 144, 1152), (300, 400, 640)])
def test_gemm_exact_integer_inputs_bit_exact(M, N, K, out_dtype):
    # codes with integer values in [-16, 16] and power-of-two scales: every
    # partial sum is exact in FP32, so the output is the one rounding of the
    # exact result.
    print(f"exact-integer gemm M={M} N={N} K={K} out={out_dtype}", flush=True)
    rng = np.random.default_rng(0)
    vals = e4m3.decode(np.arange(256, dtype=np.uint8))
    ints = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
                     and abs(vals[c]) <= 16 and c != 0x80], np.uint8)
    a = rng.choice(ints, (M, K)).astype(np.uint8)
    b = rng.choice(ints, (N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-2, 2, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-2, 2, ((N + 127) // 128, K // 128))).astype(np.float32)
    d = run(a, sa, b, sb, out_dtype)
    ref = gemm.gemm_ref(a, sa, b, sb, "bf16" if out_dtype == torch.bfloat16 else "f32")
    got = d.view(torch.int16).cpu().numpy().view(np.uint16) if out_dtype == torch.bfloat16 \
        else d.cpu().numpy().view(np.uint32)
    assert_codes_equal(got, ref.view(got.dtype), "exact-integer gemm")


def test_gemm_identity_weights():
    x = synth.activation(256, 384, seed=4)["a"]
    a, sa = quantize.quantize_1x128(x)
    b = np.zeros((384, 384), np.uint8)
    b[np.arange(384), np.arange(384)] = 0x38
    sb = np.ones((3, 3), np.float32)
    d = run(a, sa, b, sb, torch.float32)
    # one nonzero product per output: D = fl32(dec(a) * sa); the kernel's
    # accumulator starts at +0, so a -0 product comes out as +0
    want = gemm.dequant_a(a, sa).astype(np.float32) + np.float32(0.0)
    assert_codes_equal(d.cpu().numpy().view(np.uint32), want.view(np.uint32), "identity weights")


def test_gemm_writes_only_its_output():
    M, N, K = 130, 48, 256
    a, sa, b, sb = operands(M, N, K, seed=9)
    buf = torch.full((M * N + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = buf[2048:2048 + M * N].view(M, N)
    fp8bs.gemm(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:2048]).all() and torch.isnan(buf[2048 + M * N:]).all()
    ref = bf16.to_f32(gemm.gemm_ref(a, sa, b, sb)).astype(np.float64)
    assert_gemm_close(out_host_f64(out), ref, "in-place out", dense_allowance(a, sa, b, sb))


def test_gemm_training_projection_full_size():
    # 4096 x 2112 x 7168: the last 128-wide column tile holds only 64 valid
    # columns (ragged weight block).  Every output against the float64
    # definition, rms over all of them.
    M, N, K = 4096, 2112, 7168
    print("gemm full size 4096x2112x7168", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=0)
    d = run(a, sa, b, sb)
    ref = bf16.to_f32(gemm.gemm_ref(a, sa, b, sb)).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, "gemm 4096x2112x7168", dense_allowance(a, sa, b, sb))


def test_gemm_decode_shape_pow2_full():
    M, N, K = 128, 24576, 1536
    print("gemm decode 128x24576x1536 pow2", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=0, pow2=True)
    d = run(a, sa, b, sb)
    ref = bf16.to_f32(gemm.gemm_ref(a, sa, b, sb)).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, "gemm 128x24576x1536", dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("K", [128, 256, 512, 640, 896])
@pytest.mark.parametrize("M,N", [(4000, 2112), (4096, 2048)])
def test_gemm_192_tile_chunk_counts(M, N, K):
    # the 192x192 tile's three-stage pipeline with 1, 2, 4, 5 and 7 chunks
    # (loop and tail), ragged last row and column tiles, BF16 and FP32 out
    print(f"gemm 192 tile M={M} N={N} K={K}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + N + K)
    ref = gemm.gemm_f64(a, sa, b, sb)
    d = run(a, sa, b, sb)
    assert_gemm_close(out_host_f64(d), bf16.to_f32(gemm.round_out(ref, "bf16")).astype(np.float64), f"gemm {M}x{N}x{K}",
                      dense_allowance(a, sa, b, sb))
    d = run(a, sa, b, sb, torch.float32)
    assert_gemm_close(out_host_f64(d), gemm.round_out(ref, "f32").astype(np.float64), f"gemm {M}x{N}x{K} f32",
                      dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("K", [128, 256, 384, 512, 640, 1152])
def test_gemm_64_tile_chunk_counts(K):
    # the 64x64 tile's four-stage pipeline with 1, 2, 3, 4, 5 and 9 chunks
    # (loop and tail); ragged last row and column tiles; BF16 and FP32 out
    M, N = 100, 208
    print(f"gemm 64 tile M={M} N={N} K={K}", flush=True)
    assert fp8bs.gemm_tile("dense", M, N, K) == (64, 64, 0)
    a, sa, b, sb = operands(M, N, K, seed=3 * K + 1)
    ref = gemm.gemm_f64(a, sa, b, sb)
    d = run(a, sa, b, sb)
    assert_gemm_close(out_host_f64(d), bf16.to_f32(gemm.round_out(ref, "bf16")).astype(np.float64), f"gemm {M}x{N}x{K}",
                      dense_allowance(a, sa, b, sb))
    d = run(a, sa, b, sb, torch.float32)
    assert_gemm_close(out_host_f64(d), gemm.round_out(ref, "f32").astype(np.float64), f"gemm {M}x{N}x{K} f32",
                      dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("M,N,K", [(128, 7168, 2048), (64, 2112, 7168)])
def test_gemm_few_rows_full_size(M, N, K):
    # the pages' Table 1 shapes with few tokens, unsplit, on the 64x64 tile:
    # every output against the float64 definition, rms over all of them
    print(f"gemm full size {M}x{N}x{K}", flush=True)
    assert fp8bs.gemm_tile("dense", M, N, K) == (64, 64, 0)
    a, sa, b, sb = operands(M, N, K, seed=M + N)
    d = run(a, sa, b, sb)
    ref = bf16.to_f32(gemm.gemm_ref(a, sa, b, sb)).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, f"gemm {M}x{N}x{K}", dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("M,N,K,pow2", [(4096, 4096, 7168, False), (128, 24576, 1536, False)])
def test_gemm_pages_shapes_full_size(M, N, K, pow2):
    # the pages' Table 1 shape with many tokens (256x256 tiles, one round)
    # and the decode projection with FP32 scales: every output against the
    # float64 definition, rms over all of them
    print(f"gemm full size {M}x{N}x{K} pow2={pow2}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + 2 * N, pow2=pow2)
    d = run(a, sa, b, sb)
    ref = bf16.to_f32(gemm.gemm_ref(a, sa, b, sb)).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, f"gemm {M}x{N}x{K}", dense_allowance(a, sa, b, sb))
