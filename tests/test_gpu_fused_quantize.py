"""GPU parity of the GEMM that quantizes its BF16 activation on the way in
(fp8bs_gemm_fused_quantize).

Its result is defined as the 1x128 quantization of the activation followed by
the block-scaled GEMM.  Bars:
- against the CPU oracle (quantize_1x128, then the float64 GEMM definition
  rounded once to the output dtype): |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref)
  elementwise, as for the other GEMMs;
- against the library's two-step path (fp8bs_quantize_1x128, then
  fp8bs_gemm_fp8_blockscaled with flags 0): bit-exact, NaN payloads and signs
  of zero included, since both take the same codes, scales, MFMA fragments and
  promotion steps.
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import bf16, gemm, quantize
from tests.gpu_util import (assert_codes_equal, assert_gemm_close, bf16_dev, codes_dev, dense_allowance, f32_dev,
                            out_host_f64, require_gpu)

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def out_bits(d):
    if d.dtype == torch.bfloat16:
        return d.view(torch.int16).cpu().numpy().view(np.uint16)
    return d.cpu().numpy().view(np.uint32)


def two_step(x, b, sb, pow2, out_dtype):
    q, s = fp8bs.quantize_1x128(x, pow2)
    d = fp8bs.gemm(q, s, b, sb, out_dtype=out_dtype, pow2_scales=False)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("M,N,K", [(64, 128, 128), (1, 16, 128), (100, 48, 256), (300, 528, 640),
                                   (257, 256, 1024), (130, 400, 384)])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fused_quantize_recipe(M, N, K, pow2, out_dtype):
    print(f"fused quantize M={M} N={N} K={K} pow2={pow2} out={out_dtype} tile "
          f"{fp8bs.gemm_tile('fused_quantize', M, N, K)}", flush=True)
    w = synth.dense(M, N, K, seed=M + 3 * N + K)
    b_np, sb_np = quantize.quantize_128x128(w["b"], pow2)
    x = bf16_dev(w["a"])
    b, sb = codes_dev(b_np), f32_dev(sb_np)
    d = fp8bs.gemm_fused_quantize(x, b, sb, out_dtype=out_dtype, pow2=pow2)
    torch.cuda.synchronize()
    # the oracle: quantize, then the float64 definition
    a_np, sa_np = quantize.quantize_1x128(w["a"], pow2)
    ref = gemm.gemm_f64(a_np, sa_np, b_np, sb_np)
    ref = (bf16.to_f32(gemm.round_out(ref, "bf16")) if out_dtype == torch.bfloat16
           else gemm.round_out(ref, "f32")).astype(np.float64)
    assert_gemm_close(out_host_f64(d), ref, f"fused quantize {M}x{N}x{K}", dense_allowance(a_np, sa_np, b_np, sb_np))
    # the library's two steps, bit for bit
    assert_codes_equal(out_bits(d), out_bits(two_step(x, b, sb, pow2, out_dtype)), "fused vs two-step")


@pytest.mark.parametrize("pow2", [False, True])
def test_fused_quantize_special_rows(pow2):
    # rows of zeros, of values below 2^-60 (the pre-scaled division), of
    # subnormal BF16, of the largest BF16, and a row with NaN and infinities:
    # the tile scales and codes come out as the quantizer's.
    M, N, K = 96, 144, 384
    print(f"fused quantize special rows pow2={pow2}", flush=True)
    w = synth.dense(M, N, K, seed=11)
    a = w["a"].copy()
    rng = np.random.default_rng(5)
    a[0] = 0
    a[1] = 0x8000                                          # -0
    a[2] = (rng.integers(0, 0x0080, K) | (rng.integers(0, 2, K) << 15)).astype(np.uint16)   # subnormals
    tiny = np.float32(2.0 ** -80) * rng.standard_normal(K).astype(np.float32)
    a[3] = (tiny.view(np.uint32) >> 16).astype(np.uint16)
    a[4] = np.where(rng.random(K) < 0.5, 0x7F7F, 0xFF7F).astype(np.uint16)                   # +-max BF16
    a[5, 7] = 0x7FC0                                      # NaN in the first tile
    a[5, 200] = 0x7F80                                    # +inf in the second
    a[6, 300] = 0xFF80                                    # -inf in the third
    b_np, sb_np = quantize.quantize_128x128(w["b"], pow2)
    x = bf16_dev(a)
    b, sb = codes_dev(b_np), f32_dev(sb_np)
    d = fp8bs.gemm_fused_quantize(x, b, sb, out_dtype=torch.float32, pow2=pow2)
    torch.cuda.synchronize()
    assert_codes_equal(out_bits(d), out_bits(two_step(x, b, sb, pow2, torch.float32)), "special rows")


def test_fused_quantize_full_size():
    # 16384 x 256 x 7168 (two column tiles per row block) and 4096 x 2112 x
    # 7168 (17 column tiles, a partial one last): every output bit-exact
    # against the two steps.
    for (M, N, K) in ((16384, 256, 7168), (4096, 2112, 7168)):
        print(f"fused quantize full size {M}x{N}x{K}", flush=True)
        w = synth.dense(M, N, K, seed=1)
        b_np, sb_np = quantize.quantize_128x128(w["b"])
        x = bf16_dev(w["a"])
        b, sb = codes_dev(b_np), f32_dev(sb_np)
        d = fp8bs.gemm_fused_quantize(x, b, sb)
        torch.cuda.synchronize()
        assert_codes_equal(out_bits(d), out_bits(two_step(x, b, sb, False, torch.bfloat16)), f"{M}x{N}x{K}")
