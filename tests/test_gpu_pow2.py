"""GPU parity of the hardware-scaled path (power-of-two scales applied by the
scaled MFMA as E8M0 exponents, accumulated in its own FP32 accumulator).

Inputs: the workload recipes quantized by the oracle with power-of-two scales
(the same bytes go to both sides).  Bar: |gpu - ref| <= 8e-3 |ref| + 1e-3
rms(ref); bit-exact on exact-integer inputs.  The documented failure mode is
checked too: an output that depends on a scale that is not a power of two in
[2^-127, 2^127] is NaN, and no other output changes.
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import bf16, e4m3, gemm, quantize
from tests.gpu_util import (assert_codes_equal, assert_gemm_close, codes_dev, contiguous_allowance, dense_allowance,
                            f32_dev, i32_dev, masked_allowance, out_host_f64, require_gpu)

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


def operands(M, N, K, seed):
    w = synth.dense(M, N, K, seed=seed)
    a, sa = quantize.quantize_1x128(w["a"], pow2=True)
    b, sb = quantize.quantize_128x128(w["b"], pow2=True)
    return a, sa, b, sb


def run(a, sa, b, sb, out_dtype=torch.bfloat16):
    d = fp8bs.gemm(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out_dtype=out_dtype, pow2_scales=True)
    torch.cuda.synchronize()
    return d


def ref_out(a, sa, b, sb, out_dtype):
    r = gemm.gemm_f64(a, sa, b, sb)
    return (bf16.to_f32(gemm.round_out(r, "bf16")) if out_dtype == torch.bfloat16
            else gemm.round_out(r, "f32")).astype(np.float64)


# shapes that reach every tile: 128x128 (double-buffered), 192x192 (4096x2112,
# 4000x4112), 256x160 (2450x3696), 256x256, 64x64 and 128x96 (few rows), with ragged edges
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (37, 48, 384), (300, 400, 640), (4096, 2112, 1024), (4000, 7168, 256),
                                   (4096, 4096, 256), (4000, 4112, 384), (2450, 3696, 256), (128, 24576, 1536),
                                   (1, 16, 128), (100, 208, 1152), (100, 13328, 384), (513, 144, 1152)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_pow2_recipe(M, N, K, out_dtype):
    print(f"pow2 gemm M={M} N={N} K={K} out={out_dtype}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + 5 * N + K)
    d = run(a, sa, b, sb, out_dtype)
    assert_gemm_close(out_host_f64(d), ref_out(a, sa, b, sb, out_dtype), f"pow2 gemm {M}x{N}x{K}",
                      dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("M,N,K", [(256, 272, 1024), (4000, 4112, 256), (4096, 2112, 512), (4096, 4096, 256),
                                   (100, 208, 640), (100, 13328, 256)])
def test_pow2_exact_integer_bit_exact(M, N, K):
    print(f"pow2 exact-integer M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(7)
    vals = e4m3.decode(np.arange(256, dtype=np.uint8))
    ints = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
                     and abs(vals[c]) <= 16 and c != 0x80], np.uint8)
    a = rng.choice(ints, (M, K)).astype(np.uint8)
    b = rng.choice(ints, (N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-2, 2, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-2, 2, ((N + 127) // 128, K // 128))).astype(np.float32)
    d = run(a, sa, b, sb, torch.float32)
    ref = gemm.gemm_ref(a, sa, b, sb, "f32")
    assert_codes_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32), "pow2 exact-integer gemm")


def test_pow2_extreme_exponents():
    # scales 2^-127 (E8M0 byte 0, an FP32 subnormal) and 2^127 (byte 254)
    # are valid; the products stay finite
    M, N, K = 256, 256, 256
    a, sa, b, sb = operands(M, N, K, seed=3)
    sa = sa.copy()
    sb = sb.copy()
    sa[:, 5] = np.float32(2.0 ** -127)
    sa[:, 6] = np.float32(2.0 ** 100)
    sb[1, :] = np.float32(2.0 ** -20)
    d = run(a, sa, b, sb, torch.float32)
    got = out_host_f64(d)
    assert np.isfinite(got).all()
    ref = ref_out(a, sa, b, sb, torch.float32)
    for rows in (slice(0, 5), slice(7, M)):
        assert_gemm_close(got[rows], ref[rows], "pow2 ordinary rows")
    assert_gemm_close(got[6], ref[6], "row scaled by 2^100")
    assert np.all(np.abs(got[5]) <= 1e-30)   # 2^-127 times products of at most 448^2*256 scaled by 2^-7


def test_pow2_invalid_scale_gives_nan_only_where_used():
    M, N, K = 256, 384, 512
    a, sa, b, sb = operands(M, N, K, seed=4)
    sa = sa.copy()
    sb = sb.copy()
    sa[2, 17] = np.float32(3.0)            # activation row 17, chunk 2: not a power of two
    sb[2, 1] = np.float32(0.75)            # weight rows 256..383, chunk 1
    d = run(a, sa, b, sb, torch.float32)
    got = out_host_f64(d)
    bad = np.zeros((M, N), bool)
    bad[17, :] = True
    bad[:, 256:] = True
    assert np.isnan(got[bad]).all()
    good_ref = ref_out(a, sa, b, sb, torch.float32)
    assert_gemm_close(got[~bad], good_ref[~bad], "pow2 outputs with valid scales")


@pytest.mark.parametrize("G,Mt,N,K,offsets,tile", [
    (4, 1152, 2112, 384, [0, 128, 128, 640, 1024], (128, 128)),
    # 256x256 and 256x160 tiles: groups end half way into 256-row tiles,
    # rows past the last group must stay untouched
    (3, 1408, 7168, 256, [0, 384, 384, 1152], (256, 256)),
    (2, 1152, 7168, 256, [0, 640, 1024], (256, 160)),
    # the ping-pong 192x192 tile: groups of 640 and 1280 rows end inside tiles
    (2, 2048, 4096, 256, [0, 640, 1920], (192, 192)),
])
def test_pow2_contiguous(G, Mt, N, K, offsets, tile):
    assert fp8bs.gemm_tile("contiguous", Mt, N, K, G, pow2_scales=True)[:2] == tile
    print(f"pow2 contiguous G={G} Mt={Mt} N={N} K={K} tile {tile}", flush=True)
    w = synth.contiguous(G, Mt, N, K, seed=9 + G)
    a, sa = quantize.quantize_1x128(w["a"], pow2=True)
    b, sb = quantize.quantize_128x128(w["b"], pow2=True)
    offs = np.array(offsets, np.int32)
    ref = gemm.grouped_contiguous_f64(a, sa, b, sb, offs)
    used = ~np.isnan(ref[:, 0])
    d = fp8bs.grouped_gemm_contiguous(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(offs),
                                      out_dtype=torch.float32, pow2_scales=True)
    torch.cuda.synchronize()
    allow = contiguous_allowance(a, sa, b, sb, offs, np.nonzero(used)[0])
    assert_gemm_close(d.cpu().numpy().astype(np.float64)[used], ref[used].astype(np.float32).astype(np.float64),
                      "pow2 contiguous fp32", allow)
    sentinel = 0x7FC1
    out = torch.full((Mt, N), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    fp8bs.grouped_gemm_contiguous(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(offs), out=out,
                                  pow2_scales=True)
    torch.cuda.synchronize()
    raw = out.view(torch.int16).cpu().numpy()
    assert (raw[~used] == sentinel).all(), "rows outside every group were written"
    ref_b = bf16.to_f32(bf16.from_f64_rne(ref[used])).astype(np.float64)
    assert_gemm_close(out.float().cpu().numpy().astype(np.float64)[used], ref_b, "pow2 contiguous bf16", allow)


@pytest.mark.parametrize("G,cap,N,K,counts", [(3, 256, 96, 256, [0, 256, 77]),
                                              (20, 256, 4096, 256, [0, 1, 255, 256, 129, 128, 0, 7, 200, 256, 64,
                                                                    3, 0, 0, 250, 100, 31, 256, 17, 90]),
                                              # hardware scaling on the masked tile, K of four chunks
                                              (20, 256, 6144, 512, [0, 1, 255, 256, 129, 128, 0, 7, 200, 256, 64,
                                                                    3, 0, 0, 250, 100, 31, 256, 17, 90])])
def test_pow2_masked(G, cap, N, K, counts):
    print(f"pow2 masked G={G} cap={cap} N={N} K={K}", flush=True)
    w = synth.masked(G, cap, N, K, seed=G + N)
    a2, sa2 = quantize.quantize_1x128(w["a"].reshape(G * cap, K), pow2=True)
    a = a2.reshape(G, cap, K)
    sa = np.stack([sa2[:, g * cap:(g + 1) * cap] for g in range(G)])
    b, sb = quantize.quantize_128x128(w["b"], pow2=True)
    cnt = np.asarray(counts, np.int32)
    out = torch.full((G, cap, N), float("nan"), dtype=torch.float32, device="cuda")
    fp8bs.grouped_gemm_masked(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(cnt),
                              out_dtype=torch.float32, out=out, pow2_scales=True)
    torch.cuda.synchronize()
    ref = gemm.grouped_masked_f64(a, sa, b, sb, cnt)
    valid = ~np.isnan(ref[:, :, 0])
    got = out.cpu().numpy().astype(np.float64)
    assert np.isnan(got[~valid]).all(), "rows past the count were written"
    assert_gemm_close(got[valid], ref[valid].astype(np.float32).astype(np.float64), "pow2 masked",
                      masked_allowance(a, sa, b, sb, valid))
