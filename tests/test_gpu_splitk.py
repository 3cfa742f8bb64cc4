"""GPU parity of the split-K dense GEMM (fp8bs_gemm_fp8_blockscaled_splitk)
against the CPU oracle, and against the unsplit GEMM.

Inputs: the seeded workload recipe quantized by the oracle (the same bytes go
to both sides).  Bar: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) elementwise,
ref = float64 definition rounded once to the output dtype; bit-exact (and
bit-identical to the unsplit GEMM) when every partial sum is exact in FP32
(exact-integer inputs).  Shapes include the pages' Table 1 rows with few
tokens (M = 64, split; M = 128 with K = 2048, not split), ragged row and
column tiles on both split tiles (64x64 up to 128 rows, 128x96 above), uneven
chunk counts per split, the split cap, and a single chunk.
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import bf16, e4m3, gemm, quantize
from tests.gpu_util import (assert_codes_equal, assert_gemm_close, codes_dev, dense_allowance, f32_dev, out_host_f64,
                            require_gpu)

pytestmark = pytest.mark.gpu

def tile_bytes(M):
    # workspace bytes per tile partial: 64x64 split tiles up to 128 rows, else 128x96
    return (64 * 64 if M <= 128 else 128 * 96) * 4


def setup_module(module):
    require_gpu()


def operands(M, N, K, seed, pow2=False):
    w = synth.dense(M, N, K, seed=seed)
    a, sa = quantize.quantize_1x128(w["a"], pow2)
    b, sb = quantize.quantize_128x128(w["b"], pow2)
    return a, sa, b, sb


def run(a, sa, b, sb, out_dtype=torch.bfloat16, pow2=False, workspace=None):
    d = fp8bs.gemm_splitk(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out_dtype=out_dtype,
                          pow2_scales=pow2, workspace=workspace)
    torch.cuda.synchronize()
    return d


def ref_out(a, sa, b, sb, out_dtype):
    r = gemm.gemm_f64(a, sa, b, sb)
    return (bf16.to_f32(gemm.round_out(r, "bf16")) if out_dtype == torch.bfloat16
            else gemm.round_out(r, "f32")).astype(np.float64)


# (M, N, K, split tiles, splits)
SHAPES = [(64, 2112, 7168, 33, 7),     # Table 1, M = 64 (64x64 split tiles)
          (128, 2112, 7168, 66, 3),    # two 64-row tiles, 56 chunks over 3 splits
          (100, 4112, 4224, 130, 1),   # too many tiles to split
          (256, 2112, 7168, 44, 5),    # 128x96 split tiles, two row tiles
          (37, 208, 4608, 4, 18),      # ragged rows and columns, two chunks per split
          (200, 400, 4224, 10, 16),    # 33 chunks over 16 splits: two or three each
          (130, 96, 8192, 2, 32),      # the split cap
          (128, 7168, 2048, 224, 1),   # Table 1, M = 128: 16 chunks, not split
          (1, 16, 128, 1, 1)]          # a single chunk: the unsplit GEMM


@pytest.mark.parametrize("M,N,K,tiles,splits", SHAPES)
def test_splitk_workspace_size(M, N, K, tiles, splits):
    assert fp8bs.splitk_workspace_bytes(M, N, K) == (tiles * splits * tile_bytes(M) if splits > 1 else 0)


@pytest.mark.parametrize("M,N,K,tiles,splits", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_splitk_workload_recipe(M, N, K, tiles, splits, out_dtype):
    print(f"split-K gemm M={M} N={N} K={K} splits={splits} out={out_dtype}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + 3 * N + K)
    d = run(a, sa, b, sb, out_dtype)
    assert_gemm_close(out_host_f64(d), ref_out(a, sa, b, sb, out_dtype), f"split-K gemm {M}x{N}x{K}",
                      dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (37, 208, 4608), (128, 2112, 7168), (130, 96, 8192)])
def test_splitk_pow2_scales(M, N, K):
    # power-of-two scales applied by the scaled MFMA inside each split
    print(f"split-K pow2 gemm M={M} N={N} K={K}", flush=True)
    a, sa, b, sb = operands(M, N, K, seed=M + 5 * N + K, pow2=True)
    d = run(a, sa, b, sb, torch.float32, pow2=True)
    assert_gemm_close(out_host_f64(d), ref_out(a, sa, b, sb, torch.float32), f"split-K pow2 gemm {M}x{N}x{K}",
                      dense_allowance(a, sa, b, sb))


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (128, 2112, 7168), (200, 400, 4224), (130, 96, 8192)])
@pytest.mark.parametrize("pow2", [False, True])
def test_splitk_exact_integer_inputs_bit_exact(M, N, K, pow2):
    # integer codes in [-16, 16] and power-of-two scales: every partial and
    # their sum are exact in FP32, so the output is the one rounding of the
    # exact result -- and the same bits as the unsplit GEMM's
    print(f"split-K exact-integer gemm M={M} N={N} K={K} pow2={pow2}", flush=True)
    rng = np.random.default_rng(11)
    vals = e4m3.decode(np.arange(256, dtype=np.uint8))
    ints = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
                     and abs(vals[c]) <= 16 and c != 0x80], np.uint8)
    a = rng.choice(ints, (M, K)).astype(np.uint8)
    b = rng.choice(ints, (N, K)).astype(np.uint8)
    sa = (2.0 ** rng.integers(-2, 2, (K // 128, M))).astype(np.float32)
    sb = (2.0 ** rng.integers(-2, 2, ((N + 127) // 128, K // 128))).astype(np.float32)
    for out_dtype, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        d = run(a, sa, b, sb, out_dtype, pow2=pow2)
        ref = gemm.gemm_ref(a, sa, b, sb, name)
        bits = np.uint32 if name == "f32" else np.uint16
        assert_codes_equal(d.cpu().view(torch.int32 if name == "f32" else torch.int16).numpy().view(bits),
                           ref.view(bits), f"split-K exact-integer gemm ({name})")
        u = fp8bs.gemm(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out_dtype=out_dtype, pow2_scales=pow2)
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), u.view(torch.int16)), "split-K and unsplit GEMM differ"


def test_splitk_deterministic_whatever_the_workspace_held():
    # the partials are added in split order, and every byte of the workspace
    # the reduction reads is written first: a workspace full of NaN bytes,
    # reused across calls, gives the same bits every time
    M, N, K = 64, 2112, 7168
    a, sa, b, sb = operands(M, N, K, seed=3)
    ws = torch.full((fp8bs.splitk_workspace_bytes(M, N, K),), 0xFF, dtype=torch.uint8, device="cuda")
    d1 = run(a, sa, b, sb, torch.float32, workspace=ws)
    d2 = run(a, sa, b, sb, torch.float32, workspace=ws)
    ws.fill_(0x7F)
    d3 = run(a, sa, b, sb, torch.float32, workspace=ws)
    assert torch.isfinite(d1).all()
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))
    assert torch.equal(d1.view(torch.int32), d3.view(torch.int32))
