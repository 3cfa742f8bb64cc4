"""GPU parity of the grouped (MoE) GEMMs against the CPU oracle: contiguous
and masked layouts, empty groups, counts 0 and cap, rows that must stay
untouched, and the full-size workloads on every output."""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import bf16, gemm, quantize
from tests.gpu_util import (assert_gemm_close, codes_dev, contiguous_allowance, f32_dev, i32_dev, masked_allowance,
                            out_host_f64, require_gpu)

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a BF16 NaN bit pattern the kernels never write


def setup_module(module):
    require_gpu()


def sentinel_out(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def untouched(t):
    return (t.view(torch.int16).cpu().numpy() == SENTINEL).all()


def contiguous_operands(G, Mt, N, K, seed, offsets=None):
    w = synth.contiguous(G, Mt, N, K, seed=seed)
    a, sa = quantize.quantize_1x128(w["a"])
    b, sb = quantize.quantize_128x128(w["b"])
    offs = w["m_offsets"] if offsets is None else np.asarray(offsets, np.int32)
    return a, sa, b, sb, offs


def run_contiguous(a, sa, b, sb, offs, Mt, N):
    out = sentinel_out((Mt, N))
    fp8bs.grouped_gemm_contiguous(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(offs), out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G,Mt,N,K,offsets", [
    (4, 640, 96, 256, [0, 0, 256, 384, 512]),        # empty first group, rows 512.. unused
    (3, 384, 2112, 128, [0, 128, 256, 384]),
    (5, 1024, 48, 640, None),                        # seeded multinomial sizes
    (2, 256, 16, 384, [0, 0, 0]),                    # every group empty
    # 128x128 tiles at size: 128-row groups, one group is empty
    (7, 4608, 4096, 256, [0, 128, 128, 1152, 2304, 2432, 3840, 4480]),
    # the 192x192 tile (ping-pong loop): groups of 640 and 1280 rows end
    # inside a tile, rows 1920.. unused
    (2, 2048, 4096, 256, [0, 640, 1920]),
    # the 256x256 tile: a group of 384 rows ends half way into a tile, an
    # empty group, rows 1152.. unused
    (3, 1408, 7168, 256, [0, 384, 384, 1152]),
    # the 256x160 tile: groups of 640 and 384 rows end inside tiles, rows
    # 1024.. unused
    (2, 1152, 7168, 256, [0, 640, 1024]),
])
def test_contiguous(G, Mt, N, K, offsets):
    print(f"contiguous G={G} Mt={Mt} N={N} K={K} offs={offsets} tile {fp8bs.gemm_tile('contiguous', Mt, N, K, G)}",
          flush=True)
    a, sa, b, sb, offs = contiguous_operands(G, Mt, N, K, seed=G + Mt + N, offsets=offsets)
    out = run_contiguous(a, sa, b, sb, offs, Mt, N)
    ref = gemm.grouped_contiguous_f64(a, sa, b, sb, offs)
    used = ~np.isnan(ref[:, 0])
    assert untouched(out[torch.from_numpy(~used).cuda()]), "rows outside every group were written"
    if used.any():
        ref_b = bf16.to_f32(bf16.from_f64_rne(ref[used])).astype(np.float64)
        assert_gemm_close(out_host_f64(out)[used], ref_b, "contiguous",
                          contiguous_allowance(a, sa, b, sb, offs, np.nonzero(used)[0]))


def test_contiguous_fp32_out():
    a, sa, b, sb, offs = contiguous_operands(3, 512, 64, 256, seed=3)
    d = fp8bs.grouped_gemm_contiguous(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(offs),
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = gemm.grouped_contiguous_f64(a, sa, b, sb, offs)
    used = ~np.isnan(ref[:, 0])
    assert_gemm_close(d.cpu().numpy().astype(np.float64)[used],
                      ref[used].astype(np.float32).astype(np.float64), "contiguous fp32",
                      contiguous_allowance(a, sa, b, sb, offs, np.nonzero(used)[0]))


def test_contiguous_full_size():
    # every output of every group against the float64 definition, rms over
    # all valid outputs of the call
    G, Mt, N, K = 8, 8192, 4096, 7168
    print("contiguous full size 8x8192x4096x7168", flush=True)
    a, sa, b, sb, offs = contiguous_operands(G, Mt, N, K, seed=0)
    out = run_contiguous(a, sa, b, sb, offs, Mt, N)
    ref = gemm.grouped_contiguous_f64(a, sa, b, sb, offs)
    used = ~np.isnan(ref[:, 0])
    assert used.all(), "the seeded group sizes cover every row"
    ref_b = bf16.to_f32(bf16.from_f64_rne(ref)).astype(np.float64)
    del ref
    assert_gemm_close(out_host_f64(out), ref_b, "contiguous 8x8192x4096x7168", contiguous_allowance(a, sa, b, sb, offs))


def masked_operands(G, cap, N, K, seed, counts=None):
    w = synth.masked(G, cap, N, K, seed=seed)
    a2, sa2 = quantize.quantize_1x128(w["a"].reshape(G * cap, K))
    a = a2.reshape(G, cap, K)
    sa = np.stack([sa2[:, g * cap:(g + 1) * cap] for g in range(G)])
    b, sb = quantize.quantize_128x128(w["b"])
    cnt = w["masked_m"] if counts is None else np.asarray(counts, np.int32)
    return a, sa, b, sb, cnt


def run_masked(a, sa, b, sb, cnt, out_dtype=torch.bfloat16):
    G, cap, _ = a.shape
    N = b.shape[1]
    out = sentinel_out((G, cap, N)) if out_dtype == torch.bfloat16 else \
        torch.full((G, cap, N), float("nan"), dtype=torch.float32, device="cuda")
    fp8bs.grouped_gemm_masked(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), i32_dev(cnt),
                              out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G,cap,N,K,counts", [
    (3, 256, 64, 256, [0, 256, 77]),
    (3, 100, 48, 384, [100, 0, 33]),                 # capacity not a multiple of the tile
    (4, 256, 2112, 128, [1, 128, 129, 255]),
    (2, 64, 16, 512, [70, -3]),                      # counts outside [0, cap] are clamped
    (6, 256, 96, 640, None),                         # seeded uniform counts
    # the 128x256 masked-tile path (40 row tiles x 16 column tiles)
    (20, 256, 4096, 256, [0, 1, 255, 256, 129, 128, 0, 7, 200, 256, 64, 3, 0, 0, 250, 100, 31, 256, 17, 90]),
    # the masked tile's three-stage pipeline with K of exactly three chunks,
    # then with a chunk count that is not a multiple of three (counts 1, 64,
    # 129 leave whole waves without rows)
    (20, 256, 6144, 384, [0, 1, 255, 256, 129, 128, 0, 7, 200, 256, 64, 3, 0, 0, 250, 100, 31, 256, 17, 90]),
    (24, 256, 4096, 640, None),
    (64, 128, 2048, 512, None),                      # the most groups the one-wave expert lookup holds
    (65, 128, 2048, 384, None),                      # one more: the lookup in passes of 64 groups
])
def test_masked(G, cap, N, K, counts):
    print(f"masked G={G} cap={cap} N={N} K={K} counts={counts}", flush=True)
    a, sa, b, sb, cnt = masked_operands(G, cap, N, K, seed=G + cap + N, counts=counts)
    out = run_masked(a, sa, b, sb, cnt)
    ref = gemm.grouped_masked_f64(a, sa, b, sb, cnt)
    valid = ~np.isnan(ref[:, :, 0])
    assert untouched(out[torch.from_numpy(~valid).cuda()]), "rows past the count were written"
    if valid.any():
        ref_b = bf16.to_f32(bf16.from_f64_rne(ref[valid])).astype(np.float64)
        assert_gemm_close(out_host_f64(out)[valid], ref_b, "masked", masked_allowance(a, sa, b, sb, valid))


@pytest.mark.parametrize("G,cap,N,K,counts", [(2, 128, 32, 256, [50, 128]),
                                              (12, 256, 8192, 512, [256, 0, 70, 129, 1, 255, 128, 64, 65, 0, 200, 3])])
def test_masked_fp32_out(G, cap, N, K, counts):
    print(f"masked fp32 G={G} cap={cap} N={N} K={K}", flush=True)
    a, sa, b, sb, cnt = masked_operands(G, cap, N, K, seed=5, counts=counts)
    out = run_masked(a, sa, b, sb, cnt, torch.float32)
    ref = gemm.grouped_masked_f64(a, sa, b, sb, cnt)
    valid = ~np.isnan(ref[:, :, 0])
    got = out.cpu().numpy().astype(np.float64)
    assert np.isnan(got[~valid]).all()
    assert_gemm_close(got[valid], ref[valid].astype(np.float32).astype(np.float64), "masked fp32",
                      masked_allowance(a, sa, b, sb, valid))


def test_masked_decode_full_size():
    # every valid row of every expert against the float64 definition (rms
    # over all valid outputs of the call); rows past each count untouched
    G, cap, N, K = 32, 256, 7168, 2048
    print("masked full size 32x256x7168x2048", flush=True)
    a, sa, b, sb, cnt = masked_operands(G, cap, N, K, seed=0)
    out = run_masked(a, sa, b, sb, cnt)
    raw = out.view(torch.int16).cpu().numpy()
    for g in range(G):
        assert (raw[g, int(cnt[g]):] == SENTINEL).all(), f"group {g}: rows past {int(cnt[g])} written"
    ref = gemm.grouped_masked_f64(a, sa, b, sb, cnt)
    valid = ~np.isnan(ref[:, :, 0])
    assert valid.sum() == int(np.clip(cnt, 0, cap).sum())
    ref_b = bf16.to_f32(bf16.from_f64_rne(ref[valid])).astype(np.float64)
    assert_gemm_close(out_host_f64(out)[valid], ref_b, "masked 32x256x7168x2048", masked_allowance(a, sa, b, sb, valid))
