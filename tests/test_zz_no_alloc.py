"""The allocation-free split-K GEMM (fp8bs_gemm_fp8_blockscaled_splitk_noalloc,
for callers that cannot allocate) against the workspace variant it mirrors,
called through the C ABI: two calls in a row on the library's per-GPU scratch,
the second on a smaller problem (the scratch then still holds the first call's
partials), each bit-identical to the workspace call on the same inputs."""

import ctypes

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import build, fp8bs, synth
from oracle import quantize
from tests.gpu_util import codes_dev, f32_dev, require_gpu

pytestmark = pytest.mark.gpu

P, I64, I32, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32


def setup_module(module):
    require_gpu()


def _lib():
    lib = ctypes.CDLL(build.library_path())
    na = lib.fp8bs_gemm_fp8_blockscaled_splitk_noalloc
    na.argtypes = [P, P, P, P, P, I64, I64, I64, I32, U32, P]
    na.restype = ctypes.c_int
    ws = lib.fp8bs_gemm_fp8_blockscaled_splitk
    ws.argtypes = [P, P, P, P, P, I64, I64, I64, I32, U32, P, I64, P]
    ws.restype = ctypes.c_int
    return na, ws


def _operands(M, N, K, seed):
    w = synth.dense(M, N, K, seed=seed)
    a, sa = quantize.quantize_1x128(w["a"])
    b, sb = quantize.quantize_128x128(w["b"])
    return codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb)


@pytest.mark.parametrize("out_dtype,code", [(torch.bfloat16, 0), (torch.float32, 1)])
def test_noalloc_matches_workspace_call_twice_shrinking(out_dtype, code):
    na, ws = _lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 64 x 2112 x 7168: 22 tiles x 11 splits; then 37 x 208 x 4608: 3 x 18
    for (M, N, K) in [(64, 2112, 7168), (37, 208, 4608)]:
        print(f"no-alloc split-K M={M} N={N} K={K} out={out_dtype}", flush=True)
        assert fp8bs.splitk_workspace_bytes(M, N, K) > 0
        a, sa, b, sb = _operands(M, N, K, seed=M + N)
        d_na = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        d_ws = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        work = torch.empty(fp8bs.splitk_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        assert na(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), d_na.data_ptr(), M, N, K, code, 0,
                  stream) == 0
        assert ws(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(), d_ws.data_ptr(), M, N, K, code, 0,
                  work.data_ptr(), work.numel(), stream) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(d_na.float()).all()
        assert torch.equal(d_na.view(torch.int16), d_ws.view(torch.int16)), f"{M}x{N}x{K}"


def test_noalloc_binding_and_unsplit_shape():
    # through the binding; a shape that does not split uses no scratch
    for (M, N, K) in [(130, 96, 8192), (128, 7168, 2048)]:
        a, sa, b, sb = _operands(M, N, K, seed=5)
        d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        fp8bs.gemm_splitk_noalloc(a, sa, b, sb, d)
        ref = fp8bs.gemm_splitk(a, sa, b, sb)
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}"
