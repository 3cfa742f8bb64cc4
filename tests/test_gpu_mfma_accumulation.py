"""The matrix core's accumulation of one 128-wide chunk, measured.

Page 1 (the uniondaocoop.com post on DeepSeek's FP8 training) reports that the
FP8 GEMM accumulation of H800 tensor cores keeps about 14 bits and that
promoting partial sums to FP32 at a fixed K interval fixes the error growth;
page 2 ("A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on the
Hopper tensor-core implementation) describes the mechanism: products aligned
by right shifts to the largest exponent, low bits truncated.

gfx950's v_mfma_f32_16x16x128_f8f6f4, which computes one 128-wide chunk per
instruction here, behaves the same way inside the chunk: a GEMM with K = 128
and unit scales (FP32 out, so D is one MFMA result per element) differs from
the exact sum of its 128 products by far more than FP32 rounding, and stays
within the bound of a model that sums groups of 8 consecutive products after
aligning each group to its largest product and keeping 13 bits below it
(measured: about 14; tests/gpu_util.py uses the same bound).  The promotion
after every chunk is what keeps this from growing along K.
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import fp8bs, synth
from oracle import e4m3, gemm, quantize
from tests.gpu_util import codes_dev, f32_dev, mfma_allowance, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_gpu()


FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
MID = np.array([c for c in FINITE if 5 <= ((c >> 3) & 15) <= 9], np.uint8)


def families(rng, M, N):
    K = 128
    a1, b1 = rng.choice(FINITE, (M, K)), rng.choice(FINITE, (N, K))           # every exponent
    a2, b2 = rng.choice(MID, (M, K)), rng.choice(MID, (N, K))                 # values of one scale
    pos = MID[MID < 0x80]
    a3, b3 = rng.choice(pos, (M, K)), rng.choice(pos, (N, K))                 # no cancellation
    a4, b4 = rng.choice(MID, (M, K)), rng.choice(MID, (N, K))
    a4[:, 0] = 0x70
    b4[:, 0] = 0x70                                                            # one product 2^14 per output
    w = synth.dense(M, N, K, seed=3)                                           # the workload recipe
    a5, _ = quantize.quantize_1x128(w["a"])
    b5, _ = quantize.quantize_128x128(w["b"])
    return {"all exponents": (a1, b1), "one binade": (a2, b2), "positive": (a3, b3),
            "one large product": (a4, b4), "workload recipe": (a5, b5)}


@pytest.mark.parametrize("name", ["all exponents", "one binade", "positive", "one large product",
                                  "workload recipe"])
def test_single_chunk_accumulation_is_truncated_to_about_14_bits(name):
    M, N = 192, 256
    a, b = families(np.random.default_rng(17), M, N)[name]
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    sa = np.ones((1, M), np.float32)
    sb = np.ones(((N + 127) // 128, 1), np.float32)
    d = fp8bs.gemm(codes_dev(a), f32_dev(sa), codes_dev(b), f32_dev(sb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = d.cpu().numpy().astype(np.float64)
    exact = gemm.gemm_f64(a, sa, b, sb)
    err = np.abs(got - exact)
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    bound = mfma_allowance(a[mm.ravel()], np.ones((M * N, 1)), b[nn.ravel()], np.ones((M * N, 1))).reshape(M, N)
    print(f"{name}: max err/bound {np.max(err / np.where(bound > 0, bound, 1e-300)):.3f}, "
          f"inexact outputs {np.mean(err > 0):.3f}", flush=True)
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} outputs beyond the 13-bit group bound"
    # and it is not an FP32-exact sum: well beyond FP32 rounding somewhere
    p = np.abs(e4m3.decode(a)[:, None, :] * e4m3.decode(b)[None, :, :]).sum(-1)
    if name != "workload recipe":
        assert np.max(err / np.where(p > 0, p, 1)) > 2.0 ** -20, f"{name}: no error beyond FP32 rounding"
