"""Pins for the oracle's weight transposition (CPU only).

The transposed weight must carry the same values as the weight, transposed:
checked against an independent decode (torch's E4M3 type) with the block
scale looked up per element, and through the data-gradient identity
dY (W^T)^T = dY W on a ragged N, where the activation gradient is quantized
over the zero-padded width.
"""

import numpy as np
import pytest
import torch

from fp8_block_scaled_04_amd import synth
from oracle import gemm, quantize
from tests._exact import tile_scale_exact


def tdec(q):
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def block_values(q, s):
    """Values of a block-scaled weight q[R][C] with s[ceil(R/128)][C/128],
    decoded by torch and scaled element by element."""
    R, C = q.shape
    v = tdec(q)
    out = np.empty((R, C))
    for r in range(R):
        for c in range(C):
            out[r, c] = v[r, c] * float(s[r // 128, c // 128])
    return out


def random_weight(N, K, seed):
    rng = np.random.default_rng(seed)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # no NaN
    q = rng.choice(codes, (N, K)).astype(np.uint8)
    s = (rng.random(((N + 127) // 128, K // 128)) + 0.25).astype(np.float32)
    return q, s


@pytest.mark.parametrize("N,K", [(200, 384), (128, 256), (16, 128), (272, 128)])
def test_transposed_weight_has_the_same_values(N, K):
    q, s = random_weight(N, K, seed=N + K)
    qt, st = quantize.transpose_128x128(q, s)
    Np = 128 * ((N + 127) // 128)
    assert qt.shape == (K, Np) and st.shape == (K // 128, Np // 128)
    w = block_values(q, s)
    wt = block_values(qt, st)
    assert np.array_equal(wt[:, :N], w.T)
    assert np.all(qt[:, N:] == 0)                 # padded columns hold +0 codes


def test_transpose_twice_is_identity():
    q, s = random_weight(256, 384, seed=3)
    qt, st = quantize.transpose_128x128(q, s)
    q2, s2 = quantize.transpose_128x128(qt, st)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_grouped_transpose_is_per_group():
    qa, sa = random_weight(144, 256, seed=4)
    qb, sb = random_weight(144, 256, seed=5)
    qt, st = quantize.transpose_128x128(np.stack([qa, qb]), np.stack([sa, sb]))
    for g, (q, s) in enumerate(((qa, sa), (qb, sb))):
        t, u = quantize.transpose_128x128(q, s)
        assert np.array_equal(qt[g], t) and np.array_equal(st[g], u)


def test_data_gradient_through_the_transposed_weight():
    # dX = dY W with W[N][K] (N = 200 output features, K = 256 inputs): the NT
    # GEMM takes A = dY quantized 1x128 over the zero-padded width 256 and
    # B = W^T; the result must equal the float64 product of the values.
    T, N, K = 64, 200, 256
    w_bits = synth.dense(T, N, K, seed=8)["b"]                # [N][K] BF16 weight recipe
    q, s = quantize.quantize_128x128(w_bits)
    qt, st = quantize.transpose_128x128(q, s)
    dy = synth.activation(T, N, seed=9)["a"]                   # [T][N] BF16 bits
    Np = qt.shape[1]
    dy_pad = np.zeros((T, Np), np.uint16)
    dy_pad[:, :N] = dy
    a, sa = quantize.quantize_1x128(dy_pad)
    assert np.all(a[:, N:] == 0)
    # the padded last tile has the scale of the ragged tile: amax over its
    # N - 128 valid values, divided exactly
    x = synth_f32(dy)
    for t in range(T):
        assert sa[1, t] == np.float32(tile_scale_exact(float(np.max(np.abs(x[t, 128:N]))), False))
    got = gemm.gemm_f64(a, sa, qt, st)
    a_vals = tdec(a) * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    want = a_vals[:, :N] @ block_values(q, s)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-300)


def synth_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)
