"""Seeded synthetic inputs shared by tests, the smoke check and the benchmark.

This module holds no arithmetic of the method (no quantization, no scales, no
GEMM); it only draws random numbers in a fixed order and rounds them once to
BF16 (RNE, through torch's CPU cast).  Arrays are NumPy; BF16 data is carried
as uint16 bit patterns.

Recipe (every workload, seed 0 unless a test says otherwise):
  1. A: float32 standard normal, shape [rows][K];
  2. outlier channels: n = max(1, round(0.01 K)) distinct columns of A drawn
     without replacement, multiplied by 50 (in float32, before rounding);
  3. B: float32 normal with standard deviation 0.02, shape [G][N][K]
     (G = 1 for dense);
  4. group structure: contiguous layout -- group sizes 128 * Multinomial(
     total/128, uniform over G); masked layout -- valid counts drawn uniformly
     from the integers 0..cap inclusive.
The pages measure on no dataset: these stand in for activations with a few
large-magnitude channels and for small-variance weights.
"""

import numpy as np
import torch

WORKLOADS = {
    # name: parameters; "pow2" asks for power-of-two scales in both operands.
    "dense_128x256x512": dict(kind="dense", M=128, N=256, K=512, pow2=False),
    "dense_4096x2112x7168": dict(kind="dense", M=4096, N=2112, K=7168, pow2=False),
    "decode_128x24576x1536_pow2": dict(kind="dense", M=128, N=24576, K=1536, pow2=True),
    "moe_contiguous_8x8192x4096x7168": dict(kind="contiguous", G=8, Mt=8192, N=4096, K=7168, pow2=False),
    "moe_masked_32x256x7168x2048": dict(kind="masked", G=32, cap=256, N=7168, K=2048, pow2=False),
}


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), RNE, via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def n_outliers(K: int) -> int:
    return max(1, int(round(0.01 * K)))


def _activation(rng, rows: int, K: int):
    a = rng.standard_normal((rows, K), dtype=np.float32)
    cols = rng.choice(K, n_outliers(K), replace=False)
    a[:, cols] *= np.float32(50.0)
    return a, np.sort(cols)


def _weights(rng, G: int, N: int, K: int):
    return rng.standard_normal((G, N, K), dtype=np.float32) * np.float32(0.02)


def dense(M: int, N: int, K: int, seed: int = 0) -> dict:
    """A[M][K], B[N][K] as BF16 bits."""
    rng = np.random.default_rng(seed)
    a, cols = _activation(rng, M, K)
    b = _weights(rng, 1, N, K)[0]
    return dict(a=bf16_bits(a), b=bf16_bits(b), outlier_cols=cols)


def activation(M: int, K: int, seed: int = 0) -> dict:
    """Only the activation of the recipe (steps 1-2)."""
    rng = np.random.default_rng(seed)
    a, cols = _activation(rng, M, K)
    return dict(a=bf16_bits(a), outlier_cols=cols)


def contiguous(G: int, Mt: int, N: int, K: int, seed: int = 0) -> dict:
    """A[Mt][K], B[G][N][K], m_offsets[G+1] (multiples of 128)."""
    if Mt % 128:
        raise ValueError("total rows must be a multiple of 128")
    rng = np.random.default_rng(seed)
    a, cols = _activation(rng, Mt, K)
    b = _weights(rng, G, N, K)
    sizes = rng.multinomial(Mt // 128, [1.0 / G] * G) * 128
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return dict(a=bf16_bits(a), b=bf16_bits(b), m_offsets=offs, outlier_cols=cols)


def masked(G: int, cap: int, N: int, K: int, seed: int = 0) -> dict:
    """A[G][cap][K], B[G][N][K], masked_m[G] in 0..cap.  Rows past the count
    hold random data like the others."""
    rng = np.random.default_rng(seed)
    a, cols = _activation(rng, G * cap, K)
    b = _weights(rng, G, N, K)
    counts = rng.integers(0, cap + 1, G).astype(np.int32)
    return dict(a=bf16_bits(a).reshape(G, cap, K), b=bf16_bits(b), masked_m=counts,
                outlier_cols=cols)


def workload(name: str, seed: int = 0) -> dict:
    w = WORKLOADS[name]
    if w["kind"] == "dense":
        return dense(w["M"], w["N"], w["K"], seed)
    if w["kind"] == "contiguous":
        return contiguous(w["G"], w["Mt"], w["N"], w["K"], seed)
    return masked(w["G"], w["cap"], w["N"], w["K"], seed)
