"""Emulator of a limited-precision fixed-point MMA accumulator (oracle only).
Test infrastructure only; nothing on the GPU path corresponds to it.

Why it exists: page 1 (the uniondaocoop.com post on DeepSeek's FP8 training)
says the FP8 GEMM accumulation on H800 tensor cores keeps only about 14 bits,
which gave a maximum relative error near 2% at K = 4096 in their test and gets
worse as K grows, and that the fix is to copy partial sums to FP32 registers
at a fixed interval along K.  Page 2 ("A Deadly Mistake Uncovered on Deepseek
China Ai"), paragraph on the Hopper tensor-core implementation, describes the
mechanism: products are aligned by right-shifting to the largest exponent,
only the top 14 bits survive the sign-fill shift, and the rest is truncated.

The model, step by step (readings for the points the pages leave open: group
size 32, the running accumulator takes part in the alignment, 14 bits are kept
below the leading bit; the variant that counts the leading bit among the 14 is
available through `bits`):

  for each group of `group` consecutive products p_k (exact float64):
    T    = {acc} U {p_k in the group}
    E    = floor(log2(max |t|, t in T))        (leading-bit position)
    lsb  = 2^(E - bits)
    acc  = sum over t in T of floor(t / lsb) * lsb
           (floor = arithmetic, sign-fill right shift = truncation to -inf)

With `promote_every` = P (a multiple of `group`), the limited accumulator is
reset at every P-long chunk of K and its value is added into an FP32 total
with one RNE rounding (the pages' promotion to FP32 registers); otherwise a
single chain covers all of K (the behaviour the pages criticise).
"""

import numpy as np


def limited_accumulate(p, group: int = 32, bits: int = 14, promote_every=None) -> np.ndarray:
    """Accumulate products p[..., K] (float64, exact) through the model above.
    Returns float64 results of shape p.shape[:-1]."""
    p = np.asarray(p, dtype=np.float64)
    K = p.shape[-1]
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    if promote_every is not None and promote_every % group:
        raise ValueError("the promotion interval must be a multiple of the group size")
    lead = p.shape[:-1]
    acc = np.zeros(lead)
    total = np.zeros(lead, dtype=np.float32)
    for k0 in range(0, K, group):
        if promote_every is not None and k0 and k0 % promote_every == 0:
            total = (total.astype(np.float64) + acc).astype(np.float32)
            acc = np.zeros(lead)
        blk = p[..., k0:k0 + group]
        mx = np.maximum(np.abs(acc), np.max(np.abs(blk), axis=-1))
        _, e = np.frexp(mx)                       # mx = f * 2^e, f in [0.5, 1)
        lsb = np.where(mx == 0, 1.0, np.ldexp(1.0, (e - 1) - bits))
        acc = (np.floor(acc / lsb) * lsb
               + np.sum(np.floor(blk / lsb[..., None]) * lsb[..., None], axis=-1))
    if promote_every is None:
        return acc
    return (total.astype(np.float64) + acc).astype(np.float32).astype(np.float64)


def products(a_vals, b_vals) -> np.ndarray:
    """All products a[m][k] * b[n][k] -> [M][N][K] float64."""
    a = np.asarray(a_vals, np.float64)
    b = np.asarray(b_vals, np.float64)
    return a[:, None, :] * b[None, :, :]


def max_relative_error(approx, exact) -> float:
    """max |approx - exact| / max |exact| over all outputs."""
    exact = np.asarray(exact, np.float64)
    return float(np.max(np.abs(np.asarray(approx) - exact)) / np.max(np.abs(exact)))
