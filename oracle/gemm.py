"""Block-scaled FP8 GEMM references (oracle).  Test infrastructure only.

What the GEMM computes (page 1, the uniondaocoop.com post on FP8 training:
FP8 inputs, BF16 or FP32 outputs, fine-grained scaling, partial sums promoted
to FP32; page 4, "Deepseek veroeffentlicht Deepgemm", section
"Schluesselmerkmale von DeepGemm": one dense and two MoE layouts):

    D[m][n] = sum_kb  sA[kb][m] * sB[n/128][kb] * sum_{k in kb} dec(A[m][k]) * dec(B[n][k])

with A[M][K] E4M3 and 1x128 scales sA[K/128][M]; B[N][K] E4M3 and 128x128
block scales sB[ceil(N/128)][K/128]; D = A * B^T ("NT").  The method reaches
this plain definition up to rounding order, so the reference is the definition
written out: dequantize exactly to float64 and accumulate in float64 (a BLAS
float64 matmul is one step), then round once to BF16 (RNE) or FP32.

A second, independent path (``chunk_sums_exact``) uses integers: dec(c) * 2^9
is an integer of magnitude <= 229376, so every 128-long chunk sum of products
is an exact int64; chunk sums are then scaled in float64.

Grouped layouts:
  contiguous: A rows are concatenated per group; group g owns rows
              [m_offsets[g], m_offsets[g+1]) and uses B[g], sB[g].
  masked:     A[G][cap][K]; group g uses only its first masked_m[g] rows.
Rows that belong to no group are reported as NaN (not compared).

Weight gradient (page 1, paragraphs on caching FP8 activations and converting
1x128 tiles to 128x1 tiles for the backward pass): dW = dY^T X contracts over
tokens, so both operands are quantized along the token dimension -- dY^T and
X^T with one scale per 128 tokens of each row (the 128x1 tiles of dY and X,
i.e. the output of the transpose-requantize step).  As an "NT" GEMM:

    D[m][n] = sum_kb  sA[kb][m] * sB[kb][n] * sum_{k in kb} dec(A[m][k]) * dec(B[n][k])

with A[M][K], sA[K/128][M], B[N][K], sB[K/128][N] (K = tokens), FP32 out,
optionally added to an existing FP32 D (gradient accumulation).
"""

import numpy as np

from . import bf16, e4m3

TILE = 128


def dequant_a(a, sa) -> np.ndarray:
    """A[M][K] codes with sA[K/128][M] -> float64 values (exact)."""
    a = np.asarray(a, np.uint8)
    sa = np.asarray(sa, np.float32).astype(np.float64)
    return e4m3.decode(a) * np.repeat(sa.T, TILE, axis=1)


def dequant_b(b, sb) -> np.ndarray:
    """B[N][K] codes with sB[ceil(N/128)][K/128] -> float64 values (exact)."""
    b = np.asarray(b, np.uint8)
    N = b.shape[0]
    sb = np.asarray(sb, np.float32).astype(np.float64)
    full = np.repeat(np.repeat(sb, TILE, axis=0)[:N], TILE, axis=1)
    return e4m3.decode(b) * full


def gemm_f64(a, sa, b, sb) -> np.ndarray:
    """Exact-input, float64-accumulated D = deq(A) * deq(B)^T."""
    return dequant_a(a, sa) @ dequant_b(b, sb).T


def round_out(d64, out: str):
    """Round a float64 result once: 'bf16' -> uint16 bits, 'f32' -> float32."""
    if out == "bf16":
        return bf16.from_f64_rne(d64)
    if out == "f32":
        return np.asarray(d64, np.float64).astype(np.float32)
    raise ValueError(out)


def gemm_ref(a, sa, b, sb, out: str = "bf16"):
    """Dense reference: the definition in float64, rounded once to `out`."""
    return round_out(gemm_f64(a, sa, b, sb), out)


def chunk_sums_exact(a, sa, b, sb) -> np.ndarray:
    """Second path: exact int64 chunk sums of products, then float64 scaling."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    ai = np.rint(e4m3.decode(a) * 512.0).astype(np.int64)    # exact integers
    bi = np.rint(e4m3.decode(b) * 512.0).astype(np.int64)
    sa = np.asarray(sa, np.float32).astype(np.float64)
    sb = np.asarray(sb, np.float32).astype(np.float64)
    out = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // TILE):
        sl = slice(kb * TILE, (kb + 1) * TILE)
        p = ai[:, sl] @ bi[:, sl].T                            # int64, exact
        scale = sa[kb][:, None] * np.repeat(sb[:, kb], TILE)[:N][None, :]
        out += p.astype(np.float64) * 2.0 ** -18 * scale
    return out


def gemm_sample_f64(a, sa, b, sb, rows, cols) -> np.ndarray:
    """float64 D[rows[i]][cols[i]] for sampled output positions, one by one
    (for checks at sizes where the full product is too slow on the CPU)."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    A = dequant_a(np.asarray(a)[rows], np.asarray(sa)[:, rows])
    sb = np.asarray(sb)
    Bq = np.asarray(b)[cols]
    Bs = sb[cols // TILE]                                      # [n, K/128]
    B = e4m3.decode(Bq) * np.repeat(Bs.astype(np.float64), TILE, axis=1)
    return np.sum(A * B, axis=1)


def gemm_block_f64(a, sa, b, sb, rows, cols) -> np.ndarray:
    """float64 D[rows][:, cols]: the outputs at every (row, col) pair of the
    sampled rows and columns (dequantize only those rows of A and of B)."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    A = dequant_a(np.asarray(a)[rows], np.asarray(sa)[:, rows])
    Bq = np.asarray(b)[cols]
    Bs = np.asarray(sb)[cols // TILE]
    B = e4m3.decode(Bq) * np.repeat(Bs.astype(np.float64), TILE, axis=1)
    return A @ B.T


def wgrad_f64(a, sa, b, sb) -> np.ndarray:
    """Weight-gradient GEMM in float64: both operands dequantized with one
    scale per row per 128 K (the activation-style layout [K/128][rows])."""
    return dequant_a(a, sa) @ dequant_a(b, sb).T


def wgrad_ref(a, sa, b, sb, d_in=None) -> np.ndarray:
    """FP32 weight gradient: fl32(sum), or with accumulation fl32(d_in + sum)
    (the float64 total rounded once)."""
    d = wgrad_f64(a, sa, b, sb)
    if d_in is not None:
        d = d + np.asarray(d_in, np.float32).astype(np.float64)
    return d.astype(np.float32)


def grouped_contiguous_f64(a, sa, b, sb, m_offsets) -> np.ndarray:
    """Contiguous layout: D[Mt][N] float64, NaN on rows outside every group."""
    a = np.asarray(a, np.uint8)
    Mt = a.shape[0]
    G, N, _ = np.asarray(b).shape
    offs = np.asarray(m_offsets, np.int64)
    d = np.full((Mt, N), np.nan)
    for g in range(G):
        lo, hi = int(offs[g]), int(offs[g + 1])
        if hi > lo:
            d[lo:hi] = gemm_f64(a[lo:hi], np.asarray(sa)[:, lo:hi], b[g], sb[g])
    return d


def grouped_masked_f64(a, sa, b, sb, masked_m) -> np.ndarray:
    """Masked layout: A[G][cap][K], sA[G][K/128][cap] -> D[G][cap][N] float64,
    NaN on rows at or beyond masked_m[g] (those rows are never written)."""
    a = np.asarray(a, np.uint8)
    G, cap, _ = a.shape
    N = np.asarray(b).shape[1]
    d = np.full((G, cap, N), np.nan)
    for g in range(G):
        c = int(min(max(int(masked_m[g]), 0), cap))
        if c:
            d[g, :c] = gemm_f64(a[g, :c], np.asarray(sa)[g][:, :c], b[g], sb[g])
    return d
