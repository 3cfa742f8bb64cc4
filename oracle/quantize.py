"""Fine-grained FP8 quantizers (oracle).  Test infrastructure only.

What they compute, and where it comes from:

* 1x128 tiles for activations: page 1 (uniondaocoop.com post on DeepSeek's
  FP8 training framework), paragraph on fine-grained quantization -- each
  activation row is cut into tiles of 128 consecutive channels, every tile
  gets its own scale.
* 1x128 -> 128x1 conversion: the same page says activations cached in FP8
  for the backward pass are converted from 1x128 tiles to 128x1 tiles.  The
  input is the FP8 1x128 copy; each value is dequantized in FP32 and then
  requantized along the other axis (columns in blocks of 128 rows), and the
  result is written transposed so the new tiles are again contiguous rows.
* 128x128 blocks for weights: one scale per block of 128 output rows x 128
  input channels.  The pages only ask for scaling per group inside the MMA
  (page 2, "A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on
  hardware suggestions); the block shape is the workload's.
* Transposed weights: page 2, paragraph on hardware suggestions, asks for
  GEMMs on transposed operands.  The data gradient dX = dY W needs the
  weight transposed; a 128x128-block-scaled weight transposed is again
  block-scaled with the same codes and the transposed scale grid, so no
  requantization is involved.  Rows of W past the last multiple of 128 (a
  ragged N) become zero columns, so the transposed weight's K is a multiple
  of 128 (the activation gradient is quantized over the same padded width).
* Both tilings from one read of the BF16 activation: page 2, paragraph on
  hardware suggestions, asks for the FP8 cast to happen while activations
  move, so they are not read and written again just to quantize them.  The
  forward GEMM needs 1x128 tiles and the weight gradient 128x1 tiles
  (transposed); a single pass over the BF16 values can produce both.  By
  definition the 128x1 tiles of x are the 1x128 tiles of x^T, quantized from
  the BF16 values directly (one rounding, unlike the conversion from the
  cached FP8 copy above).
* Power-of-two scales: page 2, same paragraph as the 14-bit accumulation
  note, says some activations use scaling factors that are integral powers of
  two.  Read here as: round the FP32 scale UP to the next power of two, so no
  code can overflow.

Per tile (readings where the pages are silent):
  amax = max |x| over the tile (exact);
  s    = 1.0                         if amax == 0,
         fl32(amax / 448)            otherwise (correctly rounded FP32 divide;
                                     clamped below at 2^-149 so a nonzero
                                     tile never gets a zero scale);
  s    = 2^ceil(log2 s)              with the power-of-two option;
  q    = enc(fl32(x / s))            RNE to E4M3 with satfinite, after an FP32
                                     divide (not a multiply by a reciprocal).

Scale layouts (row-major, M contiguous for activations):
  quantize_1x128            x[R][C]  -> q[R][C],  s[C/128][R]
  quantize_transpose_128x1  q[M][K], s[K/128][M] -> qt[K][M], st[M/128][K]
  quantize_128x128          w[N][K]  -> q[N][K],  s[ceil(N/128)][K/128]
  quantize_dual             x[M][K]  -> q[M][K], s[K/128][M] (1x128) and
                                        qt[K][M], st[M/128][K] (128x1, transposed)
  transpose_128x128         q[N][K], s[ceil(N/128)][K/128] -> qt[K][Np], st[K/128][Np/128],
                            Np = 128 * ceil(N/128)
"""

import numpy as np

from . import bf16, e4m3

TILE = 128
_448 = np.float32(448.0)


def tile_scale(amax_f32, pow2: bool) -> np.ndarray:
    """Scale of a tile from its amax: fl32(amax/448), 1 for a zero tile,
    optionally rounded up to a power of two."""
    amax = np.asarray(amax_f32, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.divide(amax, _448, dtype=np.float32)
    # A nonzero tile never gets a zero scale: when amax/448 underflows FP32
    # (amax < 2^-140, unreachable from BF16 inputs) the smallest positive
    # FP32, 2^-149, is used instead.
    s = np.maximum(s, np.float32(2.0 ** -149))
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    if pow2:
        f, e = np.frexp(s.astype(np.float64))          # s = f * 2^e, f in [0.5, 1)
        s = np.where(f == 0.5, s.astype(np.float64), np.ldexp(1.0, e)).astype(np.float32)
    return s


def quantize_values(x_f32, s_f32) -> np.ndarray:
    """q = enc(fl32(x / s)) elementwise (s broadcast against x)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.divide(np.asarray(x_f32, np.float32), np.asarray(s_f32, np.float32),
                      dtype=np.float32)
    return e4m3.encode(y)


def quantize_rows_f32(x_f32, pow2: bool = False):
    """1x128 tiles along the last axis of a float32 matrix x[R][C].

    Returns (q[R][C] uint8, s[C/128][R] float32)."""
    x = np.asarray(x_f32, dtype=np.float32)
    R, C = x.shape
    if C % TILE:
        raise ValueError("number of columns must be a multiple of 128")
    tiles = x.reshape(R, C // TILE, TILE)
    amax = np.max(np.abs(tiles), axis=2)                      # [R, C/128]
    s = tile_scale(amax, pow2)                                # [R, C/128]
    q = quantize_values(tiles, s[:, :, None]).reshape(R, C)
    return q, np.ascontiguousarray(s.T)


def quantize_1x128(x_bf16_bits, pow2: bool = False):
    """BF16 activation x[M][K] (uint16 bits) -> (q[M][K], s[K/128][M])."""
    return quantize_rows_f32(bf16.to_f32(x_bf16_bits), pow2)


def dequantize_rows_f32(q, s) -> np.ndarray:
    """d = fl32(dec(q) * s) for 1x128-tiled q[R][C] with s[C/128][R].

    dec(q) has 4 significant bits and s has 24, so the float64 product is exact
    and the cast to float32 is the single FP32 rounding."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    srow = np.repeat(np.asarray(s, np.float32).T.astype(np.float64), TILE, axis=1)  # [R, C]
    return (e4m3.decode(q) * srow).astype(np.float32)


def quantize_transpose_128x1(q, s, pow2: bool = False):
    """1x128-tiled FP8 q[M][K], s[K/128][M]  ->  128x1 tiles, stored transposed:
    (qt[K][M], st[M/128][K]).  By definition this is quantize_rows_f32 applied
    to the transpose of the FP32-dequantized input."""
    q = np.asarray(q, dtype=np.uint8)
    M, K = q.shape
    if M % TILE or K % TILE:
        raise ValueError("M and K must be multiples of 128")
    d = dequantize_rows_f32(q, s)
    return quantize_rows_f32(np.ascontiguousarray(d.T), pow2)


def quantize_128x128(w_bf16_bits, pow2: bool = False):
    """Weight w[N][K] (uint16 BF16 bits; or [G][N][K]) -> (q, s) with one scale
    per block of up to 128 rows x 128 columns; s[ceil(N/128)][K/128] (or
    [G][...]).  A partial last row block takes its amax over its valid rows."""
    w = np.asarray(w_bf16_bits, dtype=np.uint16)
    if w.ndim == 3:
        outs = [quantize_128x128(w[g], pow2) for g in range(w.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    x = bf16.to_f32(w)
    N, K = x.shape
    if K % TILE:
        raise ValueError("K must be a multiple of 128")
    nb = -(-N // TILE)
    s = np.empty((nb, K // TILE), dtype=np.float32)
    q = np.empty((N, K), dtype=np.uint8)
    for i in range(nb):
        rows = x[i * TILE:(i + 1) * TILE]                     # <=128 rows
        blocks = rows.reshape(rows.shape[0], K // TILE, TILE)
        amax = np.max(np.abs(blocks), axis=(0, 2))            # [K/128]
        s[i] = tile_scale(amax, pow2)
        q[i * TILE:(i + 1) * TILE] = quantize_values(blocks, s[i][None, :, None]).reshape(rows.shape[0], K)
    return q, s


def transpose_128x128(q, s):
    """Block-scaled weight q[N][K], s[ceil(N/128)][K/128] (or [G][...]) ->
    the transposed weight as a block-scaled weight of the same kind:
    qt[K][Np] with qt[k][n] = q[n][k] for n < N and zero codes for
    N <= n < Np = 128*ceil(N/128); st[kb][nb] = s[nb][kb]."""
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.float32)
    if q.ndim == 3:
        outs = [transpose_128x128(q[g], s[g]) for g in range(q.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    N, K = q.shape
    if K % TILE:
        raise ValueError("K must be a multiple of 128")
    nb = -(-N // TILE)
    if s.shape != (nb, K // TILE):
        raise ValueError("scale grid does not match the weight")
    qt = np.zeros((K, nb * TILE), dtype=np.uint8)
    qt[:, :N] = q.T
    return qt, np.ascontiguousarray(s.T)


def quantize_dual(x_bf16_bits, pow2: bool = False):
    """BF16 x[M][K] (M, K multiples of 128) -> (q, s, qt, st): the 1x128
    quantization of x and the 128x1 quantization of x stored transposed, both
    from the BF16 values.  The second is by definition the 1x128 quantization
    of x^T."""
    x = np.asarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    if M % TILE or K % TILE:
        raise ValueError("M and K must be multiples of 128")
    q, s = quantize_1x128(x, pow2)
    qt, st = quantize_1x128(np.ascontiguousarray(x.T), pow2)
    return q, s, qt, st
