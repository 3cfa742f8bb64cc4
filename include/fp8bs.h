/*
 * fp8bs.h -- C ABI of libfp8bs: block-scaled FP8 GEMMs and the quantizers that
 * feed them, hand-written for AMD Instinct MI355X (gfx950).
 *
 * Method (surveyed pages):
 *   - page 1, the uniondaocoop.com board post that restates DeepSeek's FP8
 *     mixed-precision training framework: fine-grained quantization with one
 *     scale per 1x128 activation tile; FP8 GEMMs take FP8 inputs and write BF16
 *     or FP32; partial sums are copied into FP32 registers at a fixed interval
 *     along K; cached FP8 activations are converted from 1x128 to 128x1 tiles
 *     for the backward pass.
 *   - page 2, "A Deadly Mistake Uncovered on Deepseek China Ai ...": scaling
 *     factors restricted to integral powers of two for some activations; the
 *     request for MMA with per-group scaling.
 *   - page 4, "Deepseek veroeffentlicht Deepgemm ...", section
 *     "Schluesselmerkmale von DeepGemm": a dense layout and two MoE layouts.
 *
 * Formats.
 *   E4M3  : OCP 8-bit float, 1 sign / 4 exponent (bias 7) / 3 mantissa bits, no
 *           infinities, 0x7F/0xFF = NaN, largest finite 448.  Stored as bytes.
 *   BF16  : 16-bit brain float (upper half of a binary32), stored as uint16.
 *   Scales: binary32.
 *
 * Quantization rule (every quantizer; readings of points the pages leave
 * open): per tile, amax = max |x|; s = 1 if amax == 0, else
 * max(fl32(amax / 448), 2^-149) with a correctly rounded FP32 divide; with
 * FP8BS_SCALE_POW2, s is rounded up to the next power of two; every element is
 * encoded as E4M3(fl32(x / s)), round-to-nearest-even, saturating to +-448.
 * Results are bit-exact functions of the inputs.  Inputs must be finite.
 *
 * GEMM rule: D = A * B^T ("NT": both operands K-contiguous) with
 *   D[m][n] = sum over 128-wide K chunks kb of
 *             sA[kb][m] * sB[n/128][kb] * (sum_{k in kb} A[m][k] * B[n][k])
 * Each chunk's inner sum is formed in FP32 by the matrix cores and promoted
 * into a separate FP32 accumulator with its scale product (the pages'
 * promotion interval, here 128).  Output: BF16 (round-to-nearest-even) or
 * FP32.  Summation order differs from a plain dot product, so results agree
 * with an exact reference to within |d - ref| <= 8e-3 |ref| + 1e-3 rms(ref),
 * except that the matrix core sums a chunk's products in groups of 8 aligned
 * to the group's largest product with about 14 bits kept (the limited
 * accumulation page 2 describes for Hopper, inside one chunk): where chunk
 * partials cancel, an output may differ by up to that truncation bound more.
 *
 * Conventions shared by every entry point.
 *   - Pointers are device pointers (memory the current HIP device can read or
 *     write) unless stated otherwise; data pointers must be 16-byte aligned.
 *   - All tensors are dense row-major with no padding between rows.
 *   - The caller allocates, owns and frees every buffer; the library keeps no
 *     pointer after returning and allocates nothing.  The one call that needs
 *     scratch memory (fp8bs_gemm_fp8_blockscaled_splitk) takes it from the
 *     caller as a workspace argument; its _noalloc variant uses a fixed
 *     array the library holds on each GPU instead.
 *   - Every call enqueues its kernels on `stream` (NULL = the null stream) and
 *     returns without waiting; buffers must stay alive until the stream work
 *     completes.  Calls are re-entrant and thread-safe.
 *   - Arguments are checked before anything is launched; on any error nothing
 *     is launched and no memory is written.  Check order: sizes
 *     (FP8BS_ERR_SHAPE), flags / output dtype (FP8BS_ERR_FLAGS); then an empty
 *     problem (zero rows, columns or groups) returns FP8BS_OK without
 *     launching and may pass NULL pointers; otherwise null pointers
 *     (FP8BS_ERR_NULL), 16-byte alignment (FP8BS_ERR_ALIGN; the int32 group
 *     arrays need only 4), the current device (FP8BS_ERR_DEVICE).  The HIP
 *     runtime's last-error state is cleared before launching; a launch it
 *     rejects returns FP8BS_ERR_LAUNCH.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_ABI_VERSION 9

/* Same type as hipStream_t; declared here so the header needs no HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t* fp8bs_stream_t;

typedef enum {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL = 1,   /* a required pointer is NULL                        */
  FP8BS_ERR_SHAPE = 2,  /* a size is negative or breaks a divisibility rule  */
  FP8BS_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                  */
  FP8BS_ERR_FLAGS = 4,  /* unknown flag bits or output dtype                 */
  FP8BS_ERR_DEVICE = 5, /* no current HIP device, or it is not gfx950        */
  FP8BS_ERR_LAUNCH = 6  /* the HIP runtime rejected a kernel launch          */
} fp8bs_status;

/* Output dtypes of the GEMMs. */
enum { FP8BS_OUT_BF16 = 0, FP8BS_OUT_FP32 = 1 };

/*
 * Flags.  Quantizers: FP8BS_SCALE_POW2 rounds every scale up to a power of
 * two.  GEMMs (dense and grouped): FP8BS_SCALE_POW2 declares that every scale
 * of A and B is a power of two 2^e with -127 <= e <= 127 (the power-of-two
 * quantizers give that for every tile whose amax exceeds 448 * 2^-128); the
 * matrix core then applies the scales itself, as E8M0 exponents per operand
 * row and 32-wide K group, and adds each scaled 128-K chunk product to its own
 * FP32 accumulator, so the promotion takes no vector-ALU work (page 2,
 * "A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on hardware
 * suggestions: MMA that takes the group scales).  An output that depends on
 * any other scale value is NaN.
 */
enum { FP8BS_SCALE_POW2 = 1u };

/*
 * 1x128 activation quantization (page 1, paragraph on fine-grained tiles).
 *   x  : BF16 [M][K]            (input)
 *   q  : E4M3 [M][K]            (output)
 *   s  : FP32 [K/128][M]        (output; tile (m, kb) -> s[kb][m])
 * Requires M >= 0, K > 0, K % 128 == 0.  flags: 0 or FP8BS_SCALE_POW2.
 */
fp8bs_status fp8bs_quantize_1x128(const void* x, int64_t M, int64_t K,
                                  uint8_t* q, float* s, uint32_t flags,
                                  fp8bs_stream_t stream);

/*
 * 1x128 -> 128x1 transpose-requantize of a cached FP8 activation (page 1,
 * paragraph on FP8 activation caching and the backward-pass tile conversion).
 * Each value is dequantized as d = fl32(E4M3(q) * s[kb][m]); every column k
 * of each 128-row block mb is then requantized with the quantization rule and
 * written transposed, so the new tiles are contiguous rows of qt.
 *   q  : E4M3 [M][K],  s  : FP32 [K/128][M]        (input, 1x128 tiles)
 *   qt : E4M3 [K][M],  st : FP32 [M/128][K]        (output; tile (k, mb) ->
 *                                                    st[mb][k])
 * Requires M >= 0, K >= 0, M % 128 == 0, K % 128 == 0.
 */
fp8bs_status fp8bs_quantize_transpose_128x1(const uint8_t* q, const float* s,
                                            int64_t M, int64_t K,
                                            uint8_t* qt, float* st,
                                            uint32_t flags,
                                            fp8bs_stream_t stream);

/*
 * Dual quantization of a BF16 activation from one read of it (page 2, "A
 * Deadly Mistake Uncovered on Deepseek China Ai", paragraph on hardware
 * suggestions: quantize while activations move instead of reading and
 * writing them again).  Produces the 1x128 tiles of x (the forward GEMM's A
 * operand) and the 128x1 tiles of x stored transposed (the weight
 * gradient's operand), both quantized from the BF16 values: qt/st equal the
 * 1x128 quantization of x^T.  (fp8bs_quantize_transpose_128x1 instead
 * requantizes the cached FP8 copy, as page 1 describes.)
 *   x  : BF16 [M][K]                              (input)
 *   q  : E4M3 [M][K],  s  : FP32 [K/128][M]       (1x128 tiles)
 *   qt : E4M3 [K][M],  st : FP32 [M/128][K]       (128x1 tiles, transposed)
 * Requires M >= 0, K >= 0, M % 128 == 0, K % 128 == 0.  flags: 0 or
 * FP8BS_SCALE_POW2.
 */
fp8bs_status fp8bs_quantize_dual(const void* x, int64_t M, int64_t K,
                                 uint8_t* q, float* s, uint8_t* qt, float* st,
                                 uint32_t flags, fp8bs_stream_t stream);

/*
 * 128x128 block quantization of (optionally batched) weights: one scale per
 * block of up to 128 rows x 128 columns; a partial last row block uses its
 * valid rows only.  Weights for the GEMMs below are laid out this way.
 *   w  : BF16 [G][N][K]                     (input; G = 1 for one matrix)
 *   q  : E4M3 [G][N][K]                     (output)
 *   s  : FP32 [G][ceil(N/128)][K/128]       (output)
 * Requires G >= 0, N >= 0, K > 0, K % 128 == 0.
 */
fp8bs_status fp8bs_quantize_128x128(const void* w, int64_t G, int64_t N, int64_t K,
                                    uint8_t* q, float* s, uint32_t flags,
                                    fp8bs_stream_t stream);

/*
 * Transposed block-scaled weight, for the data gradient dX = dY W (page 2,
 * "A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on hardware
 * suggestions: GEMMs on transposed operands).  A 128x128-block-scaled weight
 * transposed is again block-scaled, with the same codes and the transposed
 * scale grid; nothing is requantized.  Rows of W past N become zero columns
 * up to Np = 128 * ceil(N/128), so the result is a GEMM weight operand with
 * K' = Np (quantize the activation gradient over the same zero-padded width).
 *   q  : E4M3 [G][N][K],   s  : FP32 [G][ceil(N/128)][K/128]   (input)
 *   qt : E4M3 [G][K][Np],  st : FP32 [G][K/128][Np/128]        (output;
 *        qt[g][k][n] = q[g][n][k] for n < N, 0 otherwise;
 *        st[g][kb][nb] = s[g][nb][kb])
 * Requires G >= 0, N >= 0, N % 16 == 0, K >= 0, K % 128 == 0; q and qt
 * 16-byte aligned, s and st 4-byte aligned.
 */
fp8bs_status fp8bs_transpose_128x128(const uint8_t* q, const float* s,
                                     int64_t G, int64_t N, int64_t K,
                                     uint8_t* qt, float* st,
                                     fp8bs_stream_t stream);

/*
 * Dense block-scaled FP8 GEMM (page 1, paragraphs on FP8 GEMM inputs/outputs
 * and FP32 promotion; page 4, section "Schluesselmerkmale von DeepGemm",
 * dense layout).  D = A * B^T.
 *   a  : E4M3 [M][K],   sa : FP32 [K/128][M]              (1x128 tiles)
 *   b  : E4M3 [N][K],   sb : FP32 [ceil(N/128)][K/128]    (128x128 blocks)
 *   d  : [M][N], BF16 (out_dtype = FP8BS_OUT_BF16) or FP32 (FP8BS_OUT_FP32)
 *   flags : 0, or FP8BS_SCALE_POW2 (power-of-two scales applied by the
 *           matrix core; see the flags above)
 * Requires M >= 0, N >= 0, N % 16 == 0, K > 0, K % 128 == 0, and (the
 * kernels address operand panels and scale arrays with 32-bit offsets)
 * 256 * K < 2^31 and 4 * (K/128) * M < 2^31 and 4 * (K/128) * ceil(N/128)
 * < 2^31; the grouped and weight-gradient calls apply the same limits to
 * their own scale arrays (per group, with cap or Mt rows).  Larger problems
 * return FP8BS_ERR_SHAPE.
 */
fp8bs_status fp8bs_gemm_fp8_blockscaled(const uint8_t* a, const float* sa,
                                        const uint8_t* b, const float* sb,
                                        void* d, int64_t M, int64_t N, int64_t K,
                                        int32_t out_dtype, uint32_t flags,
                                        fp8bs_stream_t stream);

/*
 * The dense GEMM above with its K chunks split over several workgroups, for
 * shapes whose output tiles are too few to occupy the GPU: decode-sized
 * activations against a projection (page 4, "Deepseek veroeffentlicht
 * Deepgemm", Table 1 "DeepGemm Performance Benchmarks": its row with M = 64,
 * N = 2112, K = 7168; page 2, paragraph on decoding, where few tokens make the
 * GEMM memory-bound).  It splits only where K has at least 32 chunks (with at
 * least two per split).  Each output tile (64 x 64 for M <= 128, else 128 x 96)
 * is computed by S workgroups, one
 * per range of K chunks, each promoting its chunks into FP32 exactly as the
 * unsplit GEMM does; the S FP32 partials are then added in split order and
 * rounded once to the output type.  The result equals the unsplit GEMM's up to
 * the order of its FP32 additions (bit for bit where those are exact), and is
 * the same on every run.  Where S would be 1 (fp8bs_gemm_splitk_workspace
 * reports 0 bytes) the call runs the unsplit GEMM and uses no workspace.
 *   a, sa, b, sb, d, M, N, K, out_dtype, flags : as fp8bs_gemm_fp8_blockscaled
 *   workspace       : device scratch of workspace_bytes bytes, at least what
 *                     fp8bs_gemm_splitk_workspace reports for M, N, K (may be
 *                     NULL when that is 0); 16-byte aligned.  Its contents on
 *                     entry do not matter and are overwritten; calls that
 *                     share a workspace must not overlap in time.
 *   workspace_bytes : its size
 * Requires what fp8bs_gemm_fp8_blockscaled requires; a workspace smaller than
 * needed returns FP8BS_ERR_SHAPE.
 */
fp8bs_status fp8bs_gemm_fp8_blockscaled_splitk(const uint8_t* a, const float* sa,
                                               const uint8_t* b, const float* sb,
                                               void* d, int64_t M, int64_t N, int64_t K,
                                               int32_t out_dtype, uint32_t flags,
                                               void* workspace, int64_t workspace_bytes,
                                               fp8bs_stream_t stream);

/*
 * fp8bs_gemm_fp8_blockscaled_splitk without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The partials go to a
 * scratch array the library holds in each GPU's memory: 12 MiB (12582912
 * bytes, 256 partial tiles), which covers every problem this call splits;
 * a problem whose split would need more returns FP8BS_ERR_SHAPE (none does
 * under the current split rule).  Nothing is allocated at call time; the
 * array's device address is looked up on the first call on each device.
 * Every call on one GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (other streams, other threads) race and may return wrong
 * results: serialize them.  The array needs no clearing: each call writes
 * every byte it reads.  Arguments and results as
 * fp8bs_gemm_fp8_blockscaled_splitk.
 */
fp8bs_status fp8bs_gemm_fp8_blockscaled_splitk_noalloc(const uint8_t* a, const float* sa,
                                                       const uint8_t* b, const float* sb,
                                                       void* d, int64_t M, int64_t N, int64_t K,
                                                       int32_t out_dtype, uint32_t flags,
                                                       fp8bs_stream_t stream);

/*
 * Workspace bytes fp8bs_gemm_fp8_blockscaled_splitk needs for M x N x K
 * (host-side query, no device): 0 when the call would not split.
 *   bytes : HOST pointer, receives the size
 * Requires the sizes fp8bs_gemm_fp8_blockscaled requires.
 */
fp8bs_status fp8bs_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/*
 * Dense block-scaled FP8 GEMM on a BF16 activation, quantized on the way in
 * (page 2, "A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on
 * hardware suggestions: cast to FP8 during the move from global to shared
 * memory; page 1, paragraph on 1x128 activation tiles).
 * D = Q(x) * B^T, where Q(x) is what fp8bs_quantize_1x128 makes of x (same
 * codes and tile scales, power-of-two scales with FP8BS_SCALE_POW2); the
 * result equals fp8bs_quantize_1x128 followed by fp8bs_gemm_fp8_blockscaled
 * with flags 0, bit for bit.  The codes are not stored.  Every 64 x 128
 * output tile quantizes its activation rows itself, so the call pays off
 * where few column tiles share them (small N).
 *   x  : BF16 [M][K]                                      (input)
 *   b  : E4M3 [N][K],   sb : FP32 [ceil(N/128)][K/128]    (128x128 blocks)
 *   d  : [M][N], BF16 (out_dtype = FP8BS_OUT_BF16) or FP32 (FP8BS_OUT_FP32)
 *   flags : 0, or FP8BS_SCALE_POW2 (the activation's tile scales rounded up
 *           to powers of two; the promotion stays in software)
 * Requires M >= 0, N >= 0, N % 16 == 0, K > 0, K % 128 == 0, 256 * K < 2^31
 * and 4 * (K/128) * ceil(N/128) < 2^31; larger problems return
 * FP8BS_ERR_SHAPE.  Pointers as for fp8bs_gemm_fp8_blockscaled.
 */
fp8bs_status fp8bs_gemm_fused_quantize(const void* x, const uint8_t* b, const float* sb,
                                       void* d, int64_t M, int64_t N, int64_t K,
                                       int32_t out_dtype, uint32_t flags,
                                       fp8bs_stream_t stream);

/*
 * Weight-gradient GEMM (page 1, paragraphs on caching FP8 activations and on
 * converting 1x128 tiles to 128x1 tiles for the backward pass): dW = dY^T X
 * contracts over tokens, so both operands carry one scale per row per 128
 * tokens -- the transposed, requantized activations that
 * fp8bs_quantize_transpose_128x1 produces.  D = A * B^T in FP32, K = tokens.
 *   a  : E4M3 [M][K],   sa : FP32 [K/128][M]     (e.g. dY^T: M = output features)
 *   b  : E4M3 [N][K],   sb : FP32 [K/128][N]     (e.g. X^T:  N = input features)
 *   d  : FP32 [M][N]; accumulate = 1 adds the product to d's contents
 *        (gradient accumulation), 0 overwrites them.
 *   flags : 0, or FP8BS_SCALE_POW2: every scale is a power of two 2^e with
 *        -127 <= e <= 127 and the scaled MFMA applies both operands' row
 *        scales itself (page 2, paragraph on MMA with per-group scaling);
 *        outputs that depend on any other scale are NaN, as for the dense
 *        GEMM.
 * Requires M >= 0, N >= 0, N % 16 == 0, K > 0, K % 128 == 0, accumulate in
 * {0, 1} and flags in {0, FP8BS_SCALE_POW2} (else FP8BS_ERR_FLAGS).
 */
fp8bs_status fp8bs_gemm_fp8_wgrad(const uint8_t* a, const float* sa,
                                  const uint8_t* b, const float* sb,
                                  float* d, int64_t M, int64_t N, int64_t K,
                                  int32_t accumulate, uint32_t flags,
                                  fp8bs_stream_t stream);

/*
 * Grouped GEMM, contiguous MoE layout (page 4, section "Schluesselmerkmale
 * von DeepGemm", the first of the two MoE layouts): the rows of every group
 * are concatenated; group g owns rows [m_offsets[g], m_offsets[g+1]) of A and
 * D and uses weight matrix b[g] with scales sb[g].
 *   a  : E4M3 [Mt][K],   sa : FP32 [K/128][Mt]
 *   b  : E4M3 [G][N][K], sb : FP32 [G][ceil(N/128)][K/128]
 *   d  : [Mt][N] BF16 or FP32
 *   m_offsets : int32 [G+1], DEVICE memory, read on the device only (the call
 *               never synchronizes).  Must be non-decreasing with m_offsets[0]
 *               == 0, every difference a multiple of 128, m_offsets[G] <= Mt;
 *               violations are not detected and give undefined results.  Rows
 *               at or past m_offsets[G] are not written.  Empty groups are
 *               allowed.
 *   flags : 0 or FP8BS_SCALE_POW2, as for the dense GEMM.
 * Requires G >= 0, Mt >= 0, Mt % 128 == 0, N % 16 == 0, K > 0, K % 128 == 0.
 */
fp8bs_status fp8bs_grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa,
                                               const uint8_t* b, const float* sb,
                                               void* d, const int32_t* m_offsets,
                                               int32_t G, int64_t Mt, int64_t N, int64_t K,
                                               int32_t out_dtype, uint32_t flags,
                                               fp8bs_stream_t stream);

/*
 * Grouped GEMM, masked MoE layout for decoding (page 4, the second MoE layout;
 * page 2, paragraph on decoding: a few hundred tokens per expert at most, so
 * the step is bound by memory, not compute): every group has a fixed
 * capacity of rows and a valid count that lives on the device.
 *   a  : E4M3 [G][cap][K],  sa : FP32 [G][K/128][cap]
 *   b  : E4M3 [G][N][K],    sb : FP32 [G][ceil(N/128)][K/128]
 *   d  : [G][cap][N] BF16 or FP32
 *   masked_m : int32 [G], DEVICE memory, read on the device only; values are
 *              clamped to [0, cap].  Rows at or past masked_m[g] of group g
 *              are neither used nor written (d keeps its previous contents).
 *   flags : 0 or FP8BS_SCALE_POW2, as for the dense GEMM.
 * Requires G >= 0, cap >= 0, N % 16 == 0, K > 0, K % 128 == 0.
 */
fp8bs_status fp8bs_grouped_gemm_fp8_masked(const uint8_t* a, const float* sa,
                                           const uint8_t* b, const float* sb,
                                           void* d, const int32_t* masked_m,
                                           int32_t G, int64_t cap, int64_t N, int64_t K,
                                           int32_t out_dtype, uint32_t flags,
                                           fp8bs_stream_t stream);

/*
 * Elementwise FP32 -> E4M3 cast with the encoding used by every quantizer
 * (round-to-nearest-even, +-inf and finite overflow saturate to +-448, the
 * sign of zero is kept, NaN maps to the NaN code of the same sign).
 *   x : FP32 [n] (input),  q : E4M3 [n] (output).  Requires n >= 0.
 */
fp8bs_status fp8bs_cast_f32_to_e4m3(const float* x, int64_t n, uint8_t* q,
                                    fp8bs_stream_t stream);

/*
 * Bandwidth reference (not a step of the method): streams src to dst with
 * nontemporal 16-byte loads, reading src_bytes and writing dst_bytes, where
 * src_bytes is dst_bytes (a copy, nontemporal 16-byte stores) or
 * 2 * dst_bytes (8-byte piece i of dst = (w0 ^ w1, w2 ^ w3) of the 32-bit
 * words of 16-byte piece i of src, ordinary stores).  The 1x128 quantizer is
 * a 2:1 read:write stream and the transposing requantizer a 1:1 stream; the
 * benchmark sets them against this.
 *   src, dst : DEVICE pointers, 16-byte aligned, not overlapping.
 * Requires dst_bytes >= 0, dst_bytes % 16 == 0.
 */
fp8bs_status fp8bs_stream_reference(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                    fp8bs_stream_t stream);

/*
 * Tile a GEMM call would run on (host-side query: no device, no launch; for
 * tests and tuning, not part of the method the pages describe).
 *   layout : 0 dense (fp8bs_gemm_fp8_blockscaled), 1 contiguous grouped,
 *            2 masked grouped, 3 weight gradient, 4 dense on a BF16
 *            activation (fp8bs_gemm_fused_quantize)
 *   rows   : M (dense, weight gradient, BF16 activation), Mt (contiguous)
 *            or cap (masked)
 *   N, K, G, flags : as passed to that call (G = 1 for dense and weight
 *            gradient)
 *   tile_m, tile_n : HOST pointers, receive the output tile (rows x columns
 *            per workgroup)
 *   ping_pong : HOST pointer, receives 1 if the tile runs the ping-pong main
 *            loop (two wave groups alternating fragment loads and MFMAs),
 *            0 otherwise
 * The size and flag checks of the named call apply (same status codes);
 * null output pointers give FP8BS_ERR_NULL.
 */
fp8bs_status fp8bs_gemm_tile(int32_t layout, int64_t rows, int64_t N, int64_t K, int32_t G,
                             uint32_t flags, int32_t* tile_m, int32_t* tile_n, int32_t* ping_pong);

/* Static, NUL-terminated description of a status code (host memory). */
const char* fp8bs_status_str(fp8bs_status status);

/* FP8BS_ABI_VERSION of the built library. */
int32_t fp8bs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
