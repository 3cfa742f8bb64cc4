// Internal launchers (host side) of libfp8bs.  Arguments are already checked
// by the C ABI layer; these only configure grids and enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// 1x128 tiles of one row handled by one lane of k_quantize_1x128 (the grid's
// y dimension is ceil(K/128 / kQ1Tiles)); the C ABI bounds that grid with it.
constexpr int kQ1Tiles = 2;

hipError_t launch_quantize_1x128(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, bool pow2,
                                 hipStream_t stream);
hipError_t launch_quantize_t128x1(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt, float* st,
                                  bool pow2, hipStream_t stream);
hipError_t launch_quantize_128x128(const void* w, int64_t G, int64_t N, int64_t K, uint8_t* q, float* s, bool pow2,
                                   hipStream_t stream);
hipError_t launch_quantize_dual(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt, float* st,
                                bool pow2, hipStream_t stream);
hipError_t launch_transpose_128x128(const uint8_t* q, const float* s, int64_t G, int64_t N, int64_t K, uint8_t* qt,
                                   float* st, hipStream_t stream);
hipError_t launch_cast_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream);
// Bandwidth reference: dst_bytes written, ratio (1 or 2) times as many read.
hipError_t launch_stream_reference(const void* src, void* dst, int64_t dst_bytes, int ratio, hipStream_t stream);

// kWgrad: dense layout, but B carries one scale per row per 128 K ([K/128][N],
// like A) and D is FP32, optionally accumulated into.
enum GemmMode { kDense = 0, kContiguous = 1, kMasked = 2, kWgrad = 3 };

struct GemmProblem {
  const uint8_t* a;       // E4M3 activations
  const float* sa;        // 1x128 scales
  const uint8_t* b;       // E4M3 weights ([G][N][K] for grouped)
  const float* sb;        // 128x128 scales (kWgrad: 1x128 scales [K/128][N])
  void* d;                // output
  const int32_t* groups;  // m_offsets [G+1] (contiguous) or masked_m [G] (masked); device
  int64_t M;              // rows: dense M, contiguous Mt, masked cap
  int64_t N, K;
  int32_t G;              // number of groups (1 for dense)
  bool out_f32;
  bool accumulate;        // kWgrad: D += A B^T
  bool hw_scale;          // every scale a power of two: the MFMA applies them and accumulates
  GemmMode mode;
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);
// The tile (rows x columns) launch_gemm uses for p, and whether it runs the
// ping-pong main loop (host only).
void gemm_tile(const GemmProblem& p, int32_t& bm, int32_t& bn, int32_t& pp);
// The ping-pong kernel on 192x192 tiles (dense and contiguous layouts; the
// rows of sA must be a multiple of 4).
hipError_t launch_gemm_pp192(const GemmProblem& p, hipStream_t stream);
// The GEMM with a BF16 activation quantized 1x128 in its operand load (dense
// layout; p.a is the BF16 activation, p.sa unused; pow2: power-of-two tile
// scales), and the column tile it runs on (64 rows x that).
hipError_t launch_gemm_qa(const GemmProblem& p, bool pow2, hipStream_t stream);
int32_t gemm_qa_tile_n(int64_t N);

}  // namespace fp8bs
