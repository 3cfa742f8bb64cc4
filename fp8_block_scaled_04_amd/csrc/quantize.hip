// Fine-grained FP8 quantizers for gfx950.
//
//   quantize_1x128            BF16 [M][K] -> E4M3 [M][K] + FP32 [K/128][M]
//   quantize_transpose_128x1  E4M3 [M][K] + [K/128][M] -> E4M3 [K][M] + FP32 [M/128][K]
//   quantize_128x128          BF16 [G][N][K] -> E4M3 + FP32 [G][ceil(N/128)][K/128]
//   cast_f32_to_e4m3          FP32 [n] -> E4M3 [n]
//
// Method: page 1 (the uniondaocoop.com post on DeepSeek's FP8 training
// framework), paragraphs on 1x128 activation tiles and on converting cached
// FP8 activations to 128x1 tiles for the backward pass; page 2 ("A Deadly
// Mistake Uncovered on Deepseek China Ai"), power-of-two scaling factors.
// Per tile: amax, s = fl32(amax/448) (see tile_scale), q = E4M3(fl32(x/s)).
//
// All four kernels are bound by HBM bandwidth: 128-bit loads and stores, tile
// amax by DPP row reductions, no LDS except for the transpose.
#include <type_traits>

#include "quant_common.h"
#include "launch.h"

namespace fp8bs {
namespace {

// Streaming (nontemporal) 16-byte loads and 16-byte stores: every byte is
// touched once, and on MI355X the nontemporal forms move a 2:1 read:write
// stream about 10% faster than cached ones (6.1 vs 5.6 TB/s, measured).  The
// 1x128 quantizer's codes are the exception: written with ordinary stores its
// 8192x7168 launch takes 30.7 instead of 33.4 us, and the GEMM that reads
// them next finds them in the cache (quantize + 4096x2112x7168 GEMM: 95 ->
// 89 us); cached loads of its input, or cached stores in the transposing
// quantizers, were slower.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 nt_load16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Batched tile scales.  A lane holds partial maxima of several tiles, each
// tile spread over a group of lanes.  A reduce-scatter across the group (at
// each exchange a lane keeps half of its tiles and takes the maximum with its
// partner's copy of that half, the partner keeping the other half) leaves
// every lane with the full maximum of one tile, so a lane computes a single
// tile scale and DPP broadcasts give every lane the scales of the tiles it
// quantizes.  Every DPP source lane lies inside its row (no lane is out of
// range).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm 1,0,3,2: lane i ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm 2,3,0,1: lane i ^ 2
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i ^ 7 (within 8 lanes)
constexpr int kDppXor8 = 0x128;        // row_ror:8: lane i ^ 8 (within the row of 16)
constexpr int kDppRowBcast = 0x150;    // row_newbcast:n: lane n of the row

// Lane j of the quad, to every lane of the quad.
__device__ __forceinline__ float quad_bcast(float v, int j) {
  switch (j) {
    case 0: return dpp<0x00>(v);
    case 1: return dpp<0x55>(v);
    case 2: return dpp<0xAA>(v);
    default: return dpp<0xFF>(v);
  }
}
// Lane n (even) of the row, to every lane of the row.
__device__ __forceinline__ float row_bcast(float v, int n) {
  switch (n) {
    case 0: return dpp<kDppRowBcast + 0>(v);
    case 2: return dpp<kDppRowBcast + 2>(v);
    case 4: return dpp<kDppRowBcast + 4>(v);
    case 6: return dpp<kDppRowBcast + 6>(v);
    case 8: return dpp<kDppRowBcast + 8>(v);
    case 10: return dpp<kDppRowBcast + 10>(v);
    case 12: return dpp<kDppRowBcast + 12>(v);
    default: return dpp<kDppRowBcast + 14>(v);
  }
}
// One exchange: of its 2H values the lane keeps the upper half if `upper`,
// else the lower, and sends the other half to its partner (lane CTRL names).
template <int CTRL, int H>
__device__ __forceinline__ void scatter_max(const float (&v)[2 * H], float (&out)[H], bool upper) {
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float keep = upper ? v[H + k] : v[k];
    const float send = upper ? v[k] : v[H + k];
    out[k] = __builtin_fmaxf(keep, dpp<CTRL>(send));
  }
}
// am: the lane's maxima of four columns whose lanes are the 8 of its half
// row.  Returns the maximum of column (lane & 3) over those 8 lanes.
__device__ __forceinline__ float colgroup_max(const float (&am)[4], int lane) {
  float a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = __builtin_fmaxf(am[j], dpp<kDppHalfMirror>(am[j]));
  float b[2], c[1];
  scatter_max<kDppXor2, 2>(a, b, (lane & 2) != 0);
  scatter_max<kDppXor1, 1>(b, c, (lane & 1) != 0);
  return c[0];
}
// am: the lane's maxima of eight tiles spread over its row of 16 lanes.
// Returns the row maximum of tile (lane >> 1) & 7.
__device__ __forceinline__ float row_max8(const float (&am)[8], int lane) {
  float a[4], b[2], c[1];
  scatter_max<kDppXor8, 4>(am, a, (lane & 8) != 0);
  scatter_max<kDppHalfMirror, 2>(a, b, (lane & 4) != 0);   // partner i ^ 7: the other bit-2 half
  scatter_max<kDppXor2, 1>(b, c, (lane & 2) != 0);
  return __builtin_fmaxf(c[0], dpp<kDppXor1>(c[0]));
}
// am: the lane's maxima of two tiles spread over its row of 16 lanes.
// Returns the row maximum of tile (lane >> 3) & 1.
__device__ __forceinline__ float row_max2(const float (&am)[2], int lane) {
  float a[1];
  scatter_max<kDppXor8, 1>(am, a, (lane & 8) != 0);
  float v = a[0];
  v = __builtin_fmaxf(v, dpp<kDppHalfMirror>(v));
  v = __builtin_fmaxf(v, dpp<kDppXor2>(v));
  return __builtin_fmaxf(v, dpp<kDppXor1>(v));
}

// ---------------------------------------------------------------------------
// 1x128: one tile = 16 lanes (one DPP row) x 8 BF16 each (one 16-byte load).
// A workgroup of 256 lanes covers 16 rows; each lane walks kQ1Tiles tiles of its
// row so that kQ1Tiles loads are in flight before any arithmetic.  Scales of 16
// consecutive rows are written together (s is [K/128][M], M contiguous).
// ---------------------------------------------------------------------------


template <bool POW2, bool SCALED>
__device__ __forceinline__ uint2 quantize8(uint4 v, const TileScale& t) {
  float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = quot<POW2>(SCALED ? x[i] * t.sx : x[i], t);
  return make_uint2(pack4_e4m3(y[0], y[1], y[2], y[3]), pack4_e4m3(y[4], y[5], y[6], y[7]));
}

// max |x| over the 8 BF16 of a 16-byte word
__device__ __forceinline__ float absmax8(uint4 w) {
  const float a = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(bf16_lo(w.x)), __builtin_fabsf(bf16_hi(w.x))),
                                  __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.y)), __builtin_fabsf(bf16_hi(w.y))));
  const float b = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(bf16_lo(w.z)), __builtin_fabsf(bf16_hi(w.z))),
                                  __builtin_fmaxf(__builtin_fabsf(bf16_lo(w.w)), __builtin_fabsf(bf16_hi(w.w))));
  return __builtin_fmaxf(a, b);
}

template <bool POW2>
__global__ __launch_bounds__(256) void k_quantize_1x128(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane16 = threadIdx.x & 15;
  const int64_t m = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t KT = K / 128;
  const int64_t kb0 = (int64_t)blockIdx.y * kQ1Tiles;
  const bool row_ok = m < M;

  uint4 v[kQ1Tiles];
#pragma unroll
  for (int t = 0; t < kQ1Tiles; ++t) {
    const int64_t kb = kb0 + t;
    v[t] = make_uint4(0, 0, 0, 0);
    if (row_ok && kb < KT)
      v[t] = nt_load16(x + m * K + kb * 128 + lane16 * 8);
  }
  static_assert(kQ1Tiles == 2, "the tile maxima are reduced two at a time");
  float am[kQ1Tiles];
#pragma unroll
  for (int t = 0; t < kQ1Tiles; ++t) am[t] = absmax8(v[t]);
  // Lane l16 computes the scale of tile (l16 >> 3); tile t's is broadcast
  // from lane 8t of the row.
  const TileScale mine = tile_scale<POW2>(row_max2(am, lane16));
  auto run = [&](auto scaled) {
    constexpr bool SC = decltype(scaled)::value;
#pragma unroll
    for (int t = 0; t < kQ1Tiles; ++t) {
      const int64_t kb = kb0 + t;
      TileScale ts;
      ts.ss = row_bcast(mine.ss, 8 * t);
      ts.r = row_bcast(mine.r, 8 * t);
      ts.sx = SC ? row_bcast(mine.sx, 8 * t) : 1.0f;
      const uint2 out = quantize8<POW2, SC>(v[t], ts);
      if (row_ok && kb < KT) *reinterpret_cast<uint2*>(q + m * K + kb * 128 + lane16 * 8) = out;
    }
  };
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(mine.sx != 1.0f) != 0, 0))
    run(std::true_type{});
  else
    run(std::false_type{});
  const int64_t kbs = kb0 + (lane16 >> 3);
  if (row_ok && (lane16 & 7) == 0 && kbs < KT) s[kbs * M + m] = mine.s;
}

// Sixteen values of one tile -> sixteen codes (byte i = value i).  SCALED:
// the tile is one of those with amax < 2^-60, evaluated on x * 2^64.  The
// callers branch on a wave-uniform flag, so the common case carries no
// per-element multiply or select.
template <bool POW2, bool SCALED>
__device__ __forceinline__ uint4 quantize16(const float (&x)[16], const TileScale& t) {
  uint32_t packed[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = quot<POW2>(SCALED ? x[4 * k + e] * t.sx : x[4 * k + e], t);
    packed[k] = pack4_e4m3(y[0], y[1], y[2], y[3]);
  }
  return make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

// The column pass shared by the transposing quantizers.  The lane holds 16
// rows of four columns (d[j][i]: column j, row i; am[j]: their maxima); the
// 8 lanes of its half row hold the column group's 128 rows.  Lane l computes
// the scale of column l & 3 and writes it (lanes 0..3 of the group, to
// srow[l & 3]); column j's codes go to qrow + j * ld as 16 contiguous bytes.
template <bool POW2>
__device__ __forceinline__ void requant_columns(const float (&d)[4][16], const float (&am)[4], int l,
                                                uint8_t* qrow, int64_t ld, float* srow) {
  const TileScale mine = tile_scale<POW2>(colgroup_max(am, l));
  auto run = [&](auto scaled) {
    constexpr bool SC = decltype(scaled)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      TileScale ts;
      ts.ss = quad_bcast(mine.ss, j);
      ts.r = quad_bcast(mine.r, j);
      ts.sx = SC ? quad_bcast(mine.sx, j) : 1.0f;
      nt_store16(qrow + j * ld, quantize16<POW2, SC>(d[j], ts));
    }
  };
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(mine.sx != 1.0f) != 0, 0))
    run(std::true_type{});
  else
    run(std::false_type{});
  if ((l & 4) == 0) __builtin_nontemporal_store(mine.s, srow + (l & 3));
}

// ---------------------------------------------------------------------------
// 1x128 -> 128x1 transpose-requantize.  One workgroup per 128x128 tile
// (rows mb, columns kb).
//
// Phase 1 stages the tile's 16 KB of codes (eight lanes per 128-byte row,
// four rows per lane) and its 128 row scales in LDS.
//
// Phase 2: lane l of wave w owns rows 16*rg .. 16*rg+15 (rg = l % 8) of
// columns 4*c4 .. 4*c4+3 (c4 = 8*w + l / 8), read as sixteen 4-byte LDS
// words.  It dequantizes d = fl32(dec(q) * s_row), takes per-column maxima
// over its 16 rows, and combines them with the 7 other lanes of its column
// group (adjacent lanes, DPP) into the column amax.  It then requantizes and
// writes, per column, 16 contiguous bytes of the transposed row; the eight
// lanes of a column group write one whole 128-byte line.
//
// LDS layout: row r starts at (r + (r >= 64)) * 128 and its 4-byte word c4
// is stored at word c4 ^ (8 * ((r / 16) % 4)).  In phase 2 the 64 lanes of a
// wave then read 64 different banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int t_row(int r) { return r + (r >= 64 ? 1 : 0); }
__device__ __forceinline__ int t_swz(int r) { return 8 * ((r >> 4) & 3); }

template <bool POW2>
__global__ __launch_bounds__(256) void k_quantize_t128x1(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                          int64_t M, int64_t K,
                                                          uint8_t* __restrict__ qt, float* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[129 * 128];
  __shared__ __attribute__((aligned(16))) float rs[128];
  const int64_t mb = blockIdx.x, kb = blockIdx.y;
  const int t = threadIdx.x;
  {
    const int seg = t & 7;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * i + (t >> 3);
      v[i] = nt_load16(q + (mb * 128 + r) * K + kb * 128 + seg * 16);
    }
    uint4 sv = make_uint4(0, 0, 0, 0);
    if (t < 32) sv = nt_load16(s + kb * M + mb * 128 + 4 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * i + (t >> 3);
      // 16-byte segment seg holds words 4*seg .. 4*seg+3; the word swizzle
      // (a multiple of 8) moves it to segment seg ^ (swz / 4).
      *reinterpret_cast<uint4*>(codes + t_row(r) * 128 + 16 * (seg ^ (t_swz(r) >> 2))) = v[i];
    }
    if (t < 32) *reinterpret_cast<uint4*>(rs + 4 * t) = sv;
  }
  __syncthreads();
  const int l = t & 63, w = t >> 6;
  const int rg = l & 7, c4 = 8 * w + (l >> 3);
  uint32_t wv[16];
  float rsv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    wv[i] = *reinterpret_cast<const uint32_t*>(codes + t_row(r) * 128 + 4 * (c4 ^ t_swz(r)));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = *reinterpret_cast<const float4*>(rs + 16 * rg + 4 * i);
    rsv[4 * i] = f.x; rsv[4 * i + 1] = f.y; rsv[4 * i + 2] = f.z; rsv[4 * i + 3] = f.w;
  }
  float d[4][16];
  float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // the four codes of the word, two per (exact) packed conversion
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[i], false);
    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[i], true);
    const float dec[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[j][i] = dec[j] * rsv[i];
      am[j] = __builtin_fmaxf(am[j], __builtin_fabsf(d[j][i]));
    }
  }
  requant_columns<POW2>(d, am, l, qt + (kb * 128 + 4 * c4) * M + mb * 128 + 16 * rg, M,
                        st + mb * K + kb * 128 + 4 * c4);
}

// ---------------------------------------------------------------------------
// Dual quantization: the 1x128 tiles of a BF16 activation and its 128x1 tiles
// (stored transposed) from one read of it (page 2, paragraph on hardware
// suggestions: cast while the activations move instead of reading and
// writing them again).  One workgroup per 128x128 tile (x = row block mb,
// y = column block kb).
//
// Row pass: instruction i of wave w loads rows 32w + 4i + l/16 (sixteen
// lanes per 256-byte row, 8 BF16 each); a row's tile amax is a DPP row max.
// The lane writes its 8 codes (ordinary stores: the forward GEMM reads them
// next) and stages its values in LDS.
//
// Column pass: lane (rg = l % 8, cg = 8w + l / 8) reads rows 16rg .. 16rg+15
// of columns 4cg .. 4cg+3 as 8-byte LDS words, takes the column maxima over
// them and over the 8 lanes of its column group (DPP), requantizes, and
// writes per column 16 contiguous codes of the transposed row (8 lanes = one
// 128-byte line).
//
// LDS: row r (256 bytes) holds its 8-byte word c8 at word c8 ^ 8*((r/16) % 4),
// so the 64 lanes of a column-pass read hit 32 different words of the banks
// (two lanes per word pair: the minimum for 64 x 8 bytes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int d_swz(int r) { return 8 * ((r >> 4) & 3); }
__device__ __forceinline__ float bf16_at(uint2 w, int j) {
  return j == 0 ? bf16_lo(w.x) : j == 1 ? bf16_hi(w.x) : j == 2 ? bf16_lo(w.y) : bf16_hi(w.y);
}

template <bool POW2>
__global__ __launch_bounds__(256) void k_quantize_dual(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       uint8_t* __restrict__ q, float* __restrict__ s,
                                                       uint8_t* __restrict__ qt, float* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * 128];
  const int64_t mb = blockIdx.x, kb = blockIdx.y;
  const int t = threadIdx.x;
  const int l = t & 63, w = t >> 6;
  {
    const int lr = l >> 4, l16 = l & 15;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 32 * w + 4 * i + lr;
      v[i] = nt_load16(x + (mb * 128 + r) * K + kb * 128 + l16 * 8);
    }
    float am[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 32 * w + 4 * i + lr;
      am[i] = absmax8(v[i]);
      *reinterpret_cast<uint4*>(tile + r * 128 + 4 * ((2 * l16) ^ d_swz(r))) = v[i];
    }
    // Lane l16 computes the scale of tile (row) (l16 >> 1) & 7 of the eight
    // its row of lanes covers; tile i's is broadcast from lane 2i.
    const TileScale mine = tile_scale<POW2>(row_max8(am, l16));
    auto run = [&](auto scaled) {
      constexpr bool SC = decltype(scaled)::value;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 32 * w + 4 * i + lr;
        TileScale ts;
        ts.ss = row_bcast(mine.ss, 2 * i);
        ts.r = row_bcast(mine.r, 2 * i);
        ts.sx = SC ? row_bcast(mine.sx, 2 * i) : 1.0f;
        *reinterpret_cast<uint2*>(q + (mb * 128 + r) * K + kb * 128 + l16 * 8) = quantize8<POW2, SC>(v[i], ts);
      }
    };
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mine.sx != 1.0f) != 0, 0))
      run(std::true_type{});
    else
      run(std::false_type{});
    if ((l16 & 1) == 0) s[kb * M + mb * 128 + 32 * w + 4 * (l16 >> 1) + lr] = mine.s;
  }
  __syncthreads();
  const int rg = l & 7, cg = 8 * w + (l >> 3);
  uint2 wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    wv[i] = *reinterpret_cast<const uint2*>(tile + r * 128 + 4 * (cg ^ d_swz(r)));
  }
  float d[4][16];
  float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[j][i] = bf16_at(wv[i], j);
      am[j] = __builtin_fmaxf(am[j], __builtin_fabsf(d[j][i]));
    }
  requant_columns<POW2>(d, am, l, qt + (kb * 128 + 4 * cg) * M + mb * 128 + 16 * rg, M,
                        st + mb * K + kb * 128 + 4 * cg);
}

// ---------------------------------------------------------------------------
// Transposed block-scaled weight (data gradient; page 2, paragraph on
// hardware suggestions, asks for GEMMs on transposed operands).  W^T keeps
// W's codes and takes the transposed scale grid; rows of W past N become
// zero columns up to the next multiple of 128.  One workgroup per 128x128
// block (x = row block of W, y = column block, z = matrix): the block is
// staged in LDS in the transpose-requantize layout above, then lane (rg, c4)
// gathers rows 16*rg .. 16*rg+15 of columns 4*c4 .. 4*c4+3 and writes them
// as 16 contiguous bytes of four rows of W^T (eight lanes per 128-byte line).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_transpose_128x128(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                           int64_t N, int64_t K, uint8_t* __restrict__ qt,
                                                           float* __restrict__ st) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[129 * 128];
  const int64_t nb = blockIdx.x, kb = blockIdx.y, g = blockIdx.z;
  const int64_t NB = (N + 127) / 128, KT = K / 128, Np = NB * 128;
  const int t = threadIdx.x;
  {
    const int seg = t & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * i + (t >> 3);
      const int64_t row = nb * 128 + r;
      const uint4 v = row < N ? nt_load16(q + (g * N + row) * K + kb * 128 + seg * 16) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(codes + t_row(r) * 128 + 16 * (seg ^ (t_swz(r) >> 2))) = v;
    }
  }
  __syncthreads();
  const int l = t & 63, w = t >> 6;
  const int rg = l & 7, c4 = 8 * w + (l >> 3);
  uint32_t wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    wv[i] = *reinterpret_cast<const uint32_t*>(codes + t_row(r) * 128 + 4 * (c4 ^ t_swz(r)));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      packed[k] = ((wv[4 * k] >> (8 * j)) & 0xFFu) | (((wv[4 * k + 1] >> (8 * j)) & 0xFFu) << 8) |
                  (((wv[4 * k + 2] >> (8 * j)) & 0xFFu) << 16) | (((wv[4 * k + 3] >> (8 * j)) & 0xFFu) << 24);
    nt_store16(qt + (g * K + kb * 128 + 4 * c4 + j) * Np + nb * 128 + 16 * rg,
               make_uint4(packed[0], packed[1], packed[2], packed[3]));
  }
  if (t == 0) st[(g * KT + kb) * NB + nb] = s[(g * NB + nb) * KT + kb];
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks.  One workgroup per block (z = matrix, x = row block,
// y = column block).  Load instruction i of wave w reads rows 32w + 4i + l/16,
// sixteen lanes per 256-byte row (8 BF16 each), so an instruction covers four
// whole rows (each lane owning half a row instead, an instruction touched 64
// rows' lines at once: 3.7 TB/s).  Block amax: DPP row max, then across the
// 4 DPP rows of a wave and the 4 waves through LDS.  Rows past N contribute
// nothing and are not written.
// ---------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void k_quantize_128x128(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                           uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float part[16];
  const int64_t nb = blockIdx.x, kb = blockIdx.y, g = blockIdx.z;
  const int64_t NB = (N + 127) / 128, KT = K / 128;
  const int t = threadIdx.x;
  const int wv = t >> 6, lr = (t & 63) >> 4, l16 = t & 15;
  const int64_t row0 = nb * 128 + 32 * wv + lr;      // row of instruction 0; instruction i adds 4i
  const int64_t col = kb * 128 + l16 * 8;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = row0 + 4 * i < N ? nt_load16(w + (g * N + row0 + 4 * i) * K + col) : make_uint4(0, 0, 0, 0);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[i].x)), __builtin_fabsf(bf16_hi(v[i].x))));
    a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[i].y)), __builtin_fabsf(bf16_hi(v[i].y))));
    a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[i].z)), __builtin_fabsf(bf16_hi(v[i].z))));
    a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(bf16_lo(v[i].w)), __builtin_fabsf(bf16_hi(v[i].w))));
  }
  a = row16_max(a);
  if ((t & 15) == 0) part[t >> 4] = a;
  __syncthreads();
  float amax = part[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) amax = __builtin_fmaxf(amax, part[i]);
  const TileScale ts = tile_scale<POW2>(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 o = (ts.sx != 1.0f) ? quantize8<POW2, true>(v[i], ts) : quantize8<POW2, false>(v[i], ts);
    if (row0 + 4 * i < N) *reinterpret_cast<uint2*>(q + (g * N + row0 + 4 * i) * K + col) = o;
  }
  if (t == 0) s[(g * NB + nb) * KT + kb] = ts.s;
}

// ---------------------------------------------------------------------------
// Elementwise FP32 -> E4M3 with the quantizers' encoding; NaN keeps its sign.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t cast4(float4 v) {
  uint32_t w = pack4_e4m3_sat(v.x, v.y, v.z, v.w);
  const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e[i] != e[i]) {
      const uint32_t nan = 0x7Fu | ((__builtin_bit_cast(uint32_t, e[i]) >> 24) & 0x80u);
      w = (w & ~(0xFFu << (8 * i))) | (nan << (8 * i));
    }
  }
  return w;
}

__global__ __launch_bounds__(256) void k_cast_e4m3(const float* __restrict__ x, int64_t n, uint8_t* __restrict__ q) {
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<uint32_t*>(q)[i] = cast4(reinterpret_cast<const float4*>(x)[i]);
  // tail (n % 4 elements), one lane
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = n4 * 4; i < n; ++i) {
      float4 v = make_float4(x[i], 0.f, 0.f, 0.f);
      q[i] = (uint8_t)(cast4(v) & 0xFFu);
    }
  }
}

}  // namespace

// ----------------------------- launchers ----------------------------------
hipError_t launch_quantize_1x128(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, bool pow2,
                                 hipStream_t stream) {
  const int64_t KT = K / 128;
  dim3 grid((unsigned)((M + 15) / 16), (unsigned)((KT + kQ1Tiles - 1) / kQ1Tiles));
  if (pow2)
    hipLaunchKernelGGL(k_quantize_1x128<true>, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, q, s);
  else
    hipLaunchKernelGGL(k_quantize_1x128<false>, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, q, s);
  return hipGetLastError();
}

hipError_t launch_quantize_t128x1(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt, float* st,
                                  bool pow2, hipStream_t stream) {
  dim3 grid((unsigned)(M / 128), (unsigned)(K / 128));
  if (pow2)
    hipLaunchKernelGGL(k_quantize_t128x1<true>, grid, dim3(256), 0, stream, q, s, M, K, qt, st);
  else
    hipLaunchKernelGGL(k_quantize_t128x1<false>, grid, dim3(256), 0, stream, q, s, M, K, qt, st);
  return hipGetLastError();
}

hipError_t launch_quantize_128x128(const void* w, int64_t G, int64_t N, int64_t K, uint8_t* q, float* s, bool pow2,
                                   hipStream_t stream) {
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)(K / 128), (unsigned)G);
  if (pow2)
    hipLaunchKernelGGL(k_quantize_128x128<true>, grid, dim3(256), 0, stream, (const uint16_t*)w, N, K, q, s);
  else
    hipLaunchKernelGGL(k_quantize_128x128<false>, grid, dim3(256), 0, stream, (const uint16_t*)w, N, K, q, s);
  return hipGetLastError();
}

// One 128x128 tile per workgroup.  Two or four tiles per workgroup with the
// next tile's values loaded during the current one were slower on 8192x7168
// (62 and 67 vs 45 us): twice the registers and a second barrier per tile.
hipError_t launch_quantize_dual(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt, float* st,
                                bool pow2, hipStream_t stream) {
  dim3 grid((unsigned)(M / 128), (unsigned)(K / 128));
  if (pow2)
    hipLaunchKernelGGL(k_quantize_dual<true>, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, q, s, qt, st);
  else
    hipLaunchKernelGGL(k_quantize_dual<false>, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, q, s, qt, st);
  return hipGetLastError();
}

hipError_t launch_transpose_128x128(const uint8_t* q, const float* s, int64_t G, int64_t N, int64_t K, uint8_t* qt,
                                   float* st, hipStream_t stream) {
  dim3 grid((unsigned)((N + 127) / 128), (unsigned)(K / 128), (unsigned)G);
  hipLaunchKernelGGL(k_transpose_128x128, grid, dim3(256), 0, stream, q, s, N, K, qt, st);
  return hipGetLastError();
}

hipError_t launch_cast_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream) {
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_cast_e4m3, dim3((unsigned)blocks), dim3(256), 0, stream, x, n, q);
  return hipGetLastError();
}

}  // namespace fp8bs
