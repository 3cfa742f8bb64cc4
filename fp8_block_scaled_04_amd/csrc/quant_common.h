// Device helpers of the quantizers (gfx950): DPP row reductions, the tile
// scale and exact division, E4M3 encoding, BF16 unpacking.
#pragma once

#include "device_common.h"

namespace fp8bs {

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// Cross-lane max over each DPP row (16 lanes) and over lane pairs.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at xor 1 and xor 2; the
// half-mirror and mirror steps then join the quads of an 8-lane half and the
// two halves of the row, so every lane ends with the row's maximum.
// ---------------------------------------------------------------------------
// Every lane reads a lane of its own row, so no lane is out of range and the
// DPP move needs no "old" value.
__device__ __forceinline__ float dpp_max_step(float v, int ctrl_id) {
  int iv = __builtin_bit_cast(int, v);
  int o;
  switch (ctrl_id) {
    case 0: o = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true); break;  // quad_perm 1,0,3,2
    case 1: o = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true); break;  // quad_perm 2,3,0,1
    case 2: o = __builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true); break; // row_half_mirror
    default: o = __builtin_amdgcn_mov_dpp(iv, 0x140, 0xF, 0xF, true); break; // row_mirror
  }
  return __builtin_fmaxf(v, __builtin_bit_cast(float, o));
}

__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max_step(v, 0);
  v = dpp_max_step(v, 1);
  v = dpp_max_step(v, 2);
  v = dpp_max_step(v, 3);
  return v;
}

// ---------------------------------------------------------------------------
// Tile scale and exact division.
//
// scale(amax) = 1 for amax == 0, else max(fl32(amax / 448), 2^-149); with
// POW2 it is rounded up to the next power of two (on the bits: a normal value
// with a nonzero mantissa moves to the next exponent; a subnormal goes to the
// next power-of-two bit pattern).
//
// fl32(x / s) is computed as  q = x*r;  t = fma(q, s, -x);  y = fma(-t, r, q)
// with r = RN(1/s) (a correctly rounded IEEE divide, once per tile).  This is
// Markstein's correction step with the residual -t = x - q*s; it returns the
// correctly rounded quotient as long as no operand or residual is subnormal.
// Writing the residual with its sign flipped keeps the sign of a zero
// quotient (x = -0 gives -0) without a separate copysign.  Tiles with
// amax < 2^-60 are evaluated on x * 2^64 and s * 2^64 (both exact), which
// keeps every operand normal.  Where the correction's preconditions still
// fail (a residual that underflows: |x| < 2^-102 on the unscaled path, or a
// subnormal quotient) both the result and the true quotient are at most
// 2^-10 with the same sign, so both encode to the E4M3 zero of that sign.
// tests/test_quant_divide.py replays these operations on the CPU for every
// pair of BF16 (x, amax) with |x| <= amax, both signs, with and without
// power-of-two scales; tests/test_gpu_exhaustive.py runs one tile per BF16
// amax through the kernels.
struct TileScale {
  float s;    // the scale written to memory
  float ss;   // s * sx
  float r;    // RN(1 / ss)
  float sx;   // 1 or 2^64
};

template <bool POW2>
__device__ __forceinline__ TileScale tile_scale(float amax) {
#pragma clang fp contract(off)
  float s = amax / kE4M3Max;
  s = __builtin_fmaxf(s, 0x1p-149f);
  if (!(amax > 0.0f)) s = 1.0f;
  if (POW2) {
    uint32_t b = __builtin_bit_cast(uint32_t, s);
    if (b >= 0x00800000u) {
      if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
    } else if (b & (b - 1u)) {
      b = 1u << (32 - __builtin_clz(b));
    }
    s = __builtin_bit_cast(float, b);
  }
  TileScale t;
  t.s = s;
  t.sx = (amax < 0x1p-60f) ? 0x1p64f : 1.0f;
  t.ss = s * t.sx;
  t.r = 1.0f / t.ss;
  return t;
}

// s > 0.  For x = -0: q = -0, t = fma(-0, s, +0) = +0, y = fma(-0, r, -0) = -0.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
#pragma clang fp contract(off)
  const float q = x * r;
  const float t = __builtin_fmaf(q, s, -x);
  return __builtin_fmaf(-t, r, q);
}

// fl32(x / ss), the quotient every quantizer encodes.  With power-of-two
// scales r = 1/ss is exact (ss lies in [2^-85, 2^120], so r is a normal power
// of two) and x * r rounds the same real number x / ss once: one multiply
// gives the correctly rounded quotient, subnormal results and signed zeros
// included.
template <bool POW2>
__device__ __forceinline__ float quot(float x, const TileScale& t) {
  return POW2 ? x * t.r : div_rn(x, t.ss, t.r);
}

// ---------------------------------------------------------------------------
// E4M3 encode (hardware OCP-FP8 conversion, round to nearest even), four
// values into one dword, byte i = value i.
//
// pack4_e4m3 is for the quantizers, whose values satisfy |y| <= 448 * (1 +
// 2^-22) < 464 (x / s with s = RN(amax / 448) exceeds 448 only when the
// scale rounded down): round to nearest even maps everything in [448, 464)
// to 448, so no clamp is needed (every BF16 amax, about half of them with a
// scale that rounded down, is checked bit-exact in
// tests/test_gpu_exhaustive.py).  pack4_e4m3_sat clamps to +-448 first
// (satfinite) for arbitrary inputs; the cast is compared with the oracle on
// all 2^32 FP32 bit patterns there.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clamp448(float y) {
  return __builtin_fminf(__builtin_fmaxf(y, -kE4M3Max), kE4M3Max);
}

// The first conversion writes bytes 0-1 and keeps bytes 2-3 of the dword it
// is given, which the second conversion overwrites: any register will do (a's
// bits; a constant zero would cost a move per call).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t pack4_e4m3_sat(float a, float b, float c, float d) {
  return pack4_e4m3(clamp448(a), clamp448(b), clamp448(c), clamp448(d));
}

// BF16 helpers: the low / high half of a dword as float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

}  // namespace fp8bs
