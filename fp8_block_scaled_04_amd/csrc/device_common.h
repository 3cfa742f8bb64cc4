// Device helpers shared by the gfx950 kernels of libfp8bs.
//
// Everything here is written for CDNA4 (gfx950): 64-lane wavefronts, DPP row
// operations, the OCP-FP8 conversion instructions and the E4M3 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// Cross-lane max over each DPP row (16 lanes) and over lane pairs.
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at xor 1 and xor 2; the
// half-mirror and mirror steps then join the quads of an 8-lane half and the
// two halves of the row, so every lane ends with the row's maximum.
// ---------------------------------------------------------------------------
// Every lane reads a lane of its own row, so no lane is out of range and the
// DPP move carries no "old" value; that lets the compiler fold it into the
// max as a DPP operand (one instruction per step).
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

__device__ __forceinline__ float pair_max(float v) { return dpp_max_step(v, 0); }

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
// keeps every operand normal; quotients that still come out subnormal encode
// to a zero E4M3 code either way.  The resulting E4M3 codes, sign included,
// were compared against enc(x / s) for every pair of BF16 (x, amax) with
// |x| <= amax and both signs of x, for all power-of-two scales, and for 4e8
// random FP32 pairs: no difference.
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

// ---------------------------------------------------------------------------
// E4M3 encode (hardware OCP-FP8 conversion, round to nearest even), four
// values into one dword, byte i = value i.
//
// pack4_e4m3 is for the quantizers, whose values satisfy |y| <= 448 * (1 +
// 2^-22) < 464: the conversion rounds everything in [448, 464] to 448
// (checked on the GPU for every FP32 value in that range), so no clamp is
// needed.  pack4_e4m3_sat clamps to +-448 first (satfinite) for arbitrary
// finite inputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clamp448(float y) {
  return __builtin_fminf(__builtin_fmaxf(y, -kE4M3Max), kE4M3Max);
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t pack4_e4m3_sat(float a, float b, float c, float d) {
  return pack4_e4m3(clamp448(a), clamp448(b), clamp448(c), clamp448(d));
}

// E4M3 byte `sel` of a dword -> float (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// BF16 helpers: the low / high half of a dword as float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two floats -> packed BF16 pair (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// ---------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X
// (workgroup i runs on XCD i % 8).  Renumber them so that consecutive logical
// ids land on the same XCD, which keeps tiles that share operand panels in one
// L2, and so that every XCD gets an equal share of the `total` ids that have
// work: XCD x takes total/8 ids (one more for x < total % 8).  `total` may be
// below the grid size (grids sized for the worst case); workgroups beyond
// their XCD's share get -1 and have nothing to do.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcds = 8;
  const int q = total / kXcds, r = total % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int share = q + (xcd < r ? 1 : 0);
  if (local >= share) return -1;
  return xcd * q + min(xcd, r) + local;
}

}  // namespace fp8bs
