// Device helpers shared by the gfx950 kernels of libfp8bs: vector types,
// BF16 packing and the XCD-aware workgroup numbering.  (The quantizers' own
// helpers are in quant_common.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;


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
