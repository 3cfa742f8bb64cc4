// Streaming reference kernels (not a step of the method): plain streams of
// the HBM-bound kernels' read:write mixes, so that those can be set against
// the throughput such a stream reaches on the same device.  The 1x128
// quantizer is a 2:1 stream (BF16 in, codes out), the transposing
// requantizer a 1:1 stream.
//
// Configuration: 8192 workgroups of 256 lanes walking the data in a
// grid-stride loop, one piece per lane per step; nontemporal loads.  1:1
// copies 16-byte pieces with nontemporal stores; 2:1 folds each 16-byte piece
// read into an 8-byte piece written with ordinary stores.  These were the
// fastest of the forms measured on an MI355X, with 58.7 MB written, 4096 to
// 16384 workgroups, and 1, 2 or 4 pieces per lane:
//   1:1: 6.10 TB/s.  Cached stores gave 5.87, two pieces per lane 5.77.
//   2:1: 6.51 TB/s.  16-byte nontemporal stores, each the XOR of two pieces
//        read, gave 5.89.  8-byte nontemporal stores gave 6.27.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace fp8bs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// 1:1: dst piece i = src piece i (16-byte pieces).
__global__ __launch_bounds__(256) void k_stream11(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                  int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) st_nt(dst + i, ld_nt(src + i));
}

// 2:1: 8-byte piece i of dst = (w0 ^ w1, w2 ^ w3) of the 32-bit words of
// 16-byte piece i of src.
__global__ __launch_bounds__(256) void k_stream21(const u32x4* __restrict__ src, u32x2* __restrict__ dst,
                                                  int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const u32x4 v = ld_nt(src + i);
    dst[i] = u32x2{v.x ^ v.y, v.z ^ v.w};
  }
}

}  // namespace

hipError_t launch_stream_reference(const void* src, void* dst, int64_t dst_bytes, int ratio, hipStream_t stream) {
  const dim3 grid(8192), block(256);
  if (ratio == 1)
    hipLaunchKernelGGL(k_stream11, grid, block, 0, stream, (const u32x4*)src, (u32x4*)dst, dst_bytes / 16);
  else
    hipLaunchKernelGGL(k_stream21, grid, block, 0, stream, (const u32x4*)src, (u32x2*)dst, dst_bytes / 8);
  return hipGetLastError();
}

}  // namespace fp8bs
