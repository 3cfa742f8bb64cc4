// Streaming reference kernel (not a step of the method): reads `ratio`
// 16-byte pieces per 16-byte piece written, with nontemporal loads and
// stores, so the HBM-bound kernels can be set against the throughput a plain
// stream of the same read:write mix reaches on the same device.  The
// 1x128 quantizer is a 2:1 stream (BF16 in, codes out), the transposing
// requantizer a 1:1 stream.
//
// Configuration: 8192 workgroups of 256 lanes walking the output in a
// grid-stride loop, one piece per lane per step for 1:1 and four for 2:1 (the
// best of 1/2/4 pieces x 1024..8192 workgroups measured on an MI355X over
// 58.7 MB outputs: 5.97 TB/s for 1:1, 5.79 TB/s for 2:1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace fp8bs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// dst piece i = XOR of src pieces RATIO*i .. RATIO*i + RATIO-1.
template <int U, int RATIO>
__global__ __launch_bounds__(256) void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U][RATIO];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RATIO; ++r) v[u][r] = ld_nt(src + (i + u * stride) * RATIO + r);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4 w = v[u][0];
#pragma unroll
      for (int r = 1; r < RATIO; ++r) w ^= v[u][r];
      st_nt(dst + i + u * stride, w);
    }
  }
  for (; i < n16; i += stride) {
    u32x4 w = ld_nt(src + i * RATIO);
#pragma unroll
    for (int r = 1; r < RATIO; ++r) w ^= ld_nt(src + i * RATIO + r);
    st_nt(dst + i, w);
  }
}

}  // namespace

hipError_t launch_stream_reference(const void* src, void* dst, int64_t dst_bytes, int ratio, hipStream_t stream) {
  const int64_t n16 = dst_bytes / 16;
  const dim3 grid(8192), block(256);
  if (ratio == 1)
    hipLaunchKernelGGL((k_stream<1, 1>), grid, block, 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  else
    hipLaunchKernelGGL((k_stream<4, 2>), grid, block, 0, stream, (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace fp8bs
