// C ABI of libfp8bs: argument checks, device check, dispatch to launchers.
// The operations and their sources on the surveyed pages are documented in
// include/fp8bs.h next to each declaration.
#include <atomic>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "fp8bs.h"
#include "launch.h"
#include "splitk.h"

namespace {

using fp8bs::GemmProblem;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The current device must be a gfx950 (MI355X / MI350X).  The answer is
// cached per device ordinal; hipGetDevice itself fails when no GPU exists.
fp8bs_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8BS_ERR_DEVICE;
  if (dev >= kMaxDevices) return FP8BS_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BS_ERR_DEVICE;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FP8BS_OK : FP8BS_ERR_DEVICE;
}

fp8bs_status launched(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH; }

constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxGridX = 0x7FFFFFFF;

// Scratch of the allocation-free split-K call: the largest split-K
// workspace (at most 256 partial tiles of at most 128 x 96 FP32), one copy per GPU,
// held until the process ends.  Host code uses the device address that
// hipGetSymbolAddress returns for the current device, never the symbol.
constexpr int64_t kScratchBytes = 256 * 128 * 96 * 4;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that
// device); nullptr if the lookup fails.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* fp8bs_status_str(fp8bs_status s) {
  switch (s) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "invalid size (negative, or breaks a divisibility rule)";
    case FP8BS_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP8BS_ERR_FLAGS: return "unknown flags or output dtype";
    case FP8BS_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case FP8BS_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t fp8bs_abi_version(void) { return FP8BS_ABI_VERSION; }

fp8bs_status fp8bs_quantize_1x128(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, uint32_t flags,
                                  fp8bs_stream_t stream) {
  if (M < 0 || K <= 0 || K % 128) return FP8BS_ERR_SHAPE;
  if ((K / 128 + fp8bs::kQ1Tiles - 1) / fp8bs::kQ1Tiles > kMaxGridY || (M + 15) / 16 > kMaxGridX) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0) return FP8BS_OK;
  if (!x || !q || !s) return FP8BS_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status st = check_device()) return st;
  (void)hipGetLastError();
  return launched(fp8bs::launch_quantize_1x128(x, M, K, q, s, flags & FP8BS_SCALE_POW2, (hipStream_t)stream));
}

fp8bs_status fp8bs_quantize_transpose_128x1(const uint8_t* q, const float* s, int64_t M, int64_t K, uint8_t* qt,
                                            float* st, uint32_t flags, fp8bs_stream_t stream) {
  if (M < 0 || K < 0 || M % 128 || K % 128) return FP8BS_ERR_SHAPE;
  if (K / 128 > kMaxGridY || M / 128 > kMaxGridX) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || K == 0) return FP8BS_OK;
  if (!q || !s || !qt || !st) return FP8BS_ERR_NULL;
  if (!aligned16(q) || !aligned16(s) || !aligned16(qt) || !aligned16(st)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_quantize_t128x1(q, s, M, K, qt, st, flags & FP8BS_SCALE_POW2, (hipStream_t)stream));
}

fp8bs_status fp8bs_quantize_128x128(const void* w, int64_t G, int64_t N, int64_t K, uint8_t* q, float* s,
                                    uint32_t flags, fp8bs_stream_t stream) {
  if (G < 0 || N < 0 || K <= 0 || K % 128) return FP8BS_ERR_SHAPE;
  if (G > kMaxGridY || K / 128 > kMaxGridY || (N + 127) / 128 > kMaxGridX) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (G == 0 || N == 0) return FP8BS_OK;
  if (!w || !q || !s) return FP8BS_ERR_NULL;
  if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_quantize_128x128(w, G, N, K, q, s, flags & FP8BS_SCALE_POW2, (hipStream_t)stream));
}

fp8bs_status fp8bs_quantize_dual(const void* x, int64_t M, int64_t K, uint8_t* q, float* s, uint8_t* qt, float* st,
                                uint32_t flags, fp8bs_stream_t stream) {
  if (M < 0 || K < 0 || M % 128 || K % 128) return FP8BS_ERR_SHAPE;
  if (K / 128 > kMaxGridY || M / 128 > kMaxGridX) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || K == 0) return FP8BS_OK;
  if (!x || !q || !s || !qt || !st) return FP8BS_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s) || !aligned16(qt) || !aligned16(st)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_quantize_dual(x, M, K, q, s, qt, st, flags & FP8BS_SCALE_POW2, (hipStream_t)stream));
}

fp8bs_status fp8bs_transpose_128x128(const uint8_t* q, const float* s, int64_t G, int64_t N, int64_t K, uint8_t* qt,
                                    float* st, fp8bs_stream_t stream) {
  if (G < 0 || N < 0 || N % 16 || K < 0 || K % 128) return FP8BS_ERR_SHAPE;
  if (G > kMaxGridY || K / 128 > kMaxGridY || (N + 127) / 128 > kMaxGridX) return FP8BS_ERR_SHAPE;
  if (G == 0 || N == 0 || K == 0) return FP8BS_OK;
  if (!q || !s || !qt || !st) return FP8BS_ERR_NULL;
  if (!aligned16(q) || !aligned16(qt) || (reinterpret_cast<uintptr_t>(s) & 3u) ||
      (reinterpret_cast<uintptr_t>(st) & 3u))
    return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_transpose_128x128(q, s, G, N, K, qt, st, (hipStream_t)stream));
}

namespace {

fp8bs_status gemm_common(int64_t N, int64_t K, int32_t out_dtype) {
  if (N < 0 || N % 16 || K <= 0 || K % 128) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_FP32) return FP8BS_ERR_FLAGS;
  return FP8BS_OK;
}

fp8bs_status gemm_pointers(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, void* d,
                           const int32_t* groups, bool need_groups) {
  if (!a || !sa || !b || !sb || !d || (need_groups && !groups)) return FP8BS_ERR_NULL;
  if (!aligned16(a) || !aligned16(sa) || !aligned16(b) || !aligned16(sb) || !aligned16(d) ||
      (need_groups && (reinterpret_cast<uintptr_t>(groups) & 3u)))
    return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

// Tile counts must fit the 32-bit workgroup index and in-kernel int math.
bool grid_fits(int64_t rows, int64_t N, int64_t groups) {
  const int64_t tiles = ((rows + 127) / 128) * ((N + 127) / 128) * groups;
  return tiles < (int64_t(1) << 30);
}

// The GEMM kernels address a tile's operand panels (up to 256 rows of K
// bytes) and a group's scale arrays through buffer descriptors with 31-bit
// sizes and 32-bit offsets: each of those regions must stay below 2^31 bytes.
// rows: rows of one group's activation-scale array (M, Mt or cap);
// wscale_rows: rows of the weight scales ([K/128][N] for the weight gradient,
// else the [N/128][K/128] block grid).
bool buffers_fit(int64_t rows, int64_t N, int64_t K, bool per_row_weight_scales) {
  constexpr int64_t kMax = 0x7FFFFFFF;
  const int64_t KT = K / 128, NB = (N + 127) / 128;
  if (K > kMax / 256) return false;                                  // a 256-row operand panel
  if (rows > 0 && KT > kMax / 4 / rows) return false;                // activation scales
  const int64_t ws = per_row_weight_scales ? N : NB;
  if (ws > 0 && KT > kMax / 4 / ws) return false;                    // weight scales
  return true;
}

}  // namespace

fp8bs_status fp8bs_gemm_fp8_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, void* d,
                                        int64_t M, int64_t N, int64_t K, int32_t out_dtype, uint32_t flags,
                                        fp8bs_stream_t stream) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  if (!grid_fits(M, N, 1) || !buffers_fit(M, N, K, false)) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, nullptr, false)) return e;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{a, sa, b, sb, d, nullptr, M, N, K, 1, out_dtype == FP8BS_OUT_FP32, false,
                (flags & FP8BS_SCALE_POW2) != 0, fp8bs::kDense};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm(p, (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_fp8_blockscaled_splitk(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                               void* d, int64_t M, int64_t N, int64_t K, int32_t out_dtype,
                                               uint32_t flags, void* workspace, int64_t workspace_bytes,
                                               fp8bs_stream_t stream) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  if (!grid_fits(M, N, 1) || !buffers_fit(M, N, K, false)) return FP8BS_ERR_SHAPE;
  const int64_t need = fp8bs::splitk_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, nullptr, false)) return e;
  if (need > 0 && !workspace) return FP8BS_ERR_NULL;
  if (need > 0 && !aligned16(workspace)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{a, sa, b, sb, d, nullptr, M, N, K, 1, out_dtype == FP8BS_OUT_FP32, false,
                (flags & FP8BS_SCALE_POW2) != 0, fp8bs::kDense};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm_splitk(p, static_cast<float*>(workspace), (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_fp8_blockscaled_splitk_noalloc(const uint8_t* a, const float* sa, const uint8_t* b,
                                                       const float* sb, void* d, int64_t M, int64_t N, int64_t K,
                                                       int32_t out_dtype, uint32_t flags, fp8bs_stream_t stream) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  if (!grid_fits(M, N, 1) || !buffers_fit(M, N, K, false)) return FP8BS_ERR_SHAPE;
  if (fp8bs::splitk_workspace_bytes(M, N, K) > kScratchBytes) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, nullptr, false)) return e;
  if (fp8bs_status e = check_device()) return e;
  void* ws = scratch_ptr();
  if (!ws) return FP8BS_ERR_DEVICE;
  GemmProblem p{a, sa, b, sb, d, nullptr, M, N, K, 1, out_dtype == FP8BS_OUT_FP32, false,
                (flags & FP8BS_SCALE_POW2) != 0, fp8bs::kDense};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm_splitk(p, static_cast<float*>(ws), (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, FP8BS_OUT_BF16)) return e;
  if (!grid_fits(M, N, 1) || !buffers_fit(M, N, K, false)) return FP8BS_ERR_SHAPE;
  if (!bytes) return FP8BS_ERR_NULL;
  *bytes = fp8bs::splitk_workspace_bytes(M, N, K);
  return FP8BS_OK;
}

fp8bs_status fp8bs_gemm_fused_quantize(const void* x, const uint8_t* b, const float* sb, void* d, int64_t M, int64_t N,
                                       int64_t K, int32_t out_dtype, uint32_t flags, fp8bs_stream_t stream) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  // 64-row tiles; the BF16 panel of a tile is 128 * K bytes, below the 256-row
  // code panel buffers_fit bounds.
  if (((M + 63) / 64) * ((N + 127) / 128) >= (int64_t(1) << 30) || !buffers_fit(0, N, K, false))
    return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!x || !b || !sb || !d) return FP8BS_ERR_NULL;
  if (!aligned16(x) || !aligned16(b) || !aligned16(sb) || !aligned16(d)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{static_cast<const uint8_t*>(x), nullptr, b, sb, d, nullptr, M, N, K, 1,
                out_dtype == FP8BS_OUT_FP32, false, false, fp8bs::kDense};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm_qa(p, (flags & FP8BS_SCALE_POW2) != 0, (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_fp8_wgrad(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb, float* d,
                                  int64_t M, int64_t N, int64_t K, int32_t accumulate, uint32_t flags,
                                  fp8bs_stream_t stream) {
  if (M < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, FP8BS_OUT_FP32)) return e;
  if (!grid_fits(M, N, 1) || !buffers_fit(M, N, K, true)) return FP8BS_ERR_SHAPE;
  if (accumulate != 0 && accumulate != 1) return FP8BS_ERR_FLAGS;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, nullptr, false)) return e;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{a, sa, b, sb, d, nullptr, M, N, K, 1, true, accumulate == 1, (flags & FP8BS_SCALE_POW2) != 0,
                fp8bs::kWgrad};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm(p, (hipStream_t)stream));
}

fp8bs_status fp8bs_grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                               void* d, const int32_t* m_offsets, int32_t G, int64_t Mt, int64_t N,
                                               int64_t K, int32_t out_dtype, uint32_t flags, fp8bs_stream_t stream) {
  if (G < 0 || Mt < 0 || Mt % 128) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  if (!grid_fits(Mt, N, 1) || !buffers_fit(Mt, N, K, false)) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (G == 0 || Mt == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, m_offsets, true)) return e;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{a, sa, b, sb, d, m_offsets, Mt, N, K, G, out_dtype == FP8BS_OUT_FP32, false,
                (flags & FP8BS_SCALE_POW2) != 0, fp8bs::kContiguous};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm(p, (hipStream_t)stream));
}

fp8bs_status fp8bs_grouped_gemm_fp8_masked(const uint8_t* a, const float* sa, const uint8_t* b, const float* sb,
                                           void* d, const int32_t* masked_m, int32_t G, int64_t cap, int64_t N,
                                           int64_t K, int32_t out_dtype, uint32_t flags, fp8bs_stream_t stream) {
  if (G < 0 || cap < 0) return FP8BS_ERR_SHAPE;
  if (fp8bs_status e = gemm_common(N, K, out_dtype)) return e;
  if (!grid_fits(cap, N, G) || !buffers_fit(cap, N, K, false)) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (G == 0 || cap == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_status e = gemm_pointers(a, sa, b, sb, d, masked_m, true)) return e;
  if (fp8bs_status e = check_device()) return e;
  GemmProblem p{a, sa, b, sb, d, masked_m, cap, N, K, G, out_dtype == FP8BS_OUT_FP32, false,
                (flags & FP8BS_SCALE_POW2) != 0, fp8bs::kMasked};
  (void)hipGetLastError();
  return launched(fp8bs::launch_gemm(p, (hipStream_t)stream));
}

fp8bs_status fp8bs_gemm_tile(int32_t layout, int64_t rows, int64_t N, int64_t K, int32_t G, uint32_t flags,
                             int32_t* tile_m, int32_t* tile_n, int32_t* ping_pong) {
  if (layout < 0 || layout > 4) return FP8BS_ERR_FLAGS;
  if (fp8bs_status e = gemm_common(N, K, FP8BS_OUT_BF16)) return e;
  if (rows < 0 || G < 0) return FP8BS_ERR_SHAPE;
  if (layout == 4) {   // fp8bs_gemm_fused_quantize
    if (G != 1) return FP8BS_ERR_SHAPE;
    if (((rows + 63) / 64) * ((N + 127) / 128) >= (int64_t(1) << 30) || !buffers_fit(0, N, K, false))
      return FP8BS_ERR_SHAPE;
    if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
    if (!tile_m || !tile_n || !ping_pong) return FP8BS_ERR_NULL;
    *tile_m = 64;
    *tile_n = fp8bs::gemm_qa_tile_n(N);
    *ping_pong = 0;
    return FP8BS_OK;
  }
  if ((layout == 0 || layout == 3) && G != 1) return FP8BS_ERR_SHAPE;
  if (layout == 1 && rows % 128) return FP8BS_ERR_SHAPE;
  if (!grid_fits(rows, N, layout == 2 ? G : 1) || !buffers_fit(rows, N, K, layout == 3)) return FP8BS_ERR_SHAPE;
  if (flags & ~(uint32_t)FP8BS_SCALE_POW2) return FP8BS_ERR_FLAGS;
  if (!tile_m || !tile_n || !ping_pong) return FP8BS_ERR_NULL;
  static const fp8bs::GemmMode modes[4] = {fp8bs::kDense, fp8bs::kContiguous, fp8bs::kMasked, fp8bs::kWgrad};
  GemmProblem p{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, rows, N, K, G, false, false,
                (flags & FP8BS_SCALE_POW2) != 0, modes[layout]};
  fp8bs::gemm_tile(p, *tile_m, *tile_n, *ping_pong);
  return FP8BS_OK;
}

fp8bs_status fp8bs_stream_reference(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                                    fp8bs_stream_t stream) {
  if (dst_bytes < 0 || dst_bytes % 16 || (src_bytes != dst_bytes && src_bytes != 2 * dst_bytes))
    return FP8BS_ERR_SHAPE;
  if (dst_bytes == 0) return FP8BS_OK;
  if (!src || !dst) return FP8BS_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_stream_reference(src, dst, dst_bytes, (int)(src_bytes / dst_bytes),
                                                 (hipStream_t)stream));
}

fp8bs_status fp8bs_cast_f32_to_e4m3(const float* x, int64_t n, uint8_t* q, fp8bs_stream_t stream) {
  if (n < 0) return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!x || !q) return FP8BS_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return FP8BS_ERR_ALIGN;
  if (fp8bs_status e = check_device()) return e;
  (void)hipGetLastError();
  return launched(fp8bs::launch_cast_e4m3(x, n, q, (hipStream_t)stream));
}

}  // extern "C"
