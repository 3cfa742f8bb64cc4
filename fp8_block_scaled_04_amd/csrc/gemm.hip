// Block-scaled FP8 GEMM for gfx950: dense, contiguous-grouped and
// masked-grouped layouts share one kernel body.
//
// What it computes (page 1, the uniondaocoop.com post on DeepSeek's FP8
// training framework: FP8 operands, BF16/FP32 outputs, partial sums promoted
// to FP32 at a fixed K interval; page 4, "Deepseek veroeffentlicht Deepgemm",
// section "Schluesselmerkmale von DeepGemm": dense and two MoE layouts):
//
//   D[m][n] = sum_kb sA[kb][m] * sB[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in chunk kb} A[m][k] * B[n][k]      (128-wide chunks)
//
// gfx950 design (the pages' Hopper scheme -- two warpgroups alternating WGMMA
// and promotion -- is prior art only):
//   * One chunk of 128 K is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16
//     output block, issued with a zero accumulator, so the MFMA result is the
//     chunk partial P in FP32.  The VALU then folds it into a second FP32
//     accumulator set with one FMA per element: acc += P * (sA * sB).  MFMA and
//     VALU are separate pipes, so the promotion overlaps the next MFMAs.
//   * The MFMA is issued with the weights as its first operand and the
//     activations as its second, i.e. it produces D^T blocks.  A lane then
//     holds four consecutive n of one m: the four values share one sA (per
//     lane) and one sB (per wave), so the scale is a single multiply per
//     16x16 block and the BF16 store is one 8-byte write.
//   * Workgroup: 256 lanes = 4 waves in a 2x2 grid; tile BM x BN, wave tile
//     BM/2 x BN/2.  A and B chunks (BM x 128 and BN x 128 bytes) and the BM
//     activation scales are streamed straight from HBM into LDS with 16-byte
//     global_load_lds (no VGPR staging), double buffered.  Rows are 128 bytes;
//     each 16-byte segment is XOR-swizzled by row so that the 16 lanes of an
//     MFMA fragment read hit distinct LDS banks.
//   * Workgroup ids are renumbered so that tiles sharing operand panels run
//     on the same XCD (own L2), then walked in groups of GROUP_M tile rows.
#include "device_common.h"
#include "launch.h"

namespace fp8bs {
namespace {

constexpr int kKC = 128;  // K chunk = promotion interval = MFMA K

template <int BM, int BN>
struct TileCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 fragments per wave
  static constexpr int A_BYTES = BM * kKC;
  static constexpr int B_BYTES = BN * kKC;
  static constexpr int SA_BYTES = BM * 4;
  static constexpr int SB_BYTES = 256;     // weight scales of the chunk (first BN/128 used)
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int A_LOADS = BM / 32;  // 8 rows per wave instruction, 4 waves
  static constexpr int B_LOADS = BN / 32;
  static constexpr int SA_WAVES = BM / 64; // 64 scales per dword-DMA instruction
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must be a multiple of 64");
  static_assert(SA_WAVES < 4, "one wave must be free to fetch the weight scales");
  static_assert(WN <= 128, "a wave's columns must share one 128-row weight block");
};

// 16-byte segment swizzle of an LDS row: rows r and r+1 live in different
// halves of a 256-byte bank line, and (r >> 1) & 7 spreads 16 consecutive rows
// over 8 segments of each half.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* d;
  const int32_t* groups;
  int64_t M, N, K;
  int32_t G;
  int32_t tiles_m, tiles_n;
  int32_t group_m;
};

template <int BM, int BN, int MODE, bool OUT_F32>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs p) {
  using C = TileCfg<BM, BN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = p.K, N = p.N;
  const int KT = (int)(K / kKC);
  const int64_t NB = (N + 127) / 128;

  // ---- tile -> (group, tm, tn) -------------------------------------------
  const int total = (int)gridDim.x;
  const int pid = xcd_remap((int)blockIdx.x, total);
  int g = 0, tm, tn;
  if (MODE == kMasked) {
    const int per_g = p.tiles_m * p.tiles_n;
    g = pid / per_g;
    const int r = pid - g * per_g;
    tn = r / p.tiles_m;
    tm = r - tn * p.tiles_m;
  } else {
    const int width = p.group_m * p.tiles_n;
    const int grp = pid / width;
    const int first_m = grp * p.group_m;
    const int gsz = min(p.tiles_m - first_m, p.group_m);
    const int r = pid - grp * width;
    tm = first_m + r % gsz;
    tn = r / gsz;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const uint8_t* a_base = p.a;
  const float* sa_base = p.sa;
  const uint8_t* b_base = p.b;
  const float* sb_base = p.sb;
  int64_t m_alloc = p.M;     // rows that exist in memory (loads are clamped to them)
  int64_t m_valid = p.M;     // rows that are computed and stored
  int64_t sa_stride = p.M;   // distance between consecutive K chunks in sA
  int64_t d_row0 = 0;        // first output row of this group's block of D
  if (MODE == kContiguous) {
    const int32_t* offs = p.groups;
    if (m0 >= offs[p.G]) return;
    int gg = 0;
    while (gg + 1 < p.G && offs[gg + 1] <= m0) ++gg;
    g = gg;
    m_valid = offs[g + 1];
    b_base += (int64_t)g * N * K;
    sb_base += (int64_t)g * NB * KT;
  } else if (MODE == kMasked) {
    int64_t cnt = p.groups[g];
    cnt = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
    if (m0 >= cnt) return;
    m_valid = cnt;
    a_base += (int64_t)g * p.M * K;
    sa_base += (int64_t)g * KT * p.M;
    b_base += (int64_t)g * N * K;
    sb_base += (int64_t)g * NB * KT;
    d_row0 = (int64_t)g * p.M;
  }
  const uint8_t* a_tile = a_base + m0 * K;
  const uint8_t* b_tile = b_base + n0 * K;

  // ---- per-lane DMA sources (byte offsets from the tile base) ------------
  uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int row = (i * 4 + wave) * 8 + (lane >> 3);
    const int seg = (lane & 7) ^ swz(row);
    int64_t gr = m0 + row;
    if (gr > m_alloc - 1) gr = m_alloc - 1;
    a_off[i] = (uint32_t)((gr - m0) * K + seg * 16);
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int row = (i * 4 + wave) * 8 + (lane >> 3);
    const int seg = (lane & 7) ^ swz(row);
    int64_t gr = n0 + row;
    if (gr > N - 1) gr = N - 1;
    b_off[i] = (uint32_t)((gr - n0) * K + seg * 16);
  }
  int64_t sa_row = m0 + wave * 64 + lane;
  if (sa_row > m_alloc - 1) sa_row = m_alloc - 1;
  // weight scales: lane l of the last wave fetches the scale of weight block
  // row n0/128 + l (clamped), so LDS holds this tile's sB values per chunk.
  int64_t sb_blk = n0 / 128 + lane;
  if (sb_blk > NB - 1) sb_blk = NB - 1;
  const float* sb_lane = sb_base + sb_blk * KT;

  auto issue = [&](int kb, int stage) {
    uint8_t* st = smem + stage * C::STAGE;
    const uint8_t* ak = a_tile + (int64_t)kb * kKC;
    const uint8_t* bk = b_tile + (int64_t)kb * kKC;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(ak + a_off[i]),
                                       (lds_void*)(st + (i * 4 + wave) * 8 * kKC), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bk + b_off[i]),
                                       (lds_void*)(st + C::A_BYTES + (i * 4 + wave) * 8 * kKC), 16, 0, 0);
    if (wave < C::SA_WAVES)
      __builtin_amdgcn_global_load_lds((const void*)(sa_base + (int64_t)kb * sa_stride + sa_row),
                                       (lds_void*)(st + C::A_BYTES + C::B_BYTES + wave * 256), 4, 0, 0);
    if (wave == 3)
      __builtin_amdgcn_global_load_lds((const void*)(sb_lane + kb),
                                       (lds_void*)(st + C::A_BYTES + C::B_BYTES + C::SA_BYTES), 4, 0, 0);
  };

  // ---- per-lane fragment read offsets -----------------------------------
  const int fr = lane & 15, fg = lane >> 4;
  const uint32_t rd0 = fr * kKC + 16 * ((2 * fg) ^ swz(fr));
  const uint32_t rd1 = fr * kKC + 16 * ((2 * fg + 1) ^ swz(fr));
  const int a_row0 = wm * C::WM, b_row0 = wn * C::WN;
  const int sb_idx = (int)((n0 + b_row0) / 128 - n0 / 128);   // this wave's weight block in the tile

  v4f acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  for (int kb = 0; kb < KT; ++kb) {
    const int stage = kb & 1;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's DMA for chunk kb has landed
    __builtin_amdgcn_s_barrier();    // ... and every other wave's; stage^1 is free

    const uint8_t* st = smem + stage * C::STAGE;
    v8i af[C::FM], bfr[C::FN];
    float sav[C::FM];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const uint8_t* base = st + (a_row0 + 16 * j) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      af[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sav[j] = reinterpret_cast<const float*>(st + C::A_BYTES + C::B_BYTES)[a_row0 + 16 * j + fr];
    }
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const uint8_t* base = st + C::A_BYTES + (b_row0 + 16 * i) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      bfr[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const float sbv = reinterpret_cast<const float*>(st + C::A_BYTES + C::B_BYTES + C::SA_BYTES)[sb_idx];

    if (kb + 1 < KT) issue(kb + 1, stage ^ 1);

    float sc[C::FM];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) sc[j] = sav[j] * sbv;

    // Software pipeline: the MFMA of block b is issued before the promotion
    // FMAs of block b-1, so the VALU works while the matrix core runs.
    constexpr int NBLK = C::FN * C::FM;
    const v4f pz = {0.f, 0.f, 0.f, 0.f};
    v4f pc[2];
    pc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[0], af[0], pz, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int b = 1; b <= NBLK; ++b) {
      if (b < NBLK)
        pc[b & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[b / C::FM], af[b % C::FM], pz,
                                                                     0, 0, 0, 0, 0, 0);
      const int pb = b - 1;
      v4f& ac = acc[pb / C::FM][pb % C::FM];
#pragma unroll
      for (int r = 0; r < 4; ++r) ac[r] = __builtin_fmaf(pc[pb & 1][r], sc[pb % C::FM], ac[r]);
    }
  }

  // ---- epilogue: lane holds D[m][n .. n+3] per fragment ------------------
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    const int64_t n = n0 + b_row0 + 16 * i + 4 * fg;
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int64_t m = m0 + a_row0 + 16 * j + fr;
      if (m < m_valid && n < N) {
        const int64_t idx = (d_row0 + m) * N + n;
        if (OUT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.d) + idx) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.d) + idx) =
              make_uint2(pack2_bf16(acc[i][j][0], acc[i][j][1]), pack2_bf16(acc[i][j][2], acc[i][j][3]));
        }
      }
    }
  }
}

template <int BM, int BN, int MODE>
hipError_t launch_cfg(const GemmProblem& pr, hipStream_t stream) {
  GemmArgs a;
  a.a = pr.a; a.sa = pr.sa; a.b = pr.b; a.sb = pr.sb; a.d = pr.d; a.groups = pr.groups;
  a.M = pr.M; a.N = pr.N; a.K = pr.K; a.G = pr.G;
  a.tiles_m = (int32_t)((pr.M + BM - 1) / BM);
  a.tiles_n = (int32_t)((pr.N + BN - 1) / BN);
  a.group_m = 8;
  int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * (MODE == kMasked ? pr.G : 1);
  if (blocks == 0) return hipSuccess;
  if (pr.out_f32)
    hipLaunchKernelGGL((k_gemm<BM, BN, MODE, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, MODE, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream) {
  switch (p.mode) {
    case kDense: return launch_cfg<128, 128, kDense>(p, stream);
    case kContiguous: return launch_cfg<128, 128, kContiguous>(p, stream);
    default: return launch_cfg<128, 128, kMasked>(p, stream);
  }
}

}  // namespace fp8bs
