// Block-scaled FP8 GEMM whose activation operand is quantized on the way in.
//
// D = Q(X) * B^T for a BF16 activation X [M][K], where Q is the 1x128 tile
// quantization of the quantizers (page 1, the uniondaocoop.com post on
// DeepSeek's FP8 training framework, paragraph on 1x128 activation tiles;
// page 2, "A Deadly Mistake Uncovered on Deepseek China Ai", paragraph on
// hardware suggestions: cast to FP8 while the activations move from global
// to shared memory instead of a separate read and write).  The result equals
// fp8bs_quantize_1x128 followed by the FP32-scale GEMM bit for bit: the same
// tile maxima, scales and codes, the same MFMA fragments and the same
// promotion acc += P * (sA * sB) per 128-wide K chunk.
//
// Tile: BM = 64 rows x BN = 128 columns, four waves; wave w owns rows
// 16w .. 16w+15 (one MFMA fragment) and every column.  An LDS stage holds one
// K chunk: the 64 activation rows as raw BF16 (256 bytes per row) and the
// 128 weight rows as codes, both moved by memory -> LDS DMA; two stages (the
// DMA of the next chunk runs during this one) and one workgroup barrier per
// chunk, so that two workgroups fit on a CU.  Measured (interleaved, bit-
// identical outputs) against 64 x 128 with three stages and 64 x 256 with
// three stages, one workgroup per CU either way: 16384 x 256 x 7168 97.5
// against 132 / 102 us, 4096 x 512 x 7168 65.2 against 64.7 / 90.1 us,
// 8192 x 128 x 7168 60.6 against 60.4 us.  Per
// chunk each lane reads from the stage the 32 BF16 values that its MFMA
// fragment needs (row fr, the K positions of segments fg and fg + 4 of the
// code layout), takes the row's maximum with the three other lanes that hold
// the rest of that row, computes the tile scale, and quantizes its 32 values
// straight into the A fragment; the scale is the row's sA for the promotion.
// Every column tile quantizes its rows again, so the kernel pays off where
// few column tiles share an activation panel (small N).
//
// LDS layout of the raw activation rows: row r at r * 256, its 16-byte
// segment g at physical segment g ^ (r % 16), so that the 16 rows a wave's
// lanes read at the same offset hit 16 different segments.  Weight rows use
// the layout of the other kernels (gemm_common.h).
#include "gemm_common.h"
#include "quant_common.h"

namespace fp8bs {
namespace {

template <int BM_, int BN_, int S_>
struct QACfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int NW = BM / 16, THREADS = 64 * NW;   // one 16-row fragment per wave
  static constexpr int FN = BN / 16;                 // weight fragments per wave
  static constexpr int NG = 4;                       // weight fragments read at a time
  static constexpr int S = S_;                       // LDS stages: the DMA runs S - 1 chunks ahead
  static constexpr int A_BYTES = BM * 2 * kKC;       // BF16 rows of one chunk
  static constexpr int STAGE = A_BYTES + BN * kKC;
  static constexpr int LDS_BYTES = S * STAGE;
  static constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KB DMAs per wave per chunk
  static constexpr int B_DMA = BN * kKC / 1024 / NW;
  static constexpr int DMA = A_DMA + B_DMA;
  static_assert(BN % 128 == 0 && FN % NG == 0, "whole weight blocks and fragment groups");
  static_assert(A_BYTES % (1024 * NW) == 0 && (BN * kKC) % (1024 * NW) == 0, "whole DMAs per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "the stages fit in LDS");
  static_assert(BM * (BN * 4 + 16) <= LDS_BYTES, "the FP32 output tile fits in the stages");
};

template <class C, bool OUT_F32, bool POW2>
__global__ __launch_bounds__(C::THREADS) void k_gemm_qa(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = C::BM, BN = C::BN, FN = C::FN, NG = C::NG, S = C::S;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KT = (int)(K / kKC);
  const int64_t NBK = (N + 127) / 128;

  // Tiles of one row block are consecutive ids, on one XCD.
  const int total = p.tiles_m * p.tiles_n;
  const int pid = xcd_remap((int)blockIdx.x, total);
  if (pid < 0) return;
  const int64_t m0 = (int64_t)(pid / p.tiles_n) * BM;
  const int64_t n0 = (int64_t)(pid % p.tiles_n) * BN;

  // ---- DMA ------------------------------------------------------------------
  // Activation instruction j (rows 4j .. 4j+3, j = wave + NW*i): lane l
  // takes row 4j + l/16 into physical segment l % 16, i.e. logical segment
  // (l % 16) ^ (row % 16).  Weight instruction j (rows 8j .. 8j+7, j = wave +
  // NW*i): lane l takes row 8j + l/8 into physical segment l % 8, logical
  // (l % 8) ^ swz(row).  Rows past M or N read as zeros (range check), chunks
  // past K come from a zero-record descriptor.
  const int64_t a_rows = min<int64_t>(M - m0, BM), b_rows = min<int64_t>(N - n0, BN);
  const v4i ra = make_rsrc(p.a + m0 * K * 2, a_rows * K * 2);
  const v4i rb = make_rsrc(p.b + n0 * K, b_rows * K);
  const v4i r_none = make_rsrc(p.b, 0);
  uint32_t a_off[C::A_DMA], b_off[C::B_DMA];
#pragma unroll
  for (int i = 0; i < C::A_DMA; ++i) {
    const int row = 4 * (wave + C::NW * i) + (lane >> 4);
    a_off[i] = (uint32_t)(row * K * 2 + 16 * ((lane & 15) ^ (row & 15)));
  }
#pragma unroll
  for (int i = 0; i < C::B_DMA; ++i) {
    const int row = 8 * (wave + C::NW * i) + (lane >> 3);
    b_off[i] = (uint32_t)(row * K + 16 * ((lane & 7) ^ swz(row)));
  }
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int kb) __attribute__((always_inline)) {
    const bool in = kb < KT;
    const uint32_t st = smem_lds + (uint32_t)(kb % S) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_DMA; ++i)
      dma16(in ? ra : r_none, st + 4 * (wave + C::NW * i) * 256, a_off[i], in ? (uint32_t)kb * 256 : 0u);
#pragma unroll
    for (int i = 0; i < C::B_DMA; ++i)
      dma16(in ? rb : r_none, st + C::A_BYTES + 8 * (wave + C::NW * i) * kKC, b_off[i],
            in ? (uint32_t)kb * kKC : 0u);
  };

  // ---- fragments ------------------------------------------------------------
  const int fr = lane & 15, fg = lane >> 4;
  // The lane's 32 activation values: logical segments 2fg, 2fg+1 (K positions
  // 16fg .. 16fg+15) and 8+2fg, 9+2fg (64+16fg .. 64+16fg+15) of row 16w+fr.
  const int arow = 16 * wave + fr;
  uint32_t a_rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) a_rd[q] = (uint32_t)(arow * 256 + 16 * (((q >> 1) * 8 + 2 * fg + (q & 1)) ^ fr));
  const uint32_t rd0 = fr * kKC + 16 * (fg ^ swz(fr));
  const uint32_t rd1 = fr * kKC + 16 * ((fg + 4) ^ swz(fr));
  const __attribute__((address_space(4))) float* sbc = (const __attribute__((address_space(4))) float*)(p.sb);
  const int64_t blk0 = n0 / 128;

  const v4f pz = {0.f, 0.f, 0.f, 0.f};
  v4f acc[FN];
#pragma unroll
  for (int i = 0; i < FN; ++i) acc[i] = pz;

  static_assert(S >= 2, "a stage to fill while one is read");
#pragma unroll
  for (int c = 0; c < S - 1; ++c) issue(c);
  for (int kb = 0; kb < KT; ++kb) {
    // This wave's DMA of chunk kb has landed once at most its DMA of the S - 2
    // later chunks is outstanding; the barrier then shows every wave's, and
    // tells that every wave is done with chunk kb - 1, whose stage chunk
    // kb + S - 1 fills.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<(S - 2) * C::DMA>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(kb + S - 1);
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* st = smem + (kb % S) * C::STAGE;
    // ---- quantize the lane's 32 values of its row (1x128 tile kb) ----------
    uint4 raw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) raw[q] = *reinterpret_cast<const uint4*>(st + a_rd[q]);
    float x[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * q + 2 * e] = bf16_lo(w[e]);
        x[8 * q + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(x[e]));
    am = __builtin_fmaxf(am, __shfl_xor(am, 16));
    am = __builtin_fmaxf(am, __shfl_xor(am, 32));
    const TileScale ts = tile_scale<POW2>(am);
    uint32_t code[8];
    auto encode = [&](auto scaled) __attribute__((always_inline)) {
      constexpr bool SC = decltype(scaled)::value;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = quot<POW2>(SC ? x[4 * k + e] * ts.sx : x[4 * k + e], ts);
        code[k] = pack4_e4m3(y[0], y[1], y[2], y[3]);
      }
    };
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(ts.sx != 1.0f) != 0, 0))
      encode(std::true_type{});
    else
      encode(std::false_type{});
    const v8i fa = {(int)code[0], (int)code[1], (int)code[2], (int)code[3],
                    (int)code[4], (int)code[5], (int)code[6], (int)code[7]};
    const float sa = ts.s;

    // ---- MFMAs and promotion, NG weight fragments at a time --------------------
#pragma unroll
    for (int g = 0; g < FN / NG; ++g) {
      v8i fb[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint8_t* bf = st + C::A_BYTES + 16 * (NG * g + i) * kKC;
        const uint4 lo = *reinterpret_cast<const uint4*>(bf + rd0);
        const uint4 hi = *reinterpret_cast<const uint4*>(bf + rd1);
        fb[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      v4f pc[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i)
        pc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[i], fa, pz, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int f = NG * g + i;
        const int64_t blk = min<int64_t>(blk0 + (16 * f) / 128, NBK - 1);
        const float sc = sa * sbc[blk * KT + kb];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[f][r] = __builtin_fmaf(pc[i][r], sc, acc[f][r]);
      }
    }
  }
  // The DMA past the last chunk (zeros) must land, and every wave be done
  // with the stages, before LDS is reused.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();

  // ---- epilogue: through LDS, then whole rows --------------------------------
  constexpr int ES = OUT_F32 ? 4 : 2;
  constexpr int RSTR = BN * ES + 16;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    uint8_t* dst = smem + arow * RSTR + (16 * i + 4 * fg) * ES;
    if (OUT_F32) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(acc[i][0], acc[i][1]), pack2_bf16(acc[i][2], acc[i][3]));
    }
  }
  lds_barrier();
  constexpr int CPR = BN * ES / 16;
  for (int q = threadIdx.x; q < BM * CPR; q += C::THREADS) {
    const int row = q / CPR, piece = q - row * CPR;
    if (row < a_rows && piece * 16 < b_rows * ES) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + row * RSTR + piece * 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.d) + ((m0 + row) * N + n0) * ES + piece * 16) = v;
    }
  }
#endif
}

template <class C>
hipError_t launch_qa_cfg(const GemmProblem& pr, bool pow2, hipStream_t stream) {
  GemmArgs a;
  a.a = pr.a; a.sa = nullptr; a.b = pr.b; a.sb = pr.sb; a.d = pr.d; a.groups = nullptr;
  a.M = pr.M; a.N = pr.N; a.K = pr.K; a.G = 1;
  a.tiles_m = (int32_t)((pr.M + C::BM - 1) / C::BM);
  a.tiles_n = (int32_t)((pr.N + C::BN - 1) / C::BN);
  a.group_m = 1;
  a.accumulate = 0;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(C::THREADS);
  if (pow2) {
    if (pr.out_f32) hipLaunchKernelGGL((k_gemm_qa<C, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_qa<C, false, true>), grid, block, 0, stream, a);
  } else {
    if (pr.out_f32) hipLaunchKernelGGL((k_gemm_qa<C, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_qa<C, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

using QATile = QACfg<64, 128, 2>;

int32_t gemm_qa_tile_n(int64_t) { return QATile::BN; }

hipError_t launch_gemm_qa(const GemmProblem& p, bool pow2, hipStream_t stream) {
  return launch_qa_cfg<QATile>(p, pow2, stream);
}

}  // namespace fp8bs
