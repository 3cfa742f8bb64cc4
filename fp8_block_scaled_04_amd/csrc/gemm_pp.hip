// Block-scaled FP8 GEMM for gfx950, ping-pong main loop.
//
// What it computes is the same as the other GEMM kernels (page 1, the
// uniondaocoop.com post on DeepSeek's FP8 training framework: FP8 operands,
// BF16/FP32 outputs, partial sums promoted to FP32 at a fixed K interval):
//
//   D[m][n] = sum_kb sA[kb][m] * sB[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in chunk kb} A[m][k] * B[n][k]      (128-wide chunks)
//
// Schedule.  Eight waves, two per SIMD, in two groups of four (one wave of
// each group on every SIMD).  Every wave alternates two phases per K chunk:
//   load:    read its MFMA fragments and scales of this chunk from LDS into
//            registers, start its share of the DMA of chunk kb+2, and form
//            the chunk's scale products sA*sB;
//   compute: one v_mfma_f32_16x16x128_f8f6f4 per 16x16 block from registers
//            only (zero accumulator: the chunk partial P), each followed by
//            the promotion FMAs acc += P * sA*sB of the block two MFMAs back.
// Group 1 runs one phase behind group 0, so on every SIMD one wave computes
// while the other loads, and a workgroup barrier between phases hands the
// matrix core from one wave to the other.  The last two blocks' FMAs of a
// chunk are carried into the wave's next compute phase, so a wave reaches the
// barrier right after issuing its last MFMA.  Every memory -> LDS DMA is
// issued by a wave in its load phase, after its LDS reads: the texture unit
// takes one 1 KB DMA per ~16 cycles per CU at best, so a DMA can wait to be
// issued, and that wait must not hold up an MFMA stream.
//
// Tile: BM x BN outputs per workgroup, wave (simd s, group g) owns rows
// s*BM/4 .. and columns g*BN/2 .. .  LDS holds three stages of the operand
// chunks (rows of 128 bytes, 16-byte segments XOR-swizzled as in the other
// kernels) plus the chunk's activation scales; group 0 moves the activation
// rows (wave 0 also the scales, one 16-byte-per-lane DMA), group 1 the
// weight rows.  Each wave reads its two weight block scales per chunk through
// the scalar cache.  The DMA of chunk kb+2 goes into the stage chunk kb-1
// occupied, which both groups have read by then.
#include <type_traits>

#include "gemm_common.h"

namespace fp8bs {
namespace {

template <int BM_, int BN_>
struct PPCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int S = 3;                           // LDS stages
  static constexpr int NW = 8, THREADS = 64 * NW;
  static constexpr int WM = BM / 4, WN = BN / 2;        // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;      // 16x16 fragments per wave
  static constexpr int NB = FM * FN;                    // MFMAs per wave per chunk
  static constexpr int A_BYTES = BM * kKC, B_BYTES = BN * kKC;
  // The chunk's activation scales (one 16-byte-per-lane DMA: 4 rows per
  // lane, up to 256 rows)
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE = SA_OFF + 1024;
  static constexpr int LDS_BYTES = S * STAGE;
  static constexpr int LOADS = BM / 32;                 // 16-byte-per-lane operand DMAs per wave per chunk
  // Wave 0 adds the activation-scale DMA.
  static_assert(BM == BN, "both groups move the same number of rows");
  static_assert(BM <= 256, "one DMA carries the tile's activation scales");
  static_assert(WN <= 128 && WN % 16 == 0 && WM % 16 == 0, "whole fragments, at most two weight blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "the stages must fit in LDS");
};

using PP192 = PPCfg<192, 192>;

template <class C, int MODE, bool OUT_F32, bool HWS>
__global__ __launch_bounds__(C::THREADS) void k_gemm_pp(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = C::BM, BN = C::BN, FM = C::FM, FN = C::FN, NB = C::NB, S = C::S;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave & 3, g = wave >> 2;
  const int64_t K = p.K, N = p.N;
  const int KT = (int)(K / kKC);
  const int64_t NBK = (N + 127) / 128;

  Tile t;
  if (!map_tile<BM, BN, MODE>(p, K, KT, NBK, t)) return;
  const int64_t m0 = t.m0, n0 = t.n0;

  // ---- DMA: buffer resources and per-lane offsets -------------------------
  const int64_t a_rows = min<int64_t>(t.m_valid - m0, BM);
  const int64_t b_rows = min<int64_t>(N - n0, BN);
  const v4i ra = make_rsrc(t.a_base + m0 * K, a_rows * K);
  const v4i rb = make_rsrc(t.b_base + n0 * K, b_rows * K);
  const v4i rsa = make_rsrc(t.sa_base, KT * t.sa_stride * 4);
  const v4i rsb = make_rsrc(t.sb_base, NBK * KT * 4);
  const v4i r_none = make_rsrc(p.a, 0);
  const v4i rop = g == 0 ? ra : rb;
  // Instruction i of wave s moves operand rows 8*(4i + s) .. +7: lane l row
  // 8*(4i+s) + l/8, physical segment l%8 = logical segment (l%8) ^ swz(row),
  // and swz(row) = 4*(s&1) + l/16 for every i.
  const uint32_t row_off = (uint32_t)(((s * 8 + (lane >> 3)) * K) + (((lane & 7) ^ (((s & 1) << 2) + (lane >> 4))) * 16));
  const uint32_t row_step = (uint32_t)(32 * K);
  const uint32_t op_lds = g == 0 ? 0u : (uint32_t)C::A_BYTES;
  // Scales.  Wave 0 moves the chunk's activation scales into LDS, rows m0 +
  // 4l .. 4l+3 in lane l (16 bytes; rows past the tile land in unused LDS).
  // The rows of sA are a multiple of 4 (the dispatcher checks), so a lane's
  // 16 bytes are either all inside a chunk's row of sA or past its end: past
  // the last chunk's row the range check returns zeros, before it they are
  // the next row's first values, never read.  The weight block scales are
  // wave-uniform: every wave reads its two through the scalar cache.
  const uint32_t sa_voff = (uint32_t)((m0 + 4 * lane) * 4);
  const uint32_t sa_step = __builtin_amdgcn_readfirstlane((uint32_t)(t.sa_stride * 4));
  const uint32_t smem_lds = lds_addr(smem);
  const __attribute__((address_space(4))) float* sbc =
      (const __attribute__((address_space(4))) float*)(t.sb_base);

  // This wave's share of chunk kb's DMA into LDS stage `stage`: LOADS
  // operand-row DMAs, and for wave 0 (SCW) the activation-scale DMA.  Chunks
  // past the end use a zero-record descriptor: zeros land in LDS and no
  // memory is read.
  // DMA instruction i of that share (i == LOADS: the scale DMA, wave 0 only).
  auto issue_one = [&](int kb, int stage, int i, auto scw) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + stage * C::STAGE;
    const bool live = kb < KT;
    if (i < C::LOADS) {
      const uint32_t koff = live ? (uint32_t)kb * kKC : 0u;
      uint32_t ro = row_off;
      asm volatile("" : "+v"(ro));
      dma16(live ? rop : r_none, st + op_lds + (4 * i + s) * 8 * kKC, ro + i * row_step, koff);
    } else if constexpr (decltype(scw)::value) {
      const uint32_t soff = __builtin_amdgcn_readfirstlane(live ? (uint32_t)kb * sa_step : 0u);
      dma16(live ? rsa : r_none, st + C::SA_OFF, sa_voff, soff);
    }
  };
  auto issue = [&](int kb, int stage, auto scw) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + stage * C::STAGE;
    const bool live = kb < KT;
    const uint32_t koff = live ? (uint32_t)kb * kKC : 0u;
    uint32_t ro = row_off;
    asm volatile("" : "+v"(ro));
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      dma16(live ? rop : r_none, st + op_lds + (4 * i + s) * 8 * kKC, ro + i * row_step, koff);
    if constexpr (decltype(scw)::value) {
      const uint32_t soff = __builtin_amdgcn_readfirstlane(live ? (uint32_t)kb * sa_step : 0u);
      dma16(live ? rsa : r_none, st + C::SA_OFF, sa_voff, soff);
    }
  };
  // Wait until at most one chunk's DMA of this wave is in flight.
  auto wait_one_chunk = [&](auto scw) __attribute__((always_inline)) {
    if constexpr (decltype(scw)::value) wait_vm_lgkm0<C::LOADS + 1>();
    else wait_vm_lgkm0<C::LOADS>();
  };

  // ---- fragments and scales ----------------------------------------------
  const int fr = lane & 15, fg = lane >> 4;
  const uint32_t rd0 = fr * kKC + 16 * (fg ^ swz(fr));
  const uint32_t rd1 = fr * kKC + 16 * ((fg + 4) ^ swz(fr));
  const int a_row0 = s * C::WM, b_row0 = g * C::WN;
  // weight block (within the tile's) of each weight fragment of the wave
  const int blk_lo = (int)((n0 + b_row0) / 128 - n0 / 128);
  int hi_from = FN;   // first fragment in the next weight block
#pragma unroll
  for (int i = FN - 1; i >= 0; --i)
    if ((int)((n0 + b_row0 + 16 * i) / 128 - n0 / 128) != blk_lo) hi_from = i;
  hi_from = __builtin_amdgcn_readfirstlane(hi_from);
  const int64_t sb_lo_off = (n0 / 128 + blk_lo) * (int64_t)KT;
  const int64_t sb_hi_off = min<int64_t>(n0 / 128 + blk_lo + 1, NBK - 1) * (int64_t)KT;

  v8i fa[FM], fb[FN];
  float sc[FN][FM];     // software promotion: sA*sB per block
  int ea[FM], eb[FN];   // hardware scaling: E8M0 bytes
  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f pz = {0.f, 0.f, 0.f, 0.f};
  v4f pc[3] = {pz, pz, pz};   // chunk partials in flight (block b in slot (kb*NB + b) % 3)
  float dsc[2] = {0.f, 0.f};  // scales of the two blocks carried into the next compute phase

  auto read_frag = [&](const uint8_t* base) __attribute__((always_inline)) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // Load phase of chunk kb (in stage `stage`): read this wave's scales and
  // fragments, with this wave's share of chunk kb+2's DMA (into the stage
  // chunk kb-1 used) interleaved, one DMA after every two fragments, so the
  // LDS and the texture unit work at the same time; then form the scale
  // products.  The DMA is issued here, not between the MFMAs: a DMA waiting
  // for the texture unit would hold up the MFMA stream behind it (measured
  // on 4096x2112x7168: 63.4 us with the DMA after the reads, 65.9 us with
  // half of each wave's share spread through its compute phase, 59.9 us
  // interleaved with the reads, that one with the epilogue below).
  // The load phase is the longer of the two (≈700 cycles per chunk against
  // ≈650 for the compute phase), so its wave issues at raised priority: where
  // the two waves of a SIMD compete for an issue slot, the loads go first
  // (4096x2112x7168: 60.4 -> 58.9 us, interleaved; raising the compute
  // phase's priority instead was slower).
  auto load = [&](int kb, int stage, auto scw) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    const uint8_t* st = smem + stage * C::STAGE;
    float sa[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) sa[j] = reinterpret_cast<const float*>(st + C::SA_OFF)[a_row0 + 16 * j + fr];
    const float sb_lo = sbc[sb_lo_off + kb];
    const float sb_hi = sbc[sb_hi_off + kb];   // used only by fragments past the block boundary
    {
      const int dst_stage = stage == 0 ? 2 : stage - 1;
      // fragment f (0 .. FM+FN-1), and DMA instruction d after every
      // EVERY fragments; the rest after the last fragment
      constexpr int NF = FM + FN;
      constexpr int NDMA = C::LOADS + 1;
      constexpr int EVERY = (NF + NDMA - 1) / NDMA;
      int d = 0;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f < FM) fa[f] = read_frag(st + (a_row0 + 16 * f) * kKC);
        else fb[f - FM] = read_frag(st + C::A_BYTES + (b_row0 + 16 * (f - FM)) * kKC);
        if ((f + 1) % EVERY == 0 && d < NDMA) {
          __builtin_amdgcn_sched_barrier(0);
          issue_one(kb + 2, dst_stage, d, scw);
          __builtin_amdgcn_sched_barrier(0);
          ++d;
        }
      }
#pragma unroll
      for (int dd = (NF / EVERY); dd < NDMA; ++dd) issue_one(kb + 2, dst_stage, dd, scw);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (HWS) {
#pragma unroll
      for (int j = 0; j < FM; ++j) ea[j] = e8m0_of(sa[j]);
      const int elo = __builtin_amdgcn_readfirstlane(e8m0_of(sb_lo));
      const int ehi = __builtin_amdgcn_readfirstlane(e8m0_of(sb_hi));
#pragma unroll
      for (int i = 0; i < FN; ++i) eb[i] = i >= hi_from ? ehi : elo;
    } else {
      const float slo = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sb_lo)));
      const float shi = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sb_hi)));
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const float sbi = i >= hi_from ? shi : slo;
#pragma unroll
        for (int j = 0; j < FM; ++j) sc[i][j] = sa[j] * sbi;
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto fma_block = [&](v4f& ac, const v4f& pv, float scale) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) ac[r] = __builtin_fmaf(pv[r], scale, ac[r]);
  };

  // Compute phase (chunk in stage `stage`): the MFMAs from registers, each
  // followed by the promotion FMAs of the block two MFMAs back.  Each MFMA
  // with its FMAs is one scheduling region, so the issue order is the program
  // order.  The stage parity fixes the partial slots.
  auto compute = [&](int stage) __attribute__((always_inline)) {
    const int base = stage * NB;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = b / FM, j = b % FM;
      if constexpr (HWS) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[i], fa[j], acc[i][j], 0, 0, 0, eb[i], 0,
                                                                     ea[j]);
      } else {
        pc[(base + b) % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[i], fa[j], pz, 0, 0, 0, 0, 0, 0);
        if (b < 2) {
          const int pb = NB - 2 + b;   // carried from the previous chunk
          fma_block(acc[pb / FM][pb % FM], pc[(base - 2 + b + 3 * NB) % 3], dsc[b]);
        } else {
          const int pb = b - 2;
          fma_block(acc[pb / FM][pb % FM], pc[(base + pb) % 3], sc[pb / FM][pb % FM]);
        }
        // the MFMA first: its FMAs then read a partial two MFMAs old (no
        // hazard waits), and the MFMA issues as soon as the matrix core is free
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!HWS) {
      dsc[0] = sc[(NB - 2) / FM][(NB - 2) % FM];
      dsc[1] = sc[(NB - 1) / FM][(NB - 1) % FM];
    }
  };

  // ---- main loop (specialised for wave 0, which also moves the scales) ---
  auto run = [&](auto scw) __attribute__((always_inline)) {
    auto sync = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      wait_one_chunk(scw);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // Prologue: chunks 0 and 1 on their way; everyone waits for chunk 0.
    issue(0, 0, scw);
    issue(1, 1, scw);
    sync();
    if (g == 1) sync();  // group 1 runs one phase behind
    auto chunk = [&](int kb, int stage) __attribute__((always_inline)) {
      load(kb, stage, scw);
      sync();
      compute(stage);
      sync();
    };
    int kb = 0;
    for (; kb + S - 1 < KT; kb += S) {
      chunk(kb, 0);
      chunk(kb + 1, 1);
      chunk(kb + 2, 2);
    }
    if (kb < KT) chunk(kb, 0);
    if (kb + 1 < KT) chunk(kb + 1, 1);
    if (g == 0) sync();  // the barrier group 1 still meets
  };
  if (wave == 0) run(std::true_type{});
  else run(std::false_type{});
  if (!HWS) {
    // the carried blocks of the last chunk (its stage parity is (KT-1) % 3)
    const int base = ((KT - 1) % 3) * NB;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int pb = NB - 2 + b;
      const int slot_i = (base + pb) % 3;
      const v4f pv = slot_i == 0 ? pc[0] : (slot_i == 1 ? pc[1] : pc[2]);
      fma_block(acc[pb / FM][pb % FM], pv, dsc[b]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // no LDS write may still be in flight at exit

  // ---- epilogue: through LDS, then whole rows -----------------------------
  // Every tile stores at the same moment, so the epilogue is a burst of the
  // whole output; written from the fragments directly (8 bytes per lane, 32
  // bytes per row segment) it took 2.2 us longer on 4096x2112x384 than
  // staged in the free LDS and stored in 16-byte pieces of whole rows.
  const int64_t m_valid = t.m_valid, d_row0 = t.d_row0;
  constexpr int ES = OUT_F32 ? 4 : 2;                 // bytes per output
  constexpr int RSTR = BN * ES + 16;                  // LDS row stride (padded)
  static_assert(BM * RSTR <= C::LDS_BYTES, "the output tile fits in LDS");
  lds_barrier();                                      // every wave is done with the stages
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int col = b_row0 + 16 * i + 4 * fg;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int row = a_row0 + 16 * j + fr;
      uint8_t* dst = smem + row * RSTR + col * ES;
      if (OUT_F32) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack2_bf16(acc[i][j][0], acc[i][j][1]), pack2_bf16(acc[i][j][2], acc[i][j][3]));
      }
    }
  }
  lds_barrier();
  constexpr int CPR = BN * ES / 16;                   // 16-byte pieces per row
  const int64_t rows = min<int64_t>(m_valid - m0, BM);
  const int64_t cols = min<int64_t>(N - n0, BN);      // a multiple of 8 (N % 16 == 0)
  for (int q = threadIdx.x; q < BM * CPR; q += C::THREADS) {
    const int row = q / CPR, piece = q - row * CPR;
    if (row < rows && piece * 16 < cols * ES) {
      const uint4 v = *reinterpret_cast<const uint4*>(smem + row * RSTR + piece * 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.d) + ((d_row0 + m0 + row) * N + n0) * ES + piece * 16) = v;
    }
  }
#endif
}

template <class C, int MODE>
hipError_t launch_pp_cfg(const GemmProblem& pr, hipStream_t stream) {
  GemmArgs a;
  a.a = pr.a; a.sa = pr.sa; a.b = pr.b; a.sb = pr.sb; a.d = pr.d; a.groups = pr.groups;
  a.M = pr.M; a.N = pr.N; a.K = pr.K; a.G = pr.G;
  a.tiles_m = (int32_t)((pr.M + C::BM - 1) / C::BM);
  if (MODE == kContiguous) a.tiles_m = (int32_t)(pr.M / C::BM + pr.G);
  a.tiles_n = (int32_t)((pr.N + C::BN - 1) / C::BN);
  a.group_m = 8;
  a.accumulate = 0;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(C::THREADS);
  if (pr.hw_scale) {
    if (pr.out_f32) hipLaunchKernelGGL((k_gemm_pp<C, MODE, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_pp<C, MODE, false, true>), grid, block, 0, stream, a);
  } else {
    if (pr.out_f32) hipLaunchKernelGGL((k_gemm_pp<C, MODE, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_gemm_pp<C, MODE, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

// Requires the rows of sA (M, or Mt) to be a multiple of 4.
hipError_t launch_gemm_pp192(const GemmProblem& p, hipStream_t stream) {
  if (p.mode == kContiguous) return launch_pp_cfg<PP192, kContiguous>(p, stream);
  return launch_pp_cfg<PP192, kDense>(p, stream);
}

}  // namespace fp8bs
