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
//     accumulator set with one FMA per element: acc += P * (sA * sB).  The
//     MFMA of block b is issued before the FMAs of block b-1, so the VALU
//     works while the matrix core runs.
//   * The MFMA is issued with the weights as its first operand and the
//     activations as its second, i.e. it produces D^T blocks.  A lane then
//     holds four consecutive n of one m: the four values share one sA (per
//     lane) and one sB (per wave), so the scale is a single multiply per
//     16x16 block and the BF16 store is one 8-byte write.
//   * Operand traffic sets the tile: L2 feeds a CU about 37 bytes per clock
//     (measured), a 16x16x128 MFMA takes 32 clocks per SIMD, so a tile must
//     load at most ~300 bytes per MFMA to keep the matrix cores busy.  A
//     256x256 tile loads 256 bytes per MFMA (8 waves, two per SIMD, wave tile
//     64x128); 128x128 (4 waves, 64x64 each) loads 512 and serves the shapes
//     that have too few 256x256 tiles to fill 256 CUs, as do 256x160 (8 waves
//     of 64x80) and 192x192 (12 waves of 64x48, three per SIMD).
//   * A and B chunks (BM x 128 and BN x 128 bytes) and the chunk's scales are
//     streamed straight from memory into LDS with buffer_load ... lds (no
//     VGPR staging; the K offset is a scalar), two or three stages, in whole
//     128-byte rows with a swizzle that lets MFMA fragments read LDS at close
//     to its full rate.  The DMA of a freed stage starts right after each
//     step's barrier.  The 128x128 tile double-buffers its MFMA fragments in
//     registers; the 256-wide tiles rotate their weight fragments through a
//     small register ring, each read two MFMA rows ahead of its use.
//   * Waves whose rows all lie past the valid rows (a masked expert's count,
//     a ragged last tile) skip their MFMAs and only keep the DMA and barrier
//     rhythm.
//   * Workgroup ids are renumbered so that tiles sharing operand panels run
//     on the same XCD (own L2), then walked in groups of group_m tile rows
//     (4 for 256-row tiles, 8 for the smaller ones).
#include "gemm_common.h"
#include "splitk.h"

namespace fp8bs {
namespace {


template <int BM_, int BN_, int WGM_, int WGN_, bool DB_, int S_ = 2, bool CS_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr bool DB = DB_;                   // fragments double buffered in registers
  static constexpr int S = S_;                      // LDS stages (chunks in flight + 1)
  static constexpr int NW = WGM * WGN;              // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 fragments per wave
  static constexpr int A_BYTES = BM * kKC;
  static constexpr int B_BYTES = BN * kKC;
  // Scale DMAs (64 floats each): waves 0..BM/64-1 fetch the activation
  // scales of the tile's rows into slots 0..BM/64-1, wave BM/64 the weight
  // scales of weight block rows n0/128 + i into slot BM/64 (the weight
  // gradient: waves BM/64.. the per-row weight scales, one slot per 64 rows).
  // Compact scales (CS) keep only the slots the dense and grouped modes use,
  // which frees LDS for a third stage of the 256x160 tile.
  static constexpr int SA_WAVES = BM / 64;
  static constexpr bool CS = CS_;
  static constexpr int SC_BYTES = CS ? (SA_WAVES + 1) * 256 : NW * 256;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int SB_OFF = A_BYTES + B_BYTES + SA_WAVES * 256;
  static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
  static constexpr int A_LOADS = BM / (8 * NW);     // 8 rows of 128 bytes per wave instruction
  // Weight rows go in groups of 8 (one 16-byte-per-lane instruction each),
  // dealt round-robin: every wave issues B_FULL, waves below B_EXTRA one
  // more and the others repeat one of theirs.  (Every DMA instruction costs
  // the texture unit about the same time whatever its width: the 4-byte
  // loads that had carried the last 32 rows of 160 cost 7 % on 4096x2112.)
  static constexpr int B_GROUPS = BN / 8;
  static constexpr int B_FULL = B_GROUPS / NW;
  static constexpr int B_EXTRA = B_GROUPS % NW;
  static_assert(B_EXTRA == 0 || B_FULL >= 1, "a wave without an extra group repeats one of its own");
  static constexpr int LDS_BYTES = S * STAGE;
  static constexpr int WG_PER_CU = (160 * 1024) / LDS_BYTES;
  static_assert(BM % (8 * NW) == 0 && BN % 16 == 0, "A rows split evenly over the waves; B rows are fragments");
  static_assert(SA_WAVES < NW, "one wave must be left for the weight scales");
  static_assert(WN % 16 == 0 && WN <= 128, "a wave's columns are whole fragments within at most two weight blocks");
  static_assert(DB_ == false || 128 % WN == 0, "the double-buffered path needs a wave's columns in one weight block");
  static_assert(LDS_BYTES <= 160 * 1024, "the stages must fit in LDS");
  static_assert(S >= 2 && (!DB || S == 2), "the double-buffered path has two stages");
};

using SmallTile = Cfg<128, 128, 2, 2, true>;
using LargeTile = Cfg<256, 256, 4, 2, false>;
// 256x160 with three stages (compact scales: 160 KB of LDS): measured on
// 4096x2112x7168 right after the quantizer wrote A, 87 -> 78 us, and 96 ->
// 83 us with cold caches; two stages for the weight gradient.
using MidTile = Cfg<256, 160, 4, 2, false, 3, true>;
using WgradMidTile = Cfg<256, 160, 4, 2, false>;
// 192x192 with 12 waves (3x4, 64x48 each: three waves per SIMD), three
// stages, compact scales (147 KB of LDS).  On 4096x2112x7168 it makes 242
// tiles of 10 % less work than the 224 of 256x160 and hides more latency
// with its third wave per SIMD: 69.7 -> 65.2 us on random codes, 66.0 ->
// 57.8 us on zero codes (interleaved A/B; outputs bit-identical).  One wave
// per SIMD (256x160 as 4 waves of 64x160) was far slower (109 us).
using Tile192 = Cfg<192, 192, 3, 4, false, 3, true>;
// Memory-bound shapes (few rows): 128x96 tiles, three stages, one
// workgroup per CU on the 24576-column decode projection.
using StreamTile = Cfg<128, 96, 2, 2, false, 3>;
// Few rows and too few larger tiles to fill the GPU: 64x64 tiles (two waves
// of 64x32), four stages, two workgroups per CU.  Each CU then takes a
// smaller share of the operands: 128 instead of 224 bytes per K column of
// its tile.  Interleaved A/B against 128x96 on rotating weight sets,
// outputs bit-identical: 128x7168x2048 13.8 -> 10.1 us, 128x8192x2048 14.2
// -> 9.9 us, 96x4096x7168 34.4 -> 20.4 us, 64x2112x7168 28.1 -> 20.9 us,
// 128x12288x1536 (384 tiles) 13.0 -> 12.4 us.  Three stages were slower on
// every shape (up to 25 %), and five, six or eight no faster.  At 768 tiles
// (128x24576x1536) it takes 16.0 against 13.9 us, so the decode projection
// keeps 128x96.
using Stream64Tile = Cfg<64, 64, 1, 2, false, 4>;
// Masked (decode-time MoE) layout: 128x256 tiles with three stages (64 KB
// of weights in flight per CU; an expert above 128 rows takes two row tiles,
// which run next to each other and share the weight panel in L2).  Waves
// past an expert's count skip their MFMAs.  32 experts x 256 capacity, N
// 7168, K 2048 (interleaved A/B against 256x256 tiles with two stages):
// 16 rows per expert 129 -> 112 us, 64 rows 139 -> 125 us, 128 rows 157 ->
// 142 us, counts uniform in 0..256 164 -> 168 us, every expert full 190 ->
// 212 us.
using MaskedTile = Cfg<128, 256, 2, 4, false, 3, true>;

// Fragment rows per wave staged at once by the epilogue: the most that
// divide FM and fit in `lds` bytes at `bytes_per_frag_row` each.
constexpr int epi_frags_per_pass(int fm, int bytes_per_frag_row, int lds) {
  int jp = fm;
  while (jp > 1 && (fm % jp != 0 || jp * bytes_per_frag_row > lds)) --jp;
  return jp;
}

template <int FM, int FN>
struct Frags {
  v8i a[FM];
  v8i b[FN];
  float sa[FM];
  float sb;
};


// HWS (hardware scaling; every scale a power of two): the MFMA applies the
// chunk's scales as E8M0 exponents per operand row -- the weight fragment's
// block scale on the first operand, each lane's activation-row scale on the
// second -- and adds the scaled chunk product to the accumulator it is given,
// so the promotion needs no VALU work.
template <class C, int MODE, bool OUT_F32, bool HWS>
__global__ __launch_bounds__(C::THREADS) void k_gemm(const GemmArgs p) {
  // The body uses AMDGPU buffer descriptors, which exist in the device pass
  // only; the host pass needs just the kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int64_t K = p.K, N = p.N;
  const int KTS = (int)(K / kKC);   // chunks of the whole K (strides of the weight-scale grid)
  int KT = KTS;                     // chunks this workgroup runs
  const int64_t NB = (N + 127) / 128;

  Tile t;
  int split_tile = 0, split = 0, kb0 = 0;
  if constexpr (MODE == kSplitK) {
    // Dense, split K: workgroup b runs split b % G (p.G splits) of tile b / G
    // (tiles column-major over tiles_m row tiles), chunks [kb0, kb1); the
    // operand and scale bases start at chunk kb0 (row strides unchanged).
    const int S = p.G;
    split_tile = (int)blockIdx.x / S;
    split = (int)blockIdx.x - split_tile * S;
    kb0 = (int)((int64_t)split * KTS / S);
    KT = (int)((int64_t)(split + 1) * KTS / S) - kb0;
    t.a_base = p.a + (int64_t)kb0 * kKC;
    t.sa_base = p.sa + (int64_t)kb0 * p.M;
    t.b_base = p.b + (int64_t)kb0 * kKC;
    t.sb_base = p.sb + kb0;
    t.m_alloc = p.M;
    t.m_valid = p.M;
    t.sa_stride = p.M;
    t.d_row0 = 0;
    t.m0 = (int64_t)(split_tile % p.tiles_m) * BM;
    t.n0 = (int64_t)(split_tile / p.tiles_m) * BN;
  } else {
    if (!map_tile<BM, BN, MODE>(p, K, KT, NB, t)) return;
  }
  const uint8_t* a_base = t.a_base;
  const float* sa_base = t.sa_base;
  const uint8_t* b_base = t.b_base;
  const float* sb_base = t.sb_base;
  const int64_t m_alloc = t.m_alloc, m_valid = t.m_valid, sa_stride = t.sa_stride, d_row0 = t.d_row0;
  const int64_t m0 = t.m0, n0 = t.n0;

  // ---- buffer resources (SGPRs) and per-lane DMA offsets ------------------
  // Rows past the valid ones (a masked expert's count, a group's end) are
  // out of range: the DMA writes zeros for them and reads no memory.
  const int64_t a_rows = min<int64_t>(m_valid - m0, BM);
  const int64_t b_rows = min<int64_t>(N - n0, BN);
  const v4i ra = make_rsrc(a_base + m0 * K, a_rows * K);
  const v4i rb = make_rsrc(b_base + n0 * K, b_rows * K);
  const v4i rsa = make_rsrc(sa_base, KT * sa_stride * 4);
  const v4i rsb = make_rsrc(sb_base, NB * KTS * 4 - (int64_t)kb0 * 4);

  // DMA instruction t = i*NW + wave moves rows 8t .. 8t+7 (whole 128-byte
  // lines), lane l taking row 8t + l/8, physical segment l%8, i.e. logical
  // segment (l%8) ^ swz(row).  With NW even, swz(row) = 4*(wave&1) + l/16
  // for every instruction of the wave, so one base offset serves all of them
  // for both operands.  The row stays in the vector offset, where the
  // hardware range check sees it: rows past the end of A or B (a ragged last
  // tile) are out of range and read as zeros.
  static_assert(C::NW % 2 == 0, "the DMA mapping needs an even number of waves");
  const uint32_t row_off = (uint32_t)(((wave * 8 + (lane >> 3)) * K) +
                                      (((lane & 7) ^ (((wave & 1) << 2) + (lane >> 4))) * 16));
  const uint32_t row_step = (uint32_t)(C::NW * 8 * K);
  // Scale DMA of this wave (one dword per lane per chunk): waves below
  // SA_WAVES fetch activation scales of rows m0 + 64*wave + lane, wave
  // SA_WAVES the weight scale of block row n0/128 + lane (both clamped).
  // (kWgrad: waves SA_WAVES .. SCW-1 fetch weight-row scales n0 + 64*(wave -
  // SA_WAVES) + lane from the [K/128][N] layout, landing right after the
  // activation scales.)  Waves from SCW on repeat wave SCW-1's DMA (the same
  // bytes to the same LDS slot): every wave then issues the same number of
  // DMAs per chunk, so the waits are compile-time constants and the loop has
  // no per-wave branches (which split its scheduling regions and made the
  // register allocator spill).
  constexpr int SCW = C::SA_WAVES + (MODE == kWgrad ? (BN + 63) / 64 : 1);
  static_assert(SCW <= C::NW, "every scale slot needs a wave");
  static_assert(!C::CS || SCW <= C::SA_WAVES + 1, "compact scales hold one weight-scale slot");
  const int scw = wave < SCW ? wave : SCW - 1;   // the scale DMA this wave issues
  const bool sa_wave = scw < C::SA_WAVES;
  int64_t sa_row = m0 + (sa_wave ? scw : 0) * 64 + lane;
  if (sa_row > m_alloc - 1) sa_row = m_alloc - 1;
  int64_t sb_blk = n0 / 128 + lane;
  if (sb_blk > NB - 1) sb_blk = NB - 1;
  int64_t sb_row = n0 + (sa_wave ? 0 : scw - C::SA_WAVES) * 64 + lane;
  if (sb_row > N - 1) sb_row = N - 1;
  const v4i rsb_w = make_rsrc(sb_base, (int64_t)KT * N * 4);
  const v4i rsc = sa_wave ? rsa : (MODE == kWgrad ? rsb_w : rsb);
  const uint32_t sc_voff = sa_wave ? (uint32_t)(sa_row * 4)
                                   : (MODE == kWgrad ? (uint32_t)(sb_row * 4) : (uint32_t)(sb_blk * KTS * 4));
  const uint32_t sc_step = __builtin_amdgcn_readfirstlane(
      sa_wave ? (uint32_t)(sa_stride * 4) : (MODE == kWgrad ? (uint32_t)(N * 4) : 4u));

  // Chunks past the end (the pipeline issues ahead) use descriptors with
  // zero records: every lane is out of range, so the hardware writes zeros
  // to LDS and reads no memory.
  const v4i r_none = make_rsrc(p.a, 0);
  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int kb, int stage) {
    const uint32_t st = smem_lds + stage * C::STAGE;
    const bool live = kb < KT;
    const uint32_t koff = live ? (uint32_t)kb * kKC : 0u;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(live ? (uint32_t)kb * sc_step : 0u);
    const v4i rak = live ? ra : r_none;
    const v4i rbk = live ? rb : r_none;
    const v4i rck = live ? rsc : r_none;
    // Recomputed per chunk (one add per instruction) rather than kept live:
    // the opaque copy stops the compiler from hoisting them into registers.
    uint32_t ro = row_off;
    asm volatile("" : "+v"(ro));
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      dma16(rak, st + (i * C::NW + wave) * 8 * kKC, ro + i * row_step, koff);
#pragma unroll
    for (int i = 0; i < C::B_FULL; ++i)
      dma16(rbk, st + C::A_BYTES + (i * C::NW + wave) * 8 * kKC, ro + i * row_step, koff);
    // Weight group B_FULL*NW + wave for waves below B_EXTRA; the others
    // repeat their last group (same bytes, same LDS rows).
    if constexpr (C::B_EXTRA > 0) {
      const int bi = wave < C::B_EXTRA ? C::B_FULL : C::B_FULL - 1;
      dma16(rbk, st + C::A_BYTES + (bi * C::NW + wave) * 8 * kKC, ro + bi * row_step, koff);
    }
    dma4(rck, st + C::SA_OFF + scw * 256, sc_voff, soff);
  };
  constexpr int DPC = C::A_LOADS + C::B_FULL + (C::B_EXTRA > 0 ? 1 : 0) + 1;   // DMA instructions per issue()
  // ---- per-lane fragment read offsets -----------------------------------
  const int fr = lane & 15, fg = lane >> 4;
  const uint32_t rd0 = fr * kKC + 16 * (fg ^ swz(fr));
  const uint32_t rd1 = fr * kKC + 16 * ((fg + 4) ^ swz(fr));
  const int a_row0 = wm * C::WM, b_row0 = wn * C::WN;
  const int sb_idx = (int)((n0 + b_row0) / 128 - n0 / 128);   // this wave's weight block in the tile

  // With fragments double buffered a wave holds every weight fragment of the
  // chunk; otherwise it holds half of them at a time (FNH).
  constexpr int FNH = C::DB ? C::FN : C::FN / 2;
  using F = Frags<C::FM, FNH>;
  auto read_a = [&](int stage, F& f) {
    const uint8_t* st = smem + stage * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const uint8_t* base = st + (a_row0 + 16 * j) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      f.a[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      f.sa[j] = reinterpret_cast<const float*>(st + C::SA_OFF)[a_row0 + 16 * j + fr];
    }
    f.sb = reinterpret_cast<const float*>(st + C::SB_OFF)[sb_idx];
  };
  // weight fragments i0 .. i0+FNH-1 of the wave
  auto read_b = [&](int stage, F& f, int i0) {
    const uint8_t* st = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < FNH; ++i) {
      const uint8_t* base = st + C::A_BYTES + (b_row0 + 16 * (i0 + i)) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      f.b[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };

  v4f acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Promotion of one chunk: the MFMA of block b is issued before the FMAs of
  // block b-1, so the VALU works while the matrix core runs.
  // The scale products sA*sB replace the activation scales of the set.
  auto scales = [&](F& f) {
#pragma unroll
    for (int j = 0; j < C::FM; ++j) f.sa[j] = f.sa[j] * f.sb;
  };
  // Blocks (i0 + i, j) for the FNH weight fragments held in f.
  auto compute_hws = [&](const F& f, int i0) {
    const int eb = e8m0_of(f.sb);
    int ea[C::FM];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) ea[j] = e8m0_of(f.sa[j]);
#pragma unroll
    for (int b = 0; b < FNH * C::FM; ++b) {
      v4f& ac = acc[i0 + b / C::FM][b % C::FM];
      ac = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[b / C::FM], f.a[b % C::FM], ac, 0, 0, 0, eb, 0,
                                                            ea[b % C::FM]);
    }
  };
  auto compute = [&](const F& f, int i0) {
    const float* sc = f.sa;
    constexpr int NBLK = FNH * C::FM;
    const v4f pz = {0.f, 0.f, 0.f, 0.f};
    v4f pc[2];
    pc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[0], f.a[0], pz, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int b = 1; b <= NBLK; ++b) {
      if (b < NBLK)
        pc[b & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[b / C::FM], f.a[b % C::FM], pz,
                                                                     0, 0, 0, 0, 0, 0);
      const int pb = b - 1;
      v4f& ac = acc[i0 + pb / C::FM][pb % C::FM];
#pragma unroll
      for (int r = 0; r < 4; ++r) ac[r] = __builtin_fmaf(pc[pb & 1][r], sc[pb % C::FM], ac[r]);
    }
    // Keep that order through scheduling: the first MFMA, then each further
    // MFMA followed by the four FMAs of the block before it, then the last
    // block's FMAs.
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int b = 1; b < NBLK; ++b) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  };

  // ---- main loop ----------------------------------------------------------
  // Every step is straight-line code (one basic block), so the scheduling
  // barriers hold and no step needs more registers than another.  A step
  // waits for this wave's outstanding LDS reads and DMA, meets the other
  // waves at the barrier (so every wave's DMA has landed and every wave is
  // done reading the stage the next DMA overwrites), starts that DMA, then
  // reads fragments and computes.  Past the last chunk the DMA goes through
  // the zero-record descriptor and reads touch a stale stage.
  if constexpr (C::DB) {
    static_assert(MODE != kWgrad, "the weight gradient runs on the 256-wide tiles");
    // Two fragment sets: chunk kb's fragments were read in the previous
    // step; read chunk kb+1's while computing chunk kb.
    F f0, f1;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    issue(1, 1);
    read_a(0, f0);
    read_b(0, f0, 0);
    auto step = [&](int kb, F& cur, F& nxt, int stage) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lgkm0<0>();   // chunk kb+1's DMA has landed
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(kb + 2, stage);
      read_a(stage ^ 1, nxt);
      read_b(stage ^ 1, nxt, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HWS) {
        compute_hws(cur, 0);
      } else {
        scales(cur);
        compute(cur, 0);
      }
    };
    int kb = 0;
    for (; kb + 1 < KT; kb += 2) {
      step(kb, f0, f1, 0);
      step(kb + 1, f1, f0, 1);
    }
    if (kb < KT) step(kb, f0, f1, 0);
  } else {
    // The activation fragments and the scales are read for the whole chunk;
    // the weight fragments rotate through a ring of register slots, each
    // read two rows of MFMAs (2*FM blocks) before its first use, so the LDS
    // reads of a step overlap its MFMAs instead of preceding them.  Slot of
    // weight fragment i: i % 4, except that the last fragment gets a fifth
    // slot when i % 4 would be slot 0 or 1, which the next chunk's first two
    // fragments are read into during the last row.
    static_assert(C::FM == 4, "the last row is written for four activation fragments");
    static_assert(C::FN >= 2, "rows() computes at least one row before the last");
    constexpr int FN = C::FN;
    constexpr bool EXTRA = (FN % 4 == 1) || (FN % 4 == 2);
    constexpr int SLOTS = EXTRA ? 5 : 4;
    auto slot = [](int i) { return (EXTRA && i == FN - 1) ? 4 : i % 4; };
    // A wave's columns lie in one 128-row weight block when WN divides 128;
    // otherwise (straddle) they may span two, and the weight scale is chosen
    // per weight fragment.
    constexpr bool STRADDLE = (128 % C::WN) != 0;
    static_assert(C::WN <= 128, "a wave's columns span at most two weight blocks");
    v8i fa[C::FM], fb[SLOTS];
    float sa[C::FM];          // activation scales (times the weight scale unless STRADDLE or ROWB)
    // Weight gradient (ROWB): every weight row has its own scale; the scales
    // of weight fragment i's four columns (of this lane) are a float4, read
    // during row i-1 (after its first block's FMAs, which free the slot of
    // row i-2) into slot i % 2.  The next chunk's row 0 goes to slot 0
    // during the last row, so with an odd FN the last row takes slot 2.
    constexpr bool ROWB = MODE == kWgrad;
    static_assert(!ROWB || C::FM >= 2, "the weight scales are read at a row's second block");
    static_assert(!ROWB || BN <= (C::NW - C::SA_WAVES) * 64, "the scale waves must cover every weight row");
    static_assert(!(ROWB && C::CS), "per-row weight scales need every scale slot");
    float4 sbr[3];
    auto sslot = [](int i) { return (i == FN - 1 && (FN - 1) % 2 == 0) ? 2 : i % 2; };
    float sb_lo = 0.f, sb_hi = 0.f;
    int ea[C::FM];              // HWS: this chunk's E8M0 bytes: activation rows (per lane) and
    int ebf[C::FN];             // the weight block of each weight fragment (uniform, SGPRs);
                                // weight gradient: the E8M0 byte of weight row fr of the fragment
    float sbrow[ROWB && HWS ? C::FN : 1];   // weight gradient, hardware scaling: those rows' scales
    const int blk_lo = sb_idx;
    const int blk_hi = (int)((n0 + b_row0 + C::WN - 1) / 128 - n0 / 128);
    auto read_a1 = [&](int stage, int j) {
      const uint8_t* base = smem + stage * C::STAGE + (a_row0 + 16 * j) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      fa[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_b1 = [&](int stage, int i) {
      const uint8_t* base = smem + stage * C::STAGE + C::A_BYTES + (b_row0 + 16 * i) * kKC;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + rd1);
      fb[slot(i)] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_sc = [&](int stage) {
      const uint8_t* st = smem + stage * C::STAGE;
#pragma unroll
      for (int j = 0; j < C::FM; ++j) sa[j] = reinterpret_cast<const float*>(st + C::SA_OFF)[a_row0 + 16 * j + fr];
      if (!ROWB) sb_lo = reinterpret_cast<const float*>(st + C::SB_OFF)[blk_lo];
      if (STRADDLE && !ROWB) sb_hi = reinterpret_cast<const float*>(st + C::SB_OFF)[blk_hi];
      // Weight gradient with hardware scaling: the scaled MFMA takes the
      // first operand's scale per row (lane fr: weight row b_row0 + 16i + fr)
      if constexpr (ROWB && HWS)
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
          sbrow[i] = reinterpret_cast<const float*>(st + C::SB_OFF)[b_row0 + 16 * i + fr];
    };
    auto read_sbr = [&](int stage, int i) {
      sbr[sslot(i)] = *reinterpret_cast<const float4*>(smem + stage * C::STAGE + C::SB_OFF + 4 * (b_row0 + 16 * i + 4 * fg));
    };
    // Scale products of weight fragment i: sa * sb(block of fragment i).
    auto row_scales = [&](int i, float* sc) {
      if (ROWB) {
#pragma unroll
        for (int j = 0; j < C::FM; ++j) sc[j] = sa[j];
        return;
      }
      const bool hi_blk = (int)((n0 + b_row0 + 16 * i) / 128 - n0 / 128) != blk_lo;
      const float sbi = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                            __builtin_bit_cast(int, hi_blk ? sb_hi : sb_lo)));
#pragma unroll
      for (int j = 0; j < C::FM; ++j) sc[j] = sa[j] * sbi;
    };
    // Blocks b = i*FM + j (weight fragment i, activation fragment j).
    constexpr int NBLK = FN * C::FM;
    constexpr int LAST = NBLK - C::FM;   // first block of the last row
    const v4f pz = {0.f, 0.f, 0.f, 0.f};
    v4f pc[2];
    auto mfma = [&](int b) {
      if constexpr (HWS) {
        const int i = b / C::FM, j = b % C::FM;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[slot(i)], fa[j], acc[i][j], 0, 0, 0,
                                                                     ebf[i], 0, ea[j]);
        return pz;
      } else {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[slot(b / C::FM)], fa[b % C::FM], pz,
                                                                0, 0, 0, 0, 0, 0);
      }
    };
    auto fma_block = [&](int b, const v4f& pv, const float* sc) {
      if constexpr (HWS) return;
      v4f& ac = acc[b / C::FM][b % C::FM];
      if (ROWB) {
        const float4 sv = sbr[sslot(b / C::FM)];
        const float sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) ac[r] = __builtin_fmaf(pv[r], sc[b % C::FM] * sw[r], ac[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) ac[r] = __builtin_fmaf(pv[r], sc[b % C::FM], ac[r]);
      }
    };
    // Rows 0 .. FN-2; weight fragment i+2 is read at the start of row i.
    // Returns, in scl, the scale products of row FN-2 (its last block's FMAs
    // run in the last row).
    auto rows = [&](int stage, float* scl) {
      float sc[2][C::FM];
      if (STRADDLE || ROWB) row_scales(0, sc[0]);
      else
#pragma unroll
        for (int j = 0; j < C::FM; ++j) sc[0][j] = sa[j];
      pc[0] = mfma(0);
      if (2 < FN) read_b1(stage, 2);
#pragma unroll
      for (int b = 1; b < LAST; ++b) {
        const int i = b / C::FM;
        pc[b & 1] = mfma(b);
        if (ROWB && !HWS && b % C::FM == 1 && i + 1 < FN) read_sbr(stage, i + 1);
        if (b % C::FM == 0) {
          if (i + 2 < FN) read_b1(stage, i + 2);
          if (STRADDLE || ROWB) row_scales(i, sc[i & 1]);
          else
#pragma unroll
            for (int j = 0; j < C::FM; ++j) sc[i & 1][j] = sa[j];
        }
        fma_block(b - 1, pc[(b - 1) & 1], sc[((b - 1) / C::FM) & 1]);
      }
#pragma unroll
      for (int j = 0; j < C::FM; ++j) scl[j] = sc[(FN - 2) & 1][j];
      // Order: MFMA, [at the start of a row: the weight read], the FMAs of the
      // previous block [and the row's scale products].  With hardware
      // scaling there are no FMAs: MFMAs and the weight reads only.
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (2 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if constexpr (HWS) {
#pragma unroll
        for (int b = 1; b < LAST; ++b) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (b % C::FM == 0 && b / C::FM + 2 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        return;
      }
#pragma unroll
      for (int b = 1; b < LAST; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ROWB && b % C::FM == 1 && b / C::FM + 1 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (b % C::FM == 0 && b / C::FM + 2 < FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (ROWB) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        else if (STRADDLE && b % C::FM == 0) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        else __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    };
    // The last row, split around the synchronisation: its first two MFMAs
    // (which need only this chunk's fragments) are issued before the wave
    // waits at the barrier, so the matrix core has work queued while the
    // waves meet; the other two right after it, before anything else.  Each
    // MFMA frees its activation fragment, which is refilled with the next
    // chunk's (from stage nstage); weight fragments 0 and 1 and the next
    // chunk's scales follow, and `mid` (the next DMA) comes last.  The FMAs
    // keep this chunk's scales.
    auto last_row = [&](int nstage, const float* scp, auto&& sync, auto&& mid) {
      float sc[C::FM];
      if (STRADDLE || ROWB) row_scales(FN - 1, sc);
      else
#pragma unroll
        for (int j = 0; j < C::FM; ++j) sc[j] = sa[j];
      pc[LAST & 1] = mfma(LAST);
      fma_block(LAST - 1, pc[(LAST - 1) & 1], scp);
      pc[(LAST + 1) & 1] = mfma(LAST + 1);
      fma_block(LAST, pc[LAST & 1], sc);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (!HWS) __builtin_amdgcn_sched_group_barrier(0x002, (STRADDLE || ROWB) ? 8 : 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (!HWS) __builtin_amdgcn_sched_group_barrier(0x002, ROWB ? 8 : 4, 0);
      __builtin_amdgcn_sched_barrier(0);
      sync();
      __builtin_amdgcn_sched_barrier(0);
      // Two MFMAs in flight: blocks LAST+2 and LAST+3 use pc slots 0 and 1,
      // which the FMAs of blocks LAST and LAST+1 have consumed (program
      // order), so pc3 is a third result register.
      const v4f p2 = mfma(LAST + 2);
      __builtin_amdgcn_sched_barrier(0);
      read_a1(nstage, 0);
      read_b1(nstage, 0);
      __builtin_amdgcn_sched_barrier(0);
      read_sc(nstage);
      if (ROWB && !HWS) read_sbr(nstage, 0);
      __builtin_amdgcn_sched_barrier(0);
      const v4f p3 = mfma(LAST + 3);
      __builtin_amdgcn_sched_barrier(0);
      read_a1(nstage, 1);
      read_b1(nstage, 1);
      read_a1(nstage, 2);
      fma_block(LAST + 1, pc[(LAST + 1) & 1], sc);
      fma_block(LAST + 2, p2, sc);
      __builtin_amdgcn_sched_barrier(0);
      read_a1(nstage, 3);
      fma_block(LAST + 3, p3, sc);
      __builtin_amdgcn_sched_barrier(0);
      mid();
    };
    // Without straddling, every row uses sa * sb: multiply once per chunk.
    auto chunk_scales = [&] {
      if constexpr (HWS) {
#pragma unroll
        for (int j = 0; j < C::FM; ++j) ea[j] = e8m0_of(sa[j]);
        if constexpr (ROWB) {
#pragma unroll
          for (int i = 0; i < C::FN; ++i) ebf[i] = e8m0_of(sbrow[i]);
          return;
        }
        const int eb_lo = __builtin_amdgcn_readfirstlane(e8m0_of(sb_lo));
        const int eb_hi = STRADDLE ? __builtin_amdgcn_readfirstlane(e8m0_of(sb_hi)) : eb_lo;
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
          ebf[i] = ((int)((n0 + b_row0 + 16 * i) / 128 - n0 / 128) != blk_lo) ? eb_hi : eb_lo;
        return;
      }
      if (!STRADDLE && !ROWB)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) sa[j] = sa[j] * sb_lo;
    };
    // Prologue: chunks 0 .. S-1 on their way to stages 0 .. S-1; once chunk
    // 0 has landed in every wave's share, its first fragments are read.
    constexpr int S = C::S;
#pragma unroll
    for (int c = 0; c < S; ++c) issue(c, c);
    // chunks 1 .. S-1 may still be in flight
    wait_vm_lgkm0<(S - 1) * DPC>();
    __builtin_amdgcn_s_barrier();
    // A wave whose rows all lie past the tile's valid rows (a masked expert's
    // count, a ragged last tile) has no MFMA work.  It still issues its share
    // of every chunk's DMA and meets every barrier (the same sequence as a
    // computing wave: wait, barrier, next DMA), but reads no fragments.  Its
    // SIMD then runs the other wave's MFMAs alone.  The choice is per wave and
    // made once, so the computing loop below is unchanged.  (Not in the
    // weight gradient, whose registers are all taken, and which is dense.)
    // (An idle wave goes on to the epilogue, whose barriers it meets too.)
    if (MODE != kWgrad && m0 + a_row0 >= m_valid) {
      auto idle_step = [&](int kb, int stage) {
        wait_vm_lgkm0<(S - 2) * DPC>();
        __builtin_amdgcn_s_barrier();
        issue(kb + S, stage);
      };
      int kb = 0;
      for (; kb + S - 1 < KT; kb += S) {
#pragma unroll
        for (int st = 0; st < S; ++st) idle_step(kb + st, st);
      }
#pragma unroll
      for (int st = 0; st < S - 1; ++st)
        if (kb + st < KT) idle_step(kb + st, st);
    } else {
    read_a1(0, 0);
    read_b1(0, 0);
    read_sc(0);
    if (ROWB && !HWS) read_sbr(0, 0);
#pragma unroll
    for (int j = 1; j < C::FM; ++j) read_a1(0, j);
    read_b1(0, 1);
    // Step kb (chunk kb in stage `stage`): rows 0 .. FN-2, then the last row,
    // inside which the wave waits for chunk kb+1's DMA (chunks kb+2 .. kb+S-1
    // may still be in flight) and meets the other waves (every wave then
    // holds all of chunk kb in registers, so its stage is free), reads chunk
    // kb+1's first fragments and starts chunk kb+S's DMA into the freed
    // stage.
    auto step = [&](int kb, int stage) {
      __builtin_amdgcn_sched_barrier(0);
      chunk_scales();
      if constexpr (HWS) __builtin_amdgcn_sched_barrier(0);   // the chunk's E8M0 bytes first
      float scp[C::FM];
      rows(stage, scp);
      __builtin_amdgcn_sched_barrier(0);
      last_row(stage + 1 == S ? 0 : stage + 1, scp,
               [&] {
                 wait_vm_lgkm0<(S - 2) * DPC>();
                 __builtin_amdgcn_s_barrier();
               },
               [&] { issue(kb + S, stage); });
    };
    int kb = 0;
    for (; kb + S - 1 < KT; kb += S) {
#pragma unroll
      for (int st = 0; st < S; ++st) step(kb + st, st);
    }
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (kb + st < KT) step(kb + st, st);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // every DMA of this wave has landed in LDS

  if constexpr (MODE == kSplitK) {
    // The tile's FP32 partial over this split's chunks, as a BM x BN block
    // of the workspace (p.d): the rows inside the matrix (the reduction reads
    // no others); columns past it hold zeros.
    float* part = reinterpret_cast<float*>(p.d) + ((int64_t)split_tile * p.G + split) * (BM * BN);
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int row = a_row0 + 16 * j + fr;
      if (m0 + row < m_valid) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
          const v4f& v = acc[i][j];
          *reinterpret_cast<float4*>(part + row * BN + b_row0 + 16 * i + 4 * fg) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    return;
  }

  // ---- epilogue: through LDS, then whole rows -----------------------------
  // Lane (fr, fg) holds D[m][n .. n+3] of each fragment: stored from there,
  // every row segment is 32 (BF16) or 64 (FP32) bytes, a part of a cache
  // line whose other parts come from other instructions and other tiles.
  // Staged in the free LDS, the tile leaves in 16-byte pieces of whole rows
  // instead (interleaved A/B, outputs bit-identical: masked MoE 32 x 256 x
  // 7168 x 2048 157 -> 144 us, decode 128 x 24576 x 1536 14.8 -> 14.3 us).
  // A tile whose output does not fit in LDS at once goes in passes of JP
  // fragment rows of every wave.
  constexpr int ES = OUT_F32 ? 4 : 2;                 // bytes per output
  constexpr int RSTR = BN * ES + 16;                  // LDS row stride (padded)
  constexpr int JP = epi_frags_per_pass(C::FM, C::WGM * 16 * RSTR, C::LDS_BYTES);
  constexpr int PR = C::WGM * 16 * JP;                // LDS rows per pass
  constexpr int CPR = BN * ES / 16;                   // 16-byte pieces per row
  static_assert(PR * RSTR <= C::LDS_BYTES, "a pass fits in LDS");
  const int64_t rows = min<int64_t>(m_valid - m0, BM);
  const int64_t cols = min<int64_t>(N - n0, BN);      // a multiple of 16 (N % 16 == 0)
#pragma unroll
  for (int j0 = 0; j0 < C::FM; j0 += JP) {
    lds_barrier();   // the stages (the previous pass) are free
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const int col = b_row0 + 16 * i + 4 * fg;
#pragma unroll
      for (int jj = 0; jj < JP; ++jj) {
        const v4f& v = acc[i][j0 + jj];
        uint8_t* dst = smem + (wm * 16 * JP + 16 * jj + fr) * RSTR + col * ES;
        if (OUT_F32) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        else *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
      }
    }
    lds_barrier();
    for (int q = threadIdx.x; q < PR * CPR; q += C::THREADS) {
      const int lrow = q / CPR, piece = q - lrow * CPR;
      const int w = lrow / (16 * JP), r = lrow - w * (16 * JP);
      const int row = w * C::WM + 16 * (j0 + r / 16) + r % 16;   // row in the tile
      if (row < rows && piece * 16 < cols * ES) {
        uint4 v = *reinterpret_cast<const uint4*>(smem + lrow * RSTR + piece * 16);
        uint4* dp = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.d) + ((d_row0 + m0 + row) * N + n0) * ES +
                                             piece * 16);
        if (MODE == kWgrad && p.accumulate) {
          const float4 o = *reinterpret_cast<const float4*>(dp);
          const float4 n = *reinterpret_cast<const float4*>(&v);
          const float4 s = make_float4(o.x + n.x, o.y + n.y, o.z + n.z, o.w + n.w);
          v = *reinterpret_cast<const uint4*>(&s);
        }
        *dp = v;
      }
    }
  }
#endif
}

template <class C, int MODE>
hipError_t launch_cfg(const GemmProblem& pr, hipStream_t stream) {
  GemmArgs a;
  a.a = pr.a; a.sa = pr.sa; a.b = pr.b; a.sb = pr.sb; a.d = pr.d; a.groups = pr.groups;
  a.M = pr.M; a.N = pr.N; a.K = pr.K; a.G = pr.G;
  a.tiles_m = (int32_t)((pr.M + C::BM - 1) / C::BM);
  // Contiguous: every group may end in a partial tile, so at most Mt/BM + G
  // tiles exist (the kernel counts the real ones from the offsets).
  if (MODE == kContiguous) a.tiles_m = (int32_t)(pr.M / C::BM + pr.G);
  a.tiles_n = (int32_t)((pr.N + C::BN - 1) / C::BN);
  // Tile rows walked together: an XCD's share of the 256-row tiles then
  // covers fewer activation rows and more weight rows (4096x2112x7168 on
  // 256x160 tiles: 4 x 7 instead of 8 x 3.5 tiles, 15.3 instead of 19.3 MB
  // of operands per L2; 1-3 % faster on the dense and weight-gradient
  // shapes, interleaved A/B); the smaller tiles keep 8 (4 made the
  // contiguous MoE shape on 128-row tiles 10 % slower).
  a.group_m = C::BM >= 256 ? 4 : 8;
  a.accumulate = pr.accumulate ? 1 : 0;
  const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * (MODE == kMasked ? pr.G : 1);
  if (blocks == 0) return hipSuccess;
  if constexpr (MODE == kWgrad) {   // FP32 out
    if (pr.hw_scale)
      hipLaunchKernelGGL((k_gemm<C, MODE, true, true>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm<C, MODE, true, false>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
  } else if (pr.hw_scale) {
    if (pr.out_f32)
      hipLaunchKernelGGL((k_gemm<C, MODE, true, true>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm<C, MODE, false, true>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
  } else {
    if (pr.out_f32)
      hipLaunchKernelGGL((k_gemm<C, MODE, true, false>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_gemm<C, MODE, false, false>), dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

// Tile choice.  Workgroups go round-robin to the 8 XCDs of 32 CUs each; a
// shape takes ceil(tiles per XCD / workgroup slots per XCD) rounds, each
// costing about the time of one tile.  Relative tile costs (measured on
// dense 8192x4096x7168): 256x256 = 1, 256x160 = 0.7, 128x128 at two
// workgroups per CU = 0.52; 192x192 = 0.65 (against 256x160 on
// 4096x2112x7168).  The 256x256 tile loads the fewest operand bytes per MFMA
// and wins whenever it fills the chip.
template <class C>
double est_rounds(int64_t tiles, double cost) {
  const int64_t per_xcd = (tiles + 7) / 8;
  const int64_t slots = 32 * C::WG_PER_CU;
  return (double)((per_xcd + slots - 1) / slots) * cost;
}

// Tile configurations the dispatcher chooses from.
enum TileChoice { kStream, kStream64, kSmall, kLarge, kMid, kT192, kPP192, kMaskedT, kWgradMid };

template <int MODE>
TileChoice choose(const GemmProblem& p) {
  if constexpr (MODE == kMasked) {
    // Memory-bound decode shapes: the masked tile, once there are enough
    // tiles to fill the GPU.
    const int64_t masked_tiles = ((p.M * p.G + MaskedTile::BM - 1) / MaskedTile::BM) *
                                 ((p.N + MaskedTile::BN - 1) / MaskedTile::BN);
    return masked_tiles >= 256 ? kMaskedT : kSmall;
  } else {
    // Few rows (decode): the weights stream from HBM once; a deep pipeline
    // over many small tiles keeps enough bytes in flight.  64x64 tiles up to
    // one and a half per CU, else 128x96.  Up to 512 rows the larger tiles
    // leave most CUs idle while 64x64 tiles fill them: up to two per CU
    // (interleaved A/B against the 128x128 tile the cost model picks,
    // outputs bit-identical: 256x2112x7168 39.8 -> 20.4 us, 256x4096x7168
    // 52.9 -> 22.9 us, 512x2112x7168 40.6 -> 24.2 us, 200x4096x4096 24.0 ->
    // 14.6 us, 512x4096x2048 (512 tiles) 15.6 -> 13.3 us).
    if constexpr (MODE == kDense) {
      const int64_t t64 = ((p.M + 63) / 64) * ((p.N + 63) / 64);
      if (p.M <= 128) return t64 <= 384 ? kStream64 : kStream;
      if (p.M <= 512 && t64 <= 512) return kStream64;
    }
    // Row tiles: dense exact; contiguous counts on average half a partial
    // tile per group.
    auto mtiles = [&](int64_t bm) {
      return MODE == kContiguous ? p.M / bm + (p.G + 1) / 2 : (p.M + bm - 1) / bm;
    };
    const double t_large = est_rounds<LargeTile>(mtiles(256) * ((p.N + 255) / 256), 1.0);
    const double t_mid = est_rounds<MidTile>(mtiles(256) * ((p.N + 159) / 160), 0.7);
    const double t_small = est_rounds<SmallTile>(mtiles(128) * ((p.N + 127) / 128), 0.52);
    if constexpr (MODE == kWgrad) {
      // per-row weight scales are read in the 256-wide tiles' loop only
      return t_large <= t_mid ? kLarge : kWgradMid;
    } else {
      // The 192x192 tile runs the ping-pong loop (gemm_pp.hip) whenever the
      // rows of sA are a multiple of 4 (it moves them 4 rows per lane; always
      // so for the contiguous layout, whose rows are a multiple of 128): it
      // costs 0.56 of a 256x256 tile (4096x2112x7168 in 60 against about 70
      // us for the 0.65 of the 12-wave 192x192 tile).  On 8x8192x4096x7168
      // contiguous it took 269 us against 289 us on 128x128 tiles.
      const bool pp = MODE == kContiguous || p.M % 4 == 0;
      const double t_192 = est_rounds<Tile192>(mtiles(192) * ((p.N + 191) / 192), pp ? 0.56 : 0.65);
      if (t_large <= t_mid && t_large <= t_192 && t_large <= t_small) return kLarge;
      if (t_192 <= t_mid && t_192 < t_small) return pp ? kPP192 : kT192;
      return t_mid <= t_small ? kMid : kSmall;
    }
  }
}

// The tiles choose() can return for each layout; only those are
// instantiated.
constexpr bool possible(int mode, TileChoice c) {
  switch (mode) {
    case kDense: return c == kStream || c == kStream64 || c == kSmall || c == kLarge || c == kMid || c == kT192 || c == kPP192;
    case kContiguous: return c == kSmall || c == kLarge || c == kMid || c == kPP192;
    case kMasked: return c == kMaskedT || c == kSmall;
    default: return c == kLarge || c == kWgradMid;
  }
}

template <class C, int MODE, TileChoice T>
hipError_t launch_if(const GemmProblem& p, hipStream_t stream) {
  if constexpr (possible(MODE, T)) return launch_cfg<C, MODE>(p, stream);
  else return hipErrorInvalidValue;
}

template <int MODE>
hipError_t dispatch(const GemmProblem& p, hipStream_t stream) {
  switch (choose<MODE>(p)) {
    case kStream: return launch_if<StreamTile, MODE, kStream>(p, stream);
    case kStream64: return launch_if<Stream64Tile, MODE, kStream64>(p, stream);
    case kSmall: return launch_if<SmallTile, MODE, kSmall>(p, stream);
    case kLarge: return launch_if<LargeTile, MODE, kLarge>(p, stream);
    case kT192: return launch_if<Tile192, MODE, kT192>(p, stream);
    case kPP192: return launch_gemm_pp192(p, stream);
    case kMaskedT: return launch_if<MaskedTile, MODE, kMaskedT>(p, stream);
    case kWgradMid: return launch_if<WgradMidTile, MODE, kWgradMid>(p, stream);
    default: return launch_if<MidTile, MODE, kMid>(p, stream);
  }
}

template <int MODE>
void tile_of(const GemmProblem& p, int32_t& bm, int32_t& bn, int32_t& pp) {
  pp = 0;
  switch (choose<MODE>(p)) {
    case kStream: bm = StreamTile::BM; bn = StreamTile::BN; break;
    case kStream64: bm = Stream64Tile::BM; bn = Stream64Tile::BN; break;
    case kSmall: bm = SmallTile::BM; bn = SmallTile::BN; break;
    case kLarge: bm = LargeTile::BM; bn = LargeTile::BN; break;
    case kT192: bm = Tile192::BM; bn = Tile192::BN; break;
    case kPP192: bm = 192; bn = 192; pp = 1; break;
    case kMaskedT: bm = MaskedTile::BM; bn = MaskedTile::BN; break;
    case kWgradMid: bm = WgradMidTile::BM; bn = WgradMidTile::BN; break;
    default: bm = MidTile::BM; bn = MidTile::BN; break;
  }
}

// ---- split K --------------------------------------------------------------
// D[m][n] = sum over the splits s = 0, 1, .. of partial s of the tile holding
// (m, n), added in that order (four outputs of one row per lane).
// Split tiles: 64x64 for at most 128 rows, 128x96 above (interleaved A/B on
// rotating weight sets, graph-timed: 64x2112x7168 12.9 -> 10.9 us,
// 128x2112x7168 16.7 -> 13.6 us, 32x4096x7168 13.1 -> 12.1 us; but
// 256x2112x7168 18.0 -> 20.2 us).
template <class T>
int64_t split_tiles(int64_t M, int64_t N) {
  return ((M + T::BM - 1) / T::BM) * ((N + T::BN - 1) / T::BN);
}
bool split_on_64(int64_t M) { return M <= 128; }

template <class T, bool OUT_F32>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, void* __restrict__ d, int64_t M,
                                                       int64_t N, int32_t S, int32_t tiles_m) {
  constexpr int BM = T::BM, BN = T::BN;
  static_assert(BN % 4 == 0, "a lane's four outputs lie in one tile");
  const int64_t n4 = N / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * n4) return;
  const int64_t m = idx / n4, c = (idx - m * n4) * 4;
  const int64_t tile = (c / BN) * tiles_m + m / BM;
  const float* pp = ws + tile * S * (BM * BN) + (m % BM) * BN + c % BN;
  float4 v = *reinterpret_cast<const float4*>(pp);
  // eight partials loaded at a time (all in flight), then added in order
  constexpr int U = 8;
  for (int s = 1; s < S; s += U) {
    float4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s + u < S) w[u] = *reinterpret_cast<const float4*>(pp + (int64_t)(s + u) * (BM * BN));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s + u < S) v = make_float4(v.x + w[u].x, v.y + w[u].y, v.z + w[u].z, v.w + w[u].w);
  }
  if (OUT_F32) *reinterpret_cast<float4*>(reinterpret_cast<float*>(d) + m * N + c) = v;
  else *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(d) + m * N + c) = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
}

template <class T>
hipError_t launch_split(const GemmProblem& pr, float* ws, int32_t S, hipStream_t stream) {
  GemmArgs a;
  a.a = pr.a; a.sa = pr.sa; a.b = pr.b; a.sb = pr.sb; a.d = ws; a.groups = nullptr;
  a.M = pr.M; a.N = pr.N; a.K = pr.K; a.G = S;
  a.tiles_m = (int32_t)((pr.M + T::BM - 1) / T::BM);
  a.tiles_n = (int32_t)((pr.N + T::BN - 1) / T::BN);
  a.group_m = 8;
  a.accumulate = 0;
  const dim3 grid((unsigned)((int64_t)a.tiles_m * a.tiles_n * S)), block(T::THREADS);
  if (pr.hw_scale) hipLaunchKernelGGL((k_gemm<T, kSplitK, true, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((k_gemm<T, kSplitK, true, false>), grid, block, 0, stream, a);
  if (hipError_t e = hipGetLastError()) return e;
  const int64_t outs = pr.M * (pr.N / 4);
  const dim3 rgrid((unsigned)((outs + 255) / 256)), rblock(256);
  if (pr.out_f32)
    hipLaunchKernelGGL((k_splitk_reduce<T, true>), rgrid, rblock, 0, stream, ws, pr.d, pr.M, pr.N, S, a.tiles_m);
  else
    hipLaunchKernelGGL((k_splitk_reduce<T, false>), rgrid, rblock, 0, stream, ws, pr.d, pr.M, pr.N, S, a.tiles_m);
  return hipGetLastError();
}

}  // namespace

// Splits: as many as fill one round of the 256 CUs with the split tiles (one
// workgroup per CU), with at least two chunks each and at most 32; only for
// K of at least 32 chunks, where the split saves more than the second launch
// and the partials' round trip cost (measured on 128x96 split tiles: 64 x
// 2112 x 7168 28.4 -> 15.6 us with 11 splits, 256 x 2112 x 7168 50.4 -> 17.7
// us with 5, but 128 x 7168 x 2048, 16 chunks, 13.8 -> 16.8 us with 3).
int32_t splitk_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = split_on_64(M) ? split_tiles<Stream64Tile>(M, N) : split_tiles<StreamTile>(M, N);
  const int64_t kt = K / kKC;
  if (tiles <= 0 || kt < 32) return 1;
  int64_t s = 256 / tiles;
  s = s > kt / 2 ? kt / 2 : s;
  s = s > 32 ? 32 : s;
  return s >= 2 ? (int32_t)s : 1;
}

int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int32_t s = splitk_splits(M, N, K);
  if (s < 2) return 0;
  const int64_t tile_bytes = (split_on_64(M) ? Stream64Tile::BM * Stream64Tile::BN : StreamTile::BM * StreamTile::BN) *
                             (int64_t)sizeof(float);
  const int64_t tiles = split_on_64(M) ? split_tiles<Stream64Tile>(M, N) : split_tiles<StreamTile>(M, N);
  return tiles * s * tile_bytes;
}

hipError_t launch_gemm_splitk(const GemmProblem& pr, float* ws, hipStream_t stream) {
  const int32_t S = splitk_splits(pr.M, pr.N, pr.K);
  if (S < 2) return launch_gemm(pr, stream);
  return split_on_64(pr.M) ? launch_split<Stream64Tile>(pr, ws, S, stream) : launch_split<StreamTile>(pr, ws, S, stream);
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream) {
  switch (p.mode) {
    case kDense: return dispatch<kDense>(p, stream);
    case kContiguous: return dispatch<kContiguous>(p, stream);
    case kWgrad: return dispatch<kWgrad>(p, stream);
    default: return dispatch<kMasked>(p, stream);
  }
}

void gemm_tile(const GemmProblem& p, int32_t& bm, int32_t& bn, int32_t& pp) {
  switch (p.mode) {
    case kDense: tile_of<kDense>(p, bm, bn, pp); break;
    case kContiguous: tile_of<kContiguous>(p, bm, bn, pp); break;
    case kWgrad: tile_of<kWgrad>(p, bm, bn, pp); break;
    default: tile_of<kMasked>(p, bm, bn, pp); break;
  }
}

}  // namespace fp8bs
