// Device helpers shared by the block-scaled FP8 GEMM kernels for gfx950:
// operand LDS layout, buffer resources and the memory -> LDS DMA, the
// grouped layouts' tile lookup, and the workgroup -> tile mapping.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace fp8bs {
namespace {

constexpr int kKC = 128;  // K chunk = promotion interval = MFMA K

// LDS layout of an operand chunk: rows of 128 bytes (one K chunk), row-major,
// with the 16-byte segments of row r XOR-swizzled: logical segment s is
// stored at segment s ^ swz(r), swz(r) = (r >> 1) & 7.  An MFMA fragment of
// 16 rows has lane l = fr + 16*fg hold row fr's logical segments fg and
// fg + 4 (the order of K inside a fragment is free as long as both operands
// use the same one).  Measured on gfx950 with 8 waves per CU, this pairing
// reads at 227 of 256 B/clk per CU; the pairing (2fg, 2fg+1) stays below 145
// with any of the swizzles tried, and unswizzled rows reach 81.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Buffer resource word 3 for raw (untyped) dword access on gfx9-class parts.
constexpr int kRsrcWord3 = 0x00020000;

typedef int v4i __attribute__((ext_vector_type(4)));

// A raw buffer resource (stride 0) over [base, base + bytes), built from
// readfirstlane'd fields so it lives in SGPRs.
__device__ __forceinline__ v4i make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const int64_t nb = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : bytes);
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)nb);
  r.w = kRsrcWord3;
  return r;
}

// Memory -> LDS DMA of 16 (4) bytes per lane: lane l's data lands at LDS byte
// address lds + 16*l (4*l); the source is rsrc.base + voff + soff, and the
// hardware range check on voff against the descriptor's size turns
// out-of-range lanes into zeros without a memory access.
//
// Issued from inline asm on purpose: the compiler, seeing an LDS DMA, would
// make every later LDS read wait for all outstanding DMA (it cannot tell the
// two LDS stages apart), which would serialise the pipeline.  Hidden in asm,
// the DMA is ordered by the "memory" clobber and waited for explicitly with
// s_waitcnt at the top of each step.  The asm sets M0 (the LDS destination);
// nothing else in these kernels uses M0.  There are no output registers.
// The scalar operands go through readfirstlane (free for values already in
// SGPRs) so the "s" constraints always get SGPRs.
__device__ __forceinline__ v4i uniform(v4i r) {
  return v4i{__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
             __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform(rsrc)),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}
// s_waitcnt vmcnt(N) lgkmcnt(0): vector memory loads complete in issue order,
// so all but the N most recent have landed.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// s_waitcnt lgkmcnt(0) (this wave's LDS reads and writes are done), then
// s_barrier: what any wave wrote to LDS before it is visible to every wave
// after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p);
}

// Valid rows of a masked group: the device-side count clamped to [0, cap].
__device__ __forceinline__ int64_t masked_count(int32_t c, int64_t cap) {
  return c < 0 ? 0 : (c > cap ? cap : (int64_t)c);
}
// Rows [lo, hi) of contiguous group g, clamped into [0, Mt] so that any
// offsets array keeps every access inside the buffers.
__device__ __forceinline__ void group_rows(const int32_t* offs, int g, int64_t mt, int64_t& lo, int64_t& hi) {
  lo = offs[g];
  hi = offs[g + 1];
  lo = lo < 0 ? 0 : (lo > mt ? mt : lo);
  hi = hi < lo ? lo : (hi > mt ? mt : hi);
}

// Per-group tile counts c(g) of the masked layout, one group per lane and
// 64 groups per pass: one vector load (or two) per pass instead of a
// dependent scalar load per group (walking 32 experts that way took a
// median 6.6 us per workgroup before its first DMA).  Every lane of the
// wave must be active.  group_total returns the sum over all G groups;
// group_find the group g holding unit x (units counted in group order, x
// below the total) and, in `first`, the number of units before g (G if x is
// not below the total).
template <class F>
__device__ __forceinline__ int group_total(int G, F c) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int v = g0 + lane < G ? c(g0 + lane) : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    total += v;
  }
  return total;
}
template <class F>
__device__ __forceinline__ int group_find(int G, F c, int x, int& first) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int v = g0 + lane < G ? c(g0 + lane) : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > x);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      first = base + __builtin_amdgcn_readlane(incl - v, l);
      return g0 + l;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  first = base;
  return G;
}

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* d;
  const int32_t* groups;
  int64_t M, N, K;
  int32_t G;
  int32_t tiles_m, tiles_n;   // dense: tile grid; grouped: per-group / worst-case bound
  int32_t group_m;
  int32_t accumulate;         // kWgrad: add to D
};

// Operand bases and row ranges of the tile a workgroup computes.
struct Tile {
  const uint8_t* a_base;
  const float* sa_base;
  const uint8_t* b_base;
  const float* sb_base;
  int64_t m_alloc;     // rows that exist in memory (loads are clamped to them)
  int64_t m_valid;     // rows that are computed and stored
  int64_t sa_stride;   // distance between consecutive K chunks in sA
  int64_t d_row0;      // first output row of this group's block of D
  int64_t m0, n0;      // first row and column of the tile
};

// Workgroup -> tile.  Returns false for workgroups without work.
template <int BM, int BN, int MODE>
__device__ __forceinline__ bool map_tile(const GemmArgs& p, int64_t K, int KT, int64_t NB, Tile& t) {
  // ---- tile -> (group, rows, columns) ------------------------------------
  // The grouped layouts launch a grid sized for the worst case; the tiles
  // that exist are counted here from the device-side group sizes, numbered
  // 0 .. total-1, and spread evenly over the XCDs.
  t.a_base = p.a;
  t.sa_base = p.sa;
  t.b_base = p.b;
  t.sb_base = p.sb;
  t.m_alloc = p.M;
  t.m_valid = p.M;
  t.sa_stride = p.M;
  t.d_row0 = 0;
  if constexpr (MODE == kMasked) {
    // Tiles in group order; within a group, m fastest.
    auto tiles_of = [&](int gg) { return (int)((masked_count(p.groups[gg], p.M) + BM - 1) / BM) * p.tiles_n; };
    int pid, g, first = 0;
    if (p.G <= 64) {
      // One load and one scan serve both the total and the search.
      const int lane = threadIdx.x & 63;
      const int v = lane < p.G ? tiles_of(lane) : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      pid = xcd_remap((int)blockIdx.x, __builtin_amdgcn_readlane(incl, 63));
      if (pid < 0) return false;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > pid);
      if (!hit) return false;
      g = __builtin_ctzll(hit);
      first = __builtin_amdgcn_readlane(incl - v, g);
    } else {
      pid = xcd_remap((int)blockIdx.x, group_total(p.G, tiles_of));
      if (pid < 0) return false;
      g = group_find(p.G, tiles_of, pid, first);
      if (g >= p.G) return false;
    }
    pid -= first;
    const int64_t rows = masked_count(p.groups[g], p.M);
    const int tcnt = (int)((rows + BM - 1) / BM);
    const int tn = pid / tcnt, tm = pid - tn * tcnt;
    t.m0 = (int64_t)tm * BM;
    t.n0 = (int64_t)tn * BN;
    t.m_valid = rows;
    t.a_base += (int64_t)g * p.M * K;
    t.sa_base += (int64_t)g * KT * p.M;
    t.b_base += (int64_t)g * p.N * K;
    t.sb_base += (int64_t)g * NB * KT;
    t.d_row0 = (int64_t)g * p.M;
  } else {
    // Dense: the grid is exact.  Contiguous: tile t of group g has index
    // (tiles of the groups before g) + t (group boundaries are multiples of
    // 128 rows, so a tile never spans two groups).
    // (Contiguous layouts have few groups -- one per expert of the GPU -- and
    // walk them in order; the lane-parallel lookup measured 4 % slower on 8
    // groups.)
    int tiles_m = p.tiles_m;
    if (MODE == kContiguous) {
      tiles_m = 0;
      for (int gg = 0; gg < p.G; ++gg) {
        int64_t lo, hi;
        group_rows(p.groups, gg, p.M, lo, hi);
        tiles_m += (int)((hi - lo + BM - 1) / BM);
      }
    }
    const int pid = xcd_remap((int)blockIdx.x, tiles_m * p.tiles_n);
    if (pid < 0) return false;
    // Walk the tiles in groups of group_m tile rows, column by column;
    // contiguous: within each group's own row tiles, so that the tiles of a
    // walk group share one expert's weight panels (8 x 8192 x 4096 x 7168 on
    // 192x192 tiles: 738 -> 587 MB fetched per call, same time; walk groups
    // spanning two experts had needed both experts' panels).
    int pidg = pid, rows_g = tiles_m, g = 0;
    int64_t lo = 0, hi = p.M;
    if (MODE == kContiguous) {
      for (; g < p.G; ++g) {
        group_rows(p.groups, g, p.M, lo, hi);
        rows_g = (int)((hi - lo + BM - 1) / BM);
        if (pidg < rows_g * p.tiles_n) break;
        pidg -= rows_g * p.tiles_n;
      }
      if (g >= p.G) return false;
    }
    const int width = p.group_m * p.tiles_n;
    const int grp = pidg / width;
    const int first_m = grp * p.group_m;
    const int gsz = min(rows_g - first_m, p.group_m);
    const int r = pidg - grp * width;
    const int tm = first_m + r % gsz;
    const int tn = r / gsz;
    t.n0 = (int64_t)tn * BN;
    t.m0 = (int64_t)tm * BM;
    if (MODE == kContiguous) {
      t.m0 = lo + (int64_t)tm * BM;
      t.m_valid = hi;
      t.b_base += (int64_t)g * p.N * K;
      t.sb_base += (int64_t)g * NB * KT;
    }
  }

  return true;
}


// E8M0 exponent byte of a power-of-two scale 2^e, -127 <= e <= 127 (byte
// e + 127; 2^-127 is an FP32 subnormal).  Any other value gives 0xFF, the
// E8M0 NaN, so every output that depends on it comes out NaN.
__device__ __forceinline__ int e8m0_of(float s) {
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  const uint32_t e = u >> 23;   // sign bit included: negative scales are invalid
  const bool normal = (u & 0x7FFFFFu) == 0 && e >= 1 && e <= 254;
  return normal ? (int)e : (u == 0x00400000u ? 0 : 0xFF);
}

}  // namespace
}  // namespace fp8bs
