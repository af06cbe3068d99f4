// Weight-gradient kernel with a stationary operand band (bf16, gfx950).
//
// Product: C[g] (M x N) = P_g^T Q_g, where P_g [n_g x M] and Q_g [n_g x N] are
// the rows of group (expert) g in row-contiguous storage: the contraction runs
// over the expert's rows, n_g of them.  At an average of a few hundred rows per
// expert the output (all of C, bf16) is far larger than the operands.
//
// Work unit: (expert g, band of columns of one operand: of Q when the band is
// on the output's column side, of P when on its row side).  The band goes into
// LDS by DMA at the start of the unit, and the unit walks the 128-wide tiles of
// the output's other side, streaming the other operand in 64-row slices
// through a DMA ring: a tile costs 128 x n_g x 2 bytes of operand reads.  Compute waves read the fragments of both operands from LDS.  Two unit
// shapes share one launch and one LDS layout (a 96 KB band region, the ring,
// the epilogue staging: 160 KB; BandCfg):
//   wide:   experts of 1..192 rows, a 256-column band, 128 x 256 output tiles
//           (each streamed slice feeds twice the outputs, so the per-slice
//           costs -- a barrier, a DMA wait -- weigh half as much);
//   narrow: experts of 193..384 rows, a 128-column band, 128 x 128 tiles.
//
// Waits.  Vector memory operations of a wave complete in issue order, so the
// wait for a slice allows exactly the operations issued after that slice's DMA
// to stay outstanding: a load wave counts what it issues and records the count
// after each slice.
//
// Schedule.  One workgroup per CU: two load waves and four or eight compute
// waves over a grid of the tile (BandShape).  The units are numbered expert-major (the bands of
// expert g follow those of g - 1; an expert has a wide unit per 256 columns or
// a narrow one per 128); each XCD owns one contiguous run of that list, split
// by estimated cost, and its workgroups stride through it, so the workgroups
// of an XCD hold neighbouring bands of one expert; each unit walks its tiles
// from its band index on, so neighbours stream different tiles at any time.
// Experts with no rows or more than 384 rows have no units here (the caller
// zero-fills the first and runs the DMA ring on the second).
//
// Epilogue: each compute wave writes its sub-tile as bf16, 32 x 64 at a time,
// into its own 4 KB staging area (LDS operations of one wave execute in order,
// so no barrier is needed) and stores it back as 128-byte row segments,
// non-temporal.
#pragma once

#include "gemm_mfma.hpp"

namespace moe {

// Issue one 64-row slice of an MC operand planned by DmaPlan::plan_mc (the
// same chunk positions as DmaPlan::issue)
template <class Plan, int NDMA, int NW>
__device__ __forceinline__ void issue_slice_asm(const Plan& p, const void* base, uint32_t bytes, uint32_t soff,
                                                uint32_t lds, int wave) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    dma_b128(base, bytes, p.off[j], soff, lds + (uint32_t)((wave + j * NW) * 64 * 16));
}

// LDS layout and wave roles, common to both unit shapes.  With the band on
// the output's row side (QBAND = false) eight compute waves (two per SIMD)
// and a 2-stage ring: the down-projection gradient at DeepSeek-V3's shape
// 1.92 -> 1.81 ms, where the gate/up one (band on the column side) went from
// 3.66 to 3.75 ms and keeps four compute waves and three stages.
template <bool QBAND>
struct BandCfg {
  static constexpr int BK = 64, SW = 128;                 // slice rows, streamed tile width
  static constexpr int NCW = QBAND ? 4 : 8, NLW = 2;      // compute and load waves
  static constexpr int NW = NCW + NLW, NTHR = 64 * NW;
  static constexpr int STAGES = QBAND ? 3 : 2;
  static constexpr int BAND_BYTES = 96 * 1024;            // band region at offset 0
  static constexpr int SLICE = BK * SW * 2;               // 64 rows x 128 columns streamed
  static constexpr int RING_OFF = BAND_BYTES;
  static constexpr int STG_OFF = RING_OFF + STAGES * SLICE;
  static constexpr int STG_WAVE = 32 * 64 * 2;            // 32 rows x 64 columns of a compute wave's sub-tile
  static constexpr int LDS_BYTES = STG_OFF + NCW * STG_WAVE;
  static constexpr int DMA = SLICE / 16 / (64 * NLW);     // DMA instructions per load wave per streamed slice
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DMA * 16 * 64 * NLW == SLICE, "DMA split");
};

// One unit shape: band width, output tile, rows it takes
template <bool QBAND, bool WIDE>
struct BandShape {
  using C = BandCfg<QBAND>;
  static constexpr int BW = WIDE ? 256 : 128;             // band width
  static constexpr int BM = QBAND ? C::SW : BW, BN = QBAND ? BW : C::SW;   // output tile
  static constexpr int KMAX = WIDE ? 192 : 384, KS = KMAX / C::BK;
  static constexpr int WM = QBAND ? 2 : 4, WN = C::NCW / WM;   // compute waves over a tile
  static constexpr int FM = BM / (32 * WM), FN = BN / (32 * WN);
  static constexpr int BAND_SLICE = C::BK * BW * 2;       // 64 rows of the band, bf16
  static constexpr int BAND_DMA = BAND_SLICE / 16 / (64 * C::NLW);   // per load wave per band slice
  static_assert(KS * BAND_SLICE <= C::BAND_BYTES, "band region");
  static_assert(BAND_DMA * 16 * 64 * C::NLW == BAND_SLICE && FN % 2 == 0 && FM >= 1, "split");
};
// experts of 1 .. kBandWideRows rows take wide units, up to kBandMaxRows
// narrow ones; the larger go to the ring
constexpr int kBandWideRows = BandShape<true, true>::KMAX;
constexpr int kBandMaxRows = BandShape<true, false>::KMAX;

// DMA of an expert's band (ns slices of 64 rows; rows past n read as zero);
// returns the DMA instructions issued by this load wave
template <class S>
__device__ __forceinline__ int issue_band_dma(const uint16_t* Bo, int64_t ld_band, int kb, int n, int ns, int band,
                                              uint32_t lds, int lw) {
  constexpr int NLW = S::C::NLW;
  DmaPlan<MC, S::BW, S::BAND_DMA, NLW> pa;
  pa.plan_mc(ld_band, band * S::BW, lw);
  const void* base = Bo + (int64_t)kb * ld_band;
  const uint32_t bytes = (uint32_t)(n * ld_band * 2);
  const uint32_t band_slice = (uint32_t)(S::C::BK * ld_band * 2);
  int vm = 0;
#pragma unroll
  for (int s = 0; s < S::KS; ++s)
    if (s < ns) {
      issue_slice_asm<decltype(pa), S::BAND_DMA, NLW>(pa, base, bytes, (uint32_t)s * band_slice,
                                                      lds + s * S::BAND_SLICE, lw);
      vm += S::BAND_DMA;
    }
  return vm;
}

// Compute waves: the TU tiles of one unit (expert g, band `band`, ns slices).
// `n` counts the streamed slices multiplied so far (their ring stages).
template <class Epi, bool QBAND, bool WIDE>
__device__ __forceinline__ void band_unit_tiles(uint32_t lds0, const typename Epi::P& ep, int g, int band, int ns,
                                                int TU, int rot, int wave, int& n) {
  using S = BandShape<QBAND, WIDE>;
  using C = typename S::C;
  constexpr int BM = S::BM, BN = S::BN, FM = S::FM, FN = S::FN;
  const int lane = threadIdx.x & 63;
  const int wm = wave / S::WN, wn = wave % S::WN;
  McFrag<BM, FM> fa;
  McFrag<BN, FN> fb;
  fa.init(wm * (BM / S::WM));
  fb.init(wn * (BN / S::WN));
  const uint32_t stg = lds0 + C::STG_OFF;     // sub-tile of compute wave w at stg + w * STG_WAVE
  floatx16 acc[FM][FN];

  for (int j = 0; j < TU; ++j) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.0f;
    // a runtime loop over the tile's slices keeps the accumulators in one
    // register set
#pragma unroll 1
    for (int s = 0; s < ns; ++s) {
      bar();
      const uint32_t sb = lds0 + C::RING_OFF + (n % C::STAGES) * C::SLICE;   // streamed slice
      const uint32_t sband = lds0 + s * S::BAND_SLICE;                       // band slice
      const uint32_t sm = QBAND ? sb : sband, sn = QBAND ? sband : sb;       // m side, n side
      // fragments of K-step kk + 1 are read while the MFMAs of step kk run
      // (two register sets), in the order the scheduling groups fix
      bf16x8 fm[2][FM], fn[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fm[0][i] = fa.read(sm, i, 0);
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) fn[0][jj] = fb.read(sn, jj, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < 4) {
#pragma unroll
          for (int i = 0; i < FM; ++i) fm[cur ^ 1][i] = fa.read(sm, i, kk + 1);
#pragma unroll
          for (int jj = 0; jj < FN; ++jj) fn[cur ^ 1][jj] = fb.read(sn, jj, kk + 1);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj)   // n-side fragment first: acc[i][jj] is m-block i x n-block jj
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fn[cur][jj], fm[cur][i], acc[i][jj], 0, 0, 0);
      }
      sched_pipelined_slice<2 * (FM + FN), FM * FN>();
      ++n;
    }
    // tile end: the sub-tile through this wave's staging area, 32 x 64 at a
    // time (LDS operations of one wave execute in order), to 128-byte row pieces
    const int jt = (j + rot * band) % TU;     // the unit's tiles in rotated order
    const int row0 = (QBAND ? jt : band) * BM, col0 = (QBAND ? band : jt) * BN;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(ep.C + g * ep.c_gstride + (int64_t)row0 * ep.ldc, (uint32_t)(BM * ep.ldc * 2));
    const uint32_t col_off = (uint32_t)(col0 + wn * (BN / S::WN) + (lane & 7) * 8) * 2;
    MOE_LDS u32x2* w2 = (MOE_LDS u32x2*)(uintptr_t)(stg + wave * C::STG_WAVE);
    const MOE_LDS u32x4* r4 = (const MOE_LDS u32x4*)(uintptr_t)(stg + wave * C::STG_WAVE);
    // one 32 x 64 piece per round: row block i, columns 64 jp .. 64 jp + 63
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int jp = 0; jp < FN / 2; ++jp) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = lane & 31, chunk = jj * 4 + q;
            const floatx16& a4 = acc[i][2 * jp + jj];
            const u32x2 v = {pack_bf16x2(a4[4 * q], a4[4 * q + 1]), pack_bf16x2(a4[4 * q + 2], a4[4 * q + 3])};
            w2[(row * 8 + (chunk ^ stage_swz(row))) * 2 + (lane >> 5)] = v;
          }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rr = it * 8 + (lane >> 3), cc = lane & 7;
          const u32x4 v = r4[rr * 8 + (cc ^ stage_swz(rr))];
          store_b128<true>(v, rs, col_off + (uint32_t)(jp * 128) +
                                      (uint32_t)((wm * (BM / S::WM) + i * 32 + rr) * ep.ldc * 2));
        }
      }
    }
  }
}

// QBAND = true: the band is columns of Q (the output's column side) and the
// unit walks the output's row tiles, streaming P; false: the band is columns
// of P and the unit walks column tiles, streaming Q.  UB = 128-column bands
// per expert (even: an expert has UB / 2 wide units or UB narrow ones), TU =
// 128-wide tiles per unit.
//
// Wave roles.  A wave's loads and stores share one in-order completion
// counter, so a wave that stores a tile's outputs and then waits for a DMA
// issued after them waits for the stores as well, and stops feeding the store
// queue while it waits.  The roles are therefore split: compute waves
// (MFMA, LDS, and the stores of their own sub-tiles; they never wait on
// memory, so their stores stream, up to the 63 operations a wave may have
// outstanding) and two load waves (every DMA, and every wait for one).  All
// run the same unit / tile / slice skeleton and meet at the same barriers:
//   unit start:  B [load: DMA of the band, and the wait for it] B
//   slice n:     [load: wait for slice n] B [load: DMA of slice n + STAGES - 1]
//                [compute: MFMAs of slice n]
//   tile end:    [compute: sub-tile -> own staging area -> global stores]
template <class Epi, bool QBAND>
__global__ __launch_bounds__(BandCfg<QBAND>::NTHR) void gemm_band_kernel(GemmArgs a, typename Epi::P ep, int UB, int TU,
                                                                 int rot) {
  using C = BandCfg<QBAND>;
  constexpr int BK = C::BK, STAGES = C::STAGES;
  static_assert(Epi::kStaged, "bf16 output");
  extern __shared__ u32x4 smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOE_LDS void*)smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_compute = wave < C::NCW;
  const bool is_load = wave >= C::NCW && wave < C::NCW + C::NLW;
  const int lw = wave - C::NCW;               // load waves
  const int* off = a.offsets;
  const int G = a.G;

  // The G + 1 offsets, loaded once: offset i sits in lane i % 64 of ov[i / 64]
  // and is fetched with readlane, so the loops hold no memory access of their
  // own that a wait could be needed for.
  static_assert(kMaxExperts + 1 <= 5 * 64, "offsets in five registers");
  int ov[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) ov[q] = q * 64 + lane <= G ? off[q * 64 + lane] : 0;
  // a wait the compiler sees (vmcnt 0, other counters at their maximum): it
  // then knows the offsets are in place and adds no waits before their uses
  __builtin_amdgcn_s_waitcnt(0x0F70);
  auto lane_at = [&](const int (&r)[5], int i) -> int {
    const int l = i & 63, q = i >> 6;
    const int v0 = __builtin_amdgcn_readlane(r[0], l), v1 = __builtin_amdgcn_readlane(r[1], l);
    const int v2 = __builtin_amdgcn_readlane(r[2], l), v3 = __builtin_amdgcn_readlane(r[3], l);
    const int v4 = __builtin_amdgcn_readlane(r[4], l);
    return q == 0 ? v0 : q == 1 ? v1 : q == 2 ? v2 : q == 3 ? v3 : v4;
  };
  auto off_at = [&](int i) { return lane_at(ov, i); };
  auto rows_of = [&](int g) { return off_at(g + 1) - off_at(g); };
  // units of an expert of n rows, and the estimated cost of one (its slices
  // plus its tiles' stores, in slices: a wide tile stores twice the bytes)
  auto units_of = [&](int n) { return (n > 0 && n <= kBandMaxRows) ? (n <= kBandWideRows ? UB / 2 : UB) : 0; };
  auto cost_of = [&](int n) { return (n + BK - 1) / BK + (n <= kBandWideRows ? 8 : 4); };

  // inclusive scans per expert, in the staging area (no epilogue uses it
  // before the barriers below): the units' cost, and their count
  int64_t* pre = (int64_t*)((char*)smem + C::STG_OFF);
  int* ucum = (int*)((char*)smem + C::STG_OFF + kMaxExperts * 8);
  static_assert(kMaxExperts <= C::NTHR && kMaxExperts * 12 <= C::NCW * C::STG_WAVE, "one thread per expert");
  {
    const int g = threadIdx.x;
    if (g < kMaxExperts) {
      const int n = g < G ? off[g + 1] - off[g] : 0;
      const int u = units_of(n);
      pre[g] = u > 0 ? (int64_t)u * cost_of(n) : 0;
      ucum[g] = u;
    }
    __syncthreads();
    for (int o = 1; o < kMaxExperts; o <<= 1) {
      const int64_t add = (g < kMaxExperts && g >= o) ? pre[g - o] : 0;
      const int uadd = (g < kMaxExperts && g >= o) ? ucum[g - o] : 0;
      __syncthreads();
      if (g < kMaxExperts) {
        pre[g] += add;
        ucum[g] += uadd;
      }
      __syncthreads();
    }
  }
  // units before expert i (i = 0..G; i = G: all of them), in registers like
  // the offsets
  int uv[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int i = q * 64 + lane;
    uv[q] = i == 0 || i > G ? 0 : ucum[i - 1];
  }
  auto ubefore = [&](int i) { return lane_at(uv, i); };
  const int U = ubefore(G);
  // values read from LDS are uniform: keep them (and all that derives from
  // them: experts, offsets, branch conditions) in scalar registers
  const int64_t W = (int64_t)__builtin_amdgcn_readfirstlane((int)(pre[G - 1] >> 32)) << 32 |
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)pre[G - 1]);
  const int grid = gridDim.x, b = blockIdx.x;
  const int X = grid < 8 ? grid : 8, xcd = b % X, wi = b / X, nx = (grid - xcd + X - 1) / X;
  // first unit of XCD x's run: the first unit whose cumulative cost reaches W x / X
  auto run_start = [&](int x) -> int {
    if (x <= 0) return 0;
    if (x >= X) return U;
    const int64_t T = W * x / X;
    int lo = 0, hi = G;                       // first g with pre[g] > T (inclusive prefix)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] > T) hi = mid; else lo = mid + 1;
    }
    if (lo >= G) return U;
    const int64_t before = lo > 0 ? pre[lo - 1] : 0;
    const int n = rows_of(lo);                // has units: its cost is above the previous prefix
    const int64_t in = (T - before + cost_of(n) - 1) / cost_of(n);
    const int u = units_of(n);
    return ubefore(lo) + (int)(in < u ? in : u);
  };
  const int run_lo = __builtin_amdgcn_readfirstlane(run_start(xcd));
  const int run_hi = __builtin_amdgcn_readfirstlane(run_start(xcd + 1));
  __syncthreads();                            // the scans' LDS is staging from here on

  struct Unit {
    int r;         // step in this workgroup's stride (-1: finished)
    int g, band;   // expert and band
    int kb, n;     // first row and row count of the expert
    int ns;        // 64-row slices
    bool wide;
  };
  // the unit of step r: unit L of the expert-major list belongs to the last
  // expert with at most L units before it
  auto settle = [&](int r, Unit& u) {
    const int L = run_lo + wi + r * nx;
    if (L >= run_hi) {
      u.r = -1;
      return;
    }
    int lo = 0, hi = G;                       // ubefore(lo) <= L < ubefore(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ubefore(mid) <= L) lo = mid; else hi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(lo);
    u.r = r;
    u.g = g;
    u.band = L - ubefore(g);
    u.kb = off_at(g);
    u.n = rows_of(g);
    u.ns = (u.n + BK - 1) / BK;
    u.wide = u.n <= kBandWideRows;
  };

  const uint16_t* P = (const uint16_t*)a.A;
  const uint16_t* Q = (const uint16_t*)a.B;
  // band operand (rows of Bo, ld_band) and streamed operand (rows of So, ld_str)
  const uint16_t* Bo = QBAND ? Q : P;
  const uint16_t* So = QBAND ? P : Q;
  const int64_t ld_band = QBAND ? a.ldb : a.lda, ld_str = QBAND ? a.lda : a.ldb;
  const uint32_t str_slice = (uint32_t)(BK * ld_str * 2);

  // ---- load waves: DMA issue and the waits for it --------------------------
  int vm = 0;                                 // DMA instructions issued by this load wave
  DmaPlan<MC, C::SW, C::DMA, C::NLW> pb;
  auto issue_band = [&](const Unit& u) {
    vm += u.wide ? issue_band_dma<BandShape<QBAND, true>>(Bo, ld_band, u.kb, u.n, u.ns, u.band, lds0, lw)
                 : issue_band_dma<BandShape<QBAND, false>>(Bo, ld_band, u.kb, u.n, u.ns, u.band, lds0, lw);
  };
  struct LdIt {
    Unit u;
    int j, s;
  } ld;
  const void* rb_base = nullptr;
  uint32_t rb_bytes = 0, sob = 0;
  auto plan_b = [&]() {
    pb.plan_mc(ld_str, ((ld.j + rot * ld.u.band) % TU) * C::SW, lw);
    rb_base = So + (int64_t)ld.u.kb * ld_str;
    rb_bytes = (uint32_t)(ld.u.n * ld_str * 2);
    sob = 0;
  };
  auto advance_ld = [&]() {
    if (++ld.s < ld.u.ns) return;
    ld.s = 0;
    if (++ld.j >= TU) {
      ld.j = 0;
      settle(ld.u.r + 1, ld.u);
    }
    if (ld.u.r >= 0) plan_b();
  };
  // `vm` after each stage's slice was issued, kept in lane `stage` of one
  // register (an array indexed by the stage would live in scratch memory, whose
  // accesses are vector memory operations that every wait would then drain)
  int marks = 0;
  int issued = 0;                             // slices issued
  auto issue_b = [&]() {
    const int stage = issued % STAGES;
    issue_slice_asm<decltype(pb), C::DMA, C::NLW>(pb, rb_base, rb_bytes, sob, lds0 + C::RING_OFF + stage * C::SLICE,
                                                  lw);
    sob += str_slice;
    vm += C::DMA;
    marks = lane == stage ? vm : marks;
    ++issued;
    advance_ld();
  };

  Unit cu;
  settle(0, cu);
  if (cu.r < 0) return;
  ld.u = cu;
  ld.j = 0;
  ld.s = 0;
  if (is_load) {
    plan_b();
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (ld.u.r >= 0) issue_b();
  }

  // The roles run separate loops over the same unit / tile / slice sequence
  // and meet at the same barriers: 2 per unit, then one per slice.
  if (is_load) {
    int n = 0;                                // slice being multiplied
    do {
      // unit start: after the first barrier every compute wave is done with
      // the previous unit's band; fetch this unit's band
      bar();
      issue_band(cu);
      wait_vmcnt_dyn<0, 0>(0);
      bar();
      Unit nu;
      settle(cu.r + 1, nu);
      for (int j = 0; j < TU; ++j) {
#pragma unroll 1
        for (int s = 0; s < cu.ns; ++s) {
          wait_vmcnt_dyn<0, 63>(vm - __builtin_amdgcn_readlane(marks, n % STAGES));
          bar();
          if (ld.u.r >= 0) issue_b();         // into the stage of slice n - 1
          ++n;
        }
      }
      cu = nu;
    } while (cu.r >= 0);
    return;
  }
  if (!is_compute) return;                    // (no other roles: NW = NCW + NLW)

  // ---- compute waves ------------------------------------------------------
  int n = 0;                                  // slice being multiplied
  do {
    bar();
    bar();
    Unit nu;
    settle(cu.r + 1, nu);
    if (cu.wide) band_unit_tiles<Epi, QBAND, true>(lds0, ep, cu.g, cu.band, cu.ns, TU, rot, wave, n);
    else band_unit_tiles<Epi, QBAND, false>(lds0, ep, cu.g, cu.band, cu.ns, TU, rot, wave, n);
    cu = nu;
  } while (cu.r >= 0);
}

}  // namespace moe
