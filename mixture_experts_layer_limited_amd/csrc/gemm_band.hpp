// Weight-gradient kernel with a stationary operand band (bf16, gfx950).
//
// Product: C[g] (M x N) = P_g^T Q_g, where P_g [n_g x M] and Q_g [n_g x N] are
// the rows of group (expert) g in row-contiguous storage: the contraction runs
// over the expert's rows, n_g of them.  At an average of a few hundred rows per
// expert the output (all of C, bf16) is far larger than the operands.
//
// Work unit: (expert g, band of 128 columns of one operand: of Q when the band
// is on the output's column side, of P when on its row side).  The band,
// n_g x 128 values (n_g <= 320), goes into LDS by DMA at the start of the unit,
// and the unit walks the 128-wide tiles of the output's other side, streaming
// the other operand in 64-row slices through a 4-stage DMA ring: a 128 x 128
// output tile costs 128 x n_g x 2 bytes of operand reads instead of twice that.
// Compute waves read the fragments of both operands from LDS.
//
// Waits.  Vector memory operations of a wave complete in issue order, so the
// wait for a slice allows exactly the operations issued after that slice's DMA
// to stay outstanding: a load wave counts what it issues and records the count
// after each slice.
//
// Schedule.  One workgroup of six waves per CU (the band, the ring and the
// epilogue staging fill the 160 KB of LDS), four compute waves of 64 x 64 over a
// 128 x 128 tile.  Each XCD owns one contiguous run of the expert-major unit
// list, split by estimated cost, and its workgroups stride through it, so the
// workgroups of an XCD hold neighbouring bands of one expert; each unit walks
// its tiles from its band index on, so neighbours stream different tiles at
// any time.  Experts with no rows or more than 320 rows are not units of this
// kernel (the caller zero-fills the first and runs the DMA ring on the second).
//
// Epilogue: each compute wave writes its 64 x 64 sub-tile as bf16, 32 rows at
// a time, into its own 4 KB staging area (LDS operations of one wave execute in
// order, so no barrier is needed) and stores it back as 128-byte row segments,
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

struct BandCfg {
  static constexpr int BM = 128, BN = 128, BK = 64, KMAX = 320, KS = KMAX / BK;
  static constexpr int WM = 2, WN = 2, FM = 2, FN = 2;
  static constexpr int NCW = 4, NLW = 2;                 // compute and load waves
  static constexpr int NW = NCW + NLW, NTHR = 64 * NW;
  static constexpr int STAGES = 4;
  static constexpr int SLICE = BK * 128 * 2;              // 64 rows x 128 columns, bf16
  static constexpr int A_OFF = 0;                         // KS slices of the band
  static constexpr int RING_OFF = KS * SLICE;
  static constexpr int STG_OFF = RING_OFF + STAGES * SLICE;
  static constexpr int STG_WAVE = 32 * 64 * 2;            // half of a compute wave's 64 x 64 sub-tile
  static constexpr int LDS_BYTES = STG_OFF + NCW * STG_WAVE;
  static constexpr int DMA = SLICE / 16 / (64 * NLW);     // DMA instructions per load wave per slice
  static constexpr int UNIT_EPI_COST = 4;                 // a tile's stores, in slices, for run splitting
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(DMA * 16 * 64 * NLW == SLICE, "DMA split");
  static_assert(WM * WN == NCW, "waves");
};

// QBAND = true: the band is 128 columns of Q (the output's column side) and
// the unit walks the output's row tiles, streaming P; false: the band is 128
// columns of P and the unit walks column tiles, streaming Q.  UB = bands per
// expert, TU = tiles per unit.
//
// Wave roles.  A wave's loads and stores share one in-order completion
// counter, so a wave that stores a tile's outputs and then waits for a DMA
// issued after them waits for the stores as well, and stops feeding the store
// queue while it waits.  The roles are therefore split: four compute waves
// (MFMA, LDS, and the stores of their own 64 x 64 sub-tiles; they never wait
// on memory, so their stores stream, up to the 63 operations a wave may have
// outstanding) and two load waves (every DMA, and every wait for one).  All
// six run the same unit / tile / slice skeleton and meet at the same barriers:
//   unit start:  B [load: DMA of the band, and the wait for it] B
//   slice n:     [load: wait for slice n] B [load: DMA of slice n + STAGES - 1]
//                [compute: MFMAs of slice n]
//   tile end:    [compute: sub-tile -> own staging area -> global stores]
template <class Epi, bool QBAND>
__global__ __launch_bounds__(BandCfg::NTHR) void gemm_band_kernel(GemmArgs a, typename Epi::P ep, int UB, int TU,
                                                                 int rot) {
  using C = BandCfg;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, KMAX = C::KMAX, KS = C::KS, STAGES = C::STAGES;
  static_assert(Epi::kStaged, "bf16 output");
  extern __shared__ u32x4 smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOE_LDS void*)smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_compute = wave < C::NCW;
  const bool is_load = wave >= C::NCW && wave < C::NCW + C::NLW;
  const int wm = (wave % C::NCW) / C::WN, wn = (wave % C::NCW) % C::WN;   // compute waves
  const int lw = wave - C::NCW;                                          // load waves
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
  auto off_at = [&](int i) -> int {
    const int l = i & 63, q = i >> 6;
    const int v0 = __builtin_amdgcn_readlane(ov[0], l), v1 = __builtin_amdgcn_readlane(ov[1], l);
    const int v2 = __builtin_amdgcn_readlane(ov[2], l), v3 = __builtin_amdgcn_readlane(ov[3], l);
    const int v4 = __builtin_amdgcn_readlane(ov[4], l);
    return q == 0 ? v0 : q == 1 ? v1 : q == 2 ? v2 : q == 3 ? v3 : v4;
  };
  // unit cost of expert g (0: not handled here); a unit is one band of one expert
  auto rows_of = [&](int g) { return off_at(g + 1) - off_at(g); };
  auto cost_of = [&](int n) { return (n > 0 && n <= KMAX) ? (n + BK - 1) / BK + C::UNIT_EPI_COST : 0; };

  // cumulative unit cost per expert (inclusive scan in the staging area, which
  // no epilogue uses before the barriers below)
  int64_t* pre = (int64_t*)((char*)smem + C::STG_OFF);
  static_assert(kMaxExperts <= C::NTHR, "one thread per expert");
  {
    const int g = threadIdx.x;
    if (g < kMaxExperts) pre[g] = g < G ? (int64_t)UB * cost_of(off[g + 1] - off[g]) : 0;
    __syncthreads();
    for (int o = 1; o < kMaxExperts; o <<= 1) {
      const int64_t add = (g < kMaxExperts && g >= o) ? pre[g - o] : 0;
      __syncthreads();
      if (g < kMaxExperts) pre[g] += add;
      __syncthreads();
    }
  }
  // values read from LDS are uniform: keep them (and all that derives from
  // them: experts, offsets, branch conditions) in scalar registers
  const int64_t W = (int64_t)__builtin_amdgcn_readfirstlane((int)(pre[G - 1] >> 32)) << 32 |
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)pre[G - 1]);
  const int grid = gridDim.x, b = blockIdx.x;
  const int X = grid < 8 ? grid : 8, xcd = b % X, wi = b / X, nx = (grid - xcd + X - 1) / X;
  // first unit of XCD x's run: the first unit whose cumulative cost reaches W x / X
  auto run_start = [&](int x) -> int {
    if (x <= 0) return 0;
    if (x >= X) return G * UB;
    const int64_t T = W * x / X;
    int lo = 0, hi = G;                       // first g with pre[g] > T (inclusive prefix)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] > T) hi = mid; else lo = mid + 1;
    }
    if (lo >= G) return G * UB;
    const int64_t before = lo > 0 ? pre[lo - 1] : 0;
    const int64_t ce = cost_of(rows_of(lo));
    const int64_t in = (T - before + ce - 1) / ce;
    return lo * UB + (int)(in < UB ? in : UB);
  };
  const int run_lo = __builtin_amdgcn_readfirstlane(run_start(xcd));
  const int run_hi = __builtin_amdgcn_readfirstlane(run_start(xcd + 1));
  __syncthreads();                            // the scan's LDS is staging from here on

  struct Unit {
    int r;         // step in this workgroup's stride (-1: finished)
    int g, band;   // expert and band
    int kb, n;     // first row and row count of the expert
    int ns;        // 64-row slices
  };
  // first step >= r holding a unit of this kernel; other experts are skipped whole
  auto settle = [&](int r, Unit& u) {
    for (;;) {
      const int L = run_lo + wi + r * nx;
      if (L >= run_hi) break;
      const int g = __builtin_amdgcn_readfirstlane(L / UB);
      const int n = rows_of(g);
      if (n > 0 && n <= KMAX) {
        u.r = r; u.g = g; u.band = L % UB; u.kb = off_at(g); u.n = n; u.ns = (n + BK - 1) / BK;
        return;
      }
      const int next = (g + 1) * UB - run_lo - wi;       // > r * nx: L is below the next expert
      r = (next + nx - 1) / nx;                          // first step in the next expert
    }
    u.r = -1;
  };

  const uint16_t* P = (const uint16_t*)a.A;
  const uint16_t* Q = (const uint16_t*)a.B;
  // band operand (rows of Bo, ld_band) and streamed operand (rows of So, ld_str)
  const uint16_t* Bo = QBAND ? Q : P;
  const uint16_t* So = QBAND ? P : Q;
  const int64_t ld_band = QBAND ? a.ldb : a.lda, ld_str = QBAND ? a.lda : a.ldb;
  const uint32_t band_slice = (uint32_t)(BK * ld_band * 2);
  const uint32_t str_slice = (uint32_t)(BK * ld_str * 2);

  // ---- load waves: DMA issue and the waits for it --------------------------
  int vm = 0;                                 // DMA instructions issued by this load wave
  DmaPlan<MC, 128, C::DMA, C::NLW> pb;
  auto issue_band = [&](const Unit& u) {
    DmaPlan<MC, 128, C::DMA, C::NLW> pa;
    pa.plan_mc(ld_band, u.band * 128, lw);
    const void* base = Bo + (int64_t)u.kb * ld_band;
    const uint32_t bytes = (uint32_t)(u.n * ld_band * 2);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (s < u.ns) {
        issue_slice_asm<decltype(pa), C::DMA, C::NLW>(pa, base, bytes, (uint32_t)s * band_slice,
                                                      lds0 + C::A_OFF + s * C::SLICE, lw);
        vm += C::DMA;
      }
  };
  struct LdIt {
    Unit u;
    int j, s;
  } ld;
  const void* rb_base = nullptr;
  uint32_t rb_bytes = 0, sob = 0;
  auto plan_b = [&]() {
    pb.plan_mc(ld_str, ((ld.j + rot * ld.u.band) % TU) * 128, lw);
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
  McFrag<BM, C::FM> fa;
  McFrag<BN, C::FN> fb;
  fa.init(wm * (BM / C::WM));
  fb.init(wn * (BN / C::WN));
  const uint32_t stg = lds0 + C::STG_OFF;     // sub-tile of compute wave w at stg + w * STG_WAVE
  floatx16 acc[C::FM][C::FN];

  int n = 0;                                  // slice being multiplied
  do {
    bar();
    bar();
    Unit nu;
    settle(cu.r + 1, nu);

    for (int j = 0; j < TU; ++j) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][jj][e] = 0.0f;
      // a runtime loop over the tile's slices keeps the accumulators in one
      // register set
#pragma unroll 1
      for (int s = 0; s < cu.ns; ++s) {
        bar();
        const uint32_t sb = lds0 + C::RING_OFF + (n % STAGES) * C::SLICE;   // streamed slice
        const uint32_t sband = lds0 + C::A_OFF + s * C::SLICE;               // band slice
        const uint32_t sm = QBAND ? sb : sband, sn = QBAND ? sband : sb;      // m side, n side
        // fragments of K-step kk + 1 are read while the MFMAs of step kk run
        // (two register sets), in the order the scheduling groups fix
        bf16x8 fm[2][C::FM], fn[2][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) fm[0][i] = fa.read(sm, i, 0);
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) fn[0][jj] = fb.read(sn, jj, 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int cur = kk & 1;
          if (kk + 1 < 4) {
#pragma unroll
            for (int i = 0; i < C::FM; ++i) fm[cur ^ 1][i] = fa.read(sm, i, kk + 1);
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj) fn[cur ^ 1][jj] = fb.read(sn, jj, kk + 1);
          }
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj)   // n-side fragment first: acc[i][jj] is m-block i x n-block jj
              acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fn[cur][jj], fm[cur][i], acc[i][jj], 0, 0, 0);
        }
        sched_pipelined_slice<2 * (C::FM + C::FN), C::FM * C::FN>();
        ++n;
      }
      // tile end: the sub-tile through this wave's staging area, 32 rows at a
      // time (LDS operations of one wave execute in order), to 128-byte row pieces
      {
        const int jt = (j + rot * cu.band) % TU;   // the unit's tiles in rotated order
        const int row0 = (QBAND ? jt : cu.band) * BM, col0 = (QBAND ? cu.band : jt) * BN;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(ep.C + cu.g * ep.c_gstride + (int64_t)row0 * ep.ldc, (uint32_t)(BM * ep.ldc * 2));
        const uint32_t col_off = (uint32_t)(col0 + wn * (BN / C::WN) + (lane & 7) * 8) * 2;
        MOE_LDS u32x2* w2 = (MOE_LDS u32x2*)(uintptr_t)(stg + wave * C::STG_WAVE);
        const MOE_LDS u32x4* r4 = (const MOE_LDS u32x4*)(uintptr_t)(stg + wave * C::STG_WAVE);
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
#pragma unroll
          for (int jj = 0; jj < C::FN; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = lane & 31, chunk = jj * 4 + q;
              const u32x2 v = {pack_bf16x2(acc[i][jj][4 * q], acc[i][jj][4 * q + 1]),
                               pack_bf16x2(acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3])};
              w2[(row * 8 + (chunk ^ stage_swz(row))) * 2 + (lane >> 5)] = v;
            }
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int rr = it * 8 + (lane >> 3), cc = lane & 7;
            const u32x4 v = r4[rr * 8 + (cc ^ stage_swz(rr))];
            store_b128<true>(v, rs, col_off + (uint32_t)((wm * (BM / C::WM) + i * 32 + rr) * ep.ldc * 2));
          }
        }
      }
    }
    cu = nu;
  } while (cu.r >= 0);
}

}  // namespace moe
