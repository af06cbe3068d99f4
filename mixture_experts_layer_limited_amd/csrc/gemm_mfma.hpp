// bf16 MFMA grouped-GEMM kernel for gfx950 (v_mfma_f32_32x32x16_bf16).
//
// Data path.  Operand tiles go from global memory straight into LDS with
// buffer_load_dwordx4 ... lds (16 bytes per lane, written to LDS in lane
// order from the M0 base), so no registers are spent on staging and STAGES
// K-slices of 64 can be in flight in an LDS ring.  Each operand of a tile gets
// a buffer resource whose range ends where its valid rows end, and each lane a
// 32-bit offset computed once per tile; a slice advances only the scalar
// offset.  Loads outside the range return zeros, which masks rows past an
// expert's end, the ragged contraction of weight gradients, and rows past N
// (those lanes get an offset beyond any range).  K-contiguous operands need K
// to be a multiple of 64.
//
// LDS layouts (16-byte chunks; LDS serves 64 banks, 16 lanes of a 16-byte read
// or 32 lanes of an 8-byte read per cycle):
//   K-contiguous operand ("KC"): row r holds its 64 K values as 8 chunks,
//     logical chunk c at position c ^ ((r >> 1) & 7).  Fragments are read with
//     ds_read_b128; the 16 lanes of a cycle read 16 consecutive rows (8 even
//     rows in one half of the banks, 8 odd rows in the other) at 8 distinct
//     positions each.
//   Row-contiguous operand ("MC", the weight in dgrad, both operands in wgrad):
//     the slice is kept as it lies in memory, 64 K-rows of ROWS values (ROWS/8
//     chunks), logical chunk c of K-row k at position c ^ (2 (k & 3) | 8 c1),
//     c1 = bit 1 of c.  Fragments are read with ds_read_b64_tr_b16: in each
//     group of 16 lanes, lane i receives element i%4 of the 8-byte piece
//     addressed by lane i/4 + 4j (j = 0..3).  Pointing lane q at K-row
//     k0 + q/4, columns n0 + 4(q%4) .. +3 hands lane i the four K values
//     k0..k0+3 of column n0 + i -- an MFMA fragment straight from the
//     row-contiguous layout.  A cycle's 32 lanes touch 4 K-rows x 4 chunks,
//     which the XOR spreads over all 16 chunk positions of the 64 banks.
//   Per-lane read offsets are computed once; the K step enters as an
//   immediate offset and the ring stage as one add per slice.
//
// Schedule.  Each XCD owns one contiguous run of the logical tiles
// (xcd_run_start) and its workgroups stride through it, so tiles running
// together on one XCD are neighbours in the expert-major order and share
// weight / activation panels in its L2.  With G >= tiles every workgroup gets
// at most one tile; with a smaller grid the kernel is persistent.  The
// loads walk (tile, slice) pairs: the DMA for the pair STAGES-1 ahead is issued
// before the current pair is multiplied, so loads of the next tile overlap the
// current tile's last slices and its epilogue.  The multiply side is a tile
// loop around a slice loop with the epilogue between slice loops, so the
// accumulators never move between register files inside the slice loop.  Tiles with an empty
// contraction are skipped (the caller zero-fills them).
//
// The MFMA takes the B fragment first, so a lane's accumulator holds four
// consecutive output columns (element e of a block: column 8*(e/4) +
// 4*(lane/32) + e%4, row lane%32) and the epilogue stores 4-column vectors.
//
// Synchronisation: s_barrier without a memory fence (a fenced barrier would
// drain every in-flight DMA) and explicit s_waitcnt vmcnt(N): a lane's DMA for
// slice s is complete once at most N of its later vector-memory operations are
// outstanding (they complete in issue order, so the epilogue's global stores
// and loads, always issued after the DMA they could be confused with, only
// lengthen a wait).
#pragma once

#include "gemm.hpp"

namespace moe {


constexpr uint32_t kOffRange = 0x80000000u;   // lane offset that is outside every range

// MX = true: fp8 operands with e8m0 scales; a stage then also holds the
// slice's scale words (one 32-bit word = four block scales per row), A's at
// word q < BM of an NW*64-word region, B's at word q < BN of a second one.
// NLW > 0: NLW load waves issue every DMA (and wait for it) beside the WM x WN
// compute waves, which then never wait on memory; 0: every wave does both.
template <int BM, int BN, int WM, int WN, int STAGES, bool MX = false, int NLW = 0, bool FP4 = false>
struct TileCfg {
  static constexpr int BK = 64;
  static constexpr int NW = WM * WN;                       // compute waves
  static constexpr int ND = NLW > 0 ? NLW : NW;            // waves that issue the DMA
  static constexpr int NTHR = 64 * (NW + NLW);
  static constexpr int FM = BM / (32 * WM);
  static constexpr int FN = BN / (32 * WN);
  static constexpr int A_BYTES = BM * 128;                 // one operand slice in LDS
  static constexpr int B_BYTES = BN * 128;
  static constexpr int SC_WORDS = MX ? NW * 64 : 0;        // words per scale region
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + 2 * SC_WORDS * 4;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int A_DMA = BM * 8 / 64 / ND;           // DMA instructions per DMA wave per slice
  static constexpr int B_DMA = BN * 8 / 64 / ND;
  // scale-word DMA per DMA wave and slice: one word per lane, the A words
  // (fp4: two per row) over SC_A instructions, the B words over SC_B
  static constexpr int SC_A = MX ? ((FP4 ? 2 : 1) * BM + 64 * ND - 1) / (64 * ND) : 0;
  static constexpr int SC_B = MX ? ((FP4 ? 2 : 1) * BN + 64 * ND - 1) / (64 * ND) : 0;
  static constexpr int SC_DMA = SC_A + SC_B;
  static_assert(!MX || (SC_WORDS >= BM && SC_WORDS >= BN), "scale regions");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(FM >= 1 && FN >= 1 && BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert(A_DMA * 64 * ND == BM * 8 && B_DMA * 64 * ND == BN * 8, "DMA split");
  static_assert(NLW == 0 || (STAGES - 1) * (A_DMA + B_DMA + SC_DMA) <= 63, "load waves: counts in range");
  static_assert(!MX || (SC_A * ND * 64 <= SC_WORDS && SC_B * ND * 64 <= SC_WORDS), "scale lanes");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "row-contiguous layout needs >= 16 chunks per K-row");
  static_assert(STAGES >= 2, "stages");
  static_assert(STAGE_BYTES <= 65536, "read immediates");
};

// logical chunk -> position helpers
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 7; }

// One DMA instruction per lane group: 16 bytes per lane from a raw buffer
// (base, bytes: reads past the range give zeros) into LDS at `lds` + 16 x lane.
// Written as assembly: the compiler does not track assembly DMA, so it inserts
// no wait of its own before later LDS reads (for the transposing LDS reads it
// would otherwise drain every DMA and store in flight); the kernel's explicit
// vmcnt waits order the reads after the data.  The instruction has no output
// register.
__device__ __forceinline__ void dma_b128(const void* base, uint32_t bytes, uint32_t voff, uint32_t soff,
                                         uint32_t lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  // every operand but the lane offset is uniform: pin them to scalar registers
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const u32x4 rs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu)),
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kRawBufferFlags};
  const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)soff);
  const uint32_t ld = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  uint32_t saved;
  // M0 (the LDS destination base) is restored before the statement ends
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(ld), "v"(voff), "s"(rs), "s"(so)
      : "memory");
#endif
}

// Per-lane byte offsets of one operand slice's DMA (relative to the operand's
// resource base); KC: element (i, k) at i*ld + k (i relative to the base row);
// MC: element (i, k) at k*ld + i (k relative to the base K-row).
template <OpLayout L, int ROWS, int NDMA, int NW>
struct DmaPlan {
  uint32_t off[NDMA];

  // KC: rowv(r) = row of tile row r relative to the resource base, or -1
  template <class RowFn>
  __device__ __forceinline__ void plan_kc(int64_t ld, RowFn rowv, int wave = -1) {
    const int lane = threadIdx.x & 63;
    if (wave < 0) wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int p = (wave + j * NW) * 64 + lane;
      const int r = p >> 3, c = (p & 7) ^ kc_swz(r);
      const int gi = rowv(r);
      off[j] = gi >= 0 ? (uint32_t)((int64_t)gi * ld * 2 + c * 16) : kOffRange;
    }
  }
  // MC: columns i0 + 8c (relative to the base); every K-row 0..63 of the slice
  // (`wave`: this wave's index among the NW waves that share the slice)
  __device__ __forceinline__ void plan_mc(int64_t ld, int i0, int wave = -1) {
    const int lane = threadIdx.x & 63;
    if (wave < 0) wave = threadIdx.x >> 6;
    constexpr int CPR = ROWS / 8;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int p = (wave + j * NW) * 64 + lane;
      const int k = p / CPR, cp = p % CPR;
      const int c1 = ((cp >> 1) & 1) ^ (k & 1);             // bit 1 of the logical chunk
      const int c = cp ^ (((k & 3) << 1) | (c1 << 3));
      off[j] = (uint32_t)((int64_t)k * ld * 2 + (int64_t)(i0 + c * 8) * 2);
    }
  }
  // one slice: instruction j fills chunk positions (wave + j*NW)*64 .. +63
  __device__ __forceinline__ void issue(const void* rbase, uint32_t rbytes, uint32_t soff, uint32_t lds_byte,
                                        int wave = -1) const {
    wave = __builtin_amdgcn_readfirstlane(wave < 0 ? (int)(threadIdx.x >> 6) : wave);
#pragma unroll
    for (int j = 0; j < NDMA; ++j)
      dma_b128(rbase, rbytes, off[j], soff, lds_byte + (uint32_t)((wave + j * NW) * 64 * 16));
  }
};

// Per-lane LDS read offsets (bytes within an operand slice) of the fragments
// a wave reads: NF fragments of 32 tile rows starting at row0 + 32 f.
template <OpLayout L, int ROWS, int NF>
struct FragPlan {
  uint32_t off[4];          // KC: per K-step (same for every fragment)
  McFrag<ROWS, NF> mc;      // MC

  __device__ __forceinline__ void init(int row0) {
    const int lane = threadIdx.x & 63;
    if (L == KC) {
      const int r = lane & 31, h = lane >> 5;               // row0 is a multiple of 32
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        off[kk] = (uint32_t)((row0 + r) * 128 + (((2 * kk + h) ^ kc_swz(r)) * 16));
    } else {
      mc.init(row0);
    }
  }
  // fragment f, K-step kk; `base` = byte address of the operand slice
  __device__ __forceinline__ bf16x8 read(uint32_t base, int f, int kk) const {
    if (L == KC) {
      const MOE_LDS bf16x8* p = (const MOE_LDS bf16x8*)(uintptr_t)(base + off[kk] + f * 32 * 128);
      return *p;
    } else {
      return mc.read(base, f, kk);
    }
  }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `later` slices of DMA (D operations each) are outstanding
template <int MAXL, int D>
__device__ __forceinline__ void wait_slices_after(int later) {
  if constexpr (MAXL <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<MAXL * D>();
    else wait_slices_after<MAXL - 1, D>(later);
  }
}

// wait until at most n (0 <= n) vector-memory operations of this wave are
// outstanding; n is uniform.  Counts above 63 (the counter's range) wait for 63.
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID) wait_vmcnt_dyn<MID, HI>(n);
    else wait_vmcnt_dyn<LO, MID - 1>(n);
  }
}

__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// position in the (tile, slice) sequence of one workgroup
struct SliceIter {
  int r;          // step of the current tile in the workgroup's stride (-1: finished)
  int ks, nk;     // slice within the tile, slices of the tile
  TileCoord c;
};

// Scheduling groups of one 64-deep slice (four K-steps) whose fragments are
// double-buffered: step 0's R LDS reads, then for steps 0..2 the next step's R
// reads interleaved with the first of this step's MF MFMAs, then step 3's MFMAs.  Without
// them the compiler issues each step's reads right before its MFMAs and waits
// for them, exposing the LDS latency on every step.
template <int R, int MF, int Q>
__device__ __forceinline__ void sched_step_groups() {
  if constexpr (Q < MF) {
    // front-loaded: ceil(R / MF) reads before each MFMA until the R are issued
    constexpr int per = (R + MF - 1) / MF;
    constexpr int reads = R - per * Q >= per ? per : (R - per * Q > 0 ? R - per * Q : 0);
    if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_step_groups<R, MF, Q + 1>();
  }
}
template <int R, int MF>
__device__ __forceinline__ void sched_pipelined_slice() {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  sched_step_groups<R, MF, 0>();
  sched_step_groups<R, MF, 0>();
  sched_step_groups<R, MF, 0>();
  __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
}

// MX = true: both operands K-contiguous fp8 e4m3 codes with e8m0 scales (`s`),
// multiplied with v_mfma_scale_f32_32x32x64_f8f6f4 (operand layout at
// MxArgs in gemm.hpp); GemmArgs then count K, lda, ldb in 2-byte units, so a slice of
// BK = 64 units is 128 fp8 values and the data path is the bf16 one.
template <int BM, int BN, int WM, int WN, int STAGES, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi,
          bool MX = false, bool FP4 = false, int NLW = 0>
// (every configuration fills a CU's LDS with one workgroup, so at most two
// waves share a SIMD, three with load waves: the compiler may give each the
// registers of two, or a third of the SIMD's)
__global__ __launch_bounds__(64 * (WM * WN + NLW)) __attribute__((amdgpu_waves_per_eu(1, NLW > 0 ? 3 : 2))) void
gemm_mfma_kernel(GemmArgs a, MxArgs s, typename Epi::P ep, int NT, int MT) {
  using C = TileCfg<BM, BN, WM, WN, STAGES, MX, NLW, FP4>;
  constexpr bool WS = NLW > 0;
  static_assert(!MX || (LA == KC && LB == KC && MODE != RAGGED_K), "MXFP8: K-contiguous row-ragged products");
  // FP4: two scale words per row and slice, fetched by lanes 2 r and 2 r + 1
  static_assert(!FP4 || (MX && 2 * BM <= C::SC_WORDS && 2 * BN <= C::SC_WORDS), "fp4 scale regions");
  constexpr int BK = C::BK, FM = C::FM, FN = C::FN;
  constexpr int DMA_PER_SLICE = C::A_DMA + C::B_DMA + C::SC_DMA;
  extern __shared__ u32x4 smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOE_LDS void*)smem;

  const int total = total_tiles<MODE>(a, NT, MT);
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;       // compute waves
  const bool is_load = WS && wave >= C::NW;
  const int dw = WS ? wave - C::NW : wave;         // index among the DMA waves
  // each XCD walks one contiguous run of tiles (xcd_run_start); with a grid
  // of at least `total` workgroups every workgroup gets at most one tile
  const int X = G < 8 ? G : 8, xcd = b % X, wi = b / X, nx = (G - xcd + X - 1) / X;
  const int run_lo = xcd_run_start<MODE>(a, a.offsets, total, MT * NT, xcd, X);
  const int run_hi = xcd_run_start<MODE>(a, a.offsets, total, MT * NT, xcd + 1, X);

  // next step >= r holding a tile of this workgroup with a non-empty contraction
  auto settle = [&](int r, SliceIter& it) {
    for (;; ++r) {
      const int L = run_lo + wi + r * nx;
      if (L >= run_hi) break;
      resolve_tile<MODE, BM>(a, L, NT, MT, it.c);
      it.nk = (it.c.k_end - it.c.k_begin + BK - 1) / BK;
      // a tile starting past its group's rows has nothing to do (only a tile
      // prefix built for another tile height could produce one)
      if (it.c.m0 >= it.c.m_end) it.nk = 0;
      if (MODE == RAGGED_K && it.c.k_end - it.c.k_begin <= a.k_skip) {
        // the whole group is skipped (empty, or left to another kernel): go
        // to this workgroup's first step in the next group
        const int next = (it.c.g + 1) * MT * NT - run_lo - wi;   // > r * nx
        r = (next + nx - 1) / nx - 1;
        continue;
      }
      if (it.nk > 0) {
        it.r = r;
        it.ks = 0;
        return;
      }
    }
    it.r = -1;
  };

  // DMA state of the load iterator: resources, per-lane offsets, slice strides
  DmaPlan<LA, BM, C::A_DMA, C::ND> pa;
  DmaPlan<LB, BN, C::B_DMA, C::ND> pb;
  const void* ra_base = nullptr;   // operand resources: base address and byte range
  const void* rb_base = nullptr;
  uint32_t ra_bytes = 0, rb_bytes = 0;
  uint32_t soa = 0, sob = 0;
  // MX: scale-word resources, per-lane offsets and the slice's byte offsets
  const uint8_t* rsa_base = nullptr;
  const uint8_t* rsb_base = nullptr;
  uint32_t rsa_bytes = 0, rsb_bytes = 0, sosa = 0, sosb = 0;
  uint32_t sa_off[C::SC_A > 0 ? C::SC_A : 1], sb_off[C::SC_B > 0 ? C::SC_B : 1];
  // grouped scale words per slice: one (fp8, 128 values) or two (fp4, 256)
  constexpr int kWordsPerSlice = FP4 ? 2 : 1;
  const int nb = MX ? a.K / (FP4 ? 8 : 16) : 0;     // blocks of 32 values along K (K in 2-byte units)
  const uint32_t stride_a = LA == KC ? BK * 2 : (uint32_t)(BK * a.lda * 2);
  const uint32_t stride_b = LB == KC ? BK * 2 : (uint32_t)(BK * a.ldb * 2);

  auto plan_tile = [&](const TileCoord& c) {
    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* B = (const uint16_t*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * a.b_gstride : 0);
    if (LA == KC) {
      // rows m0 .. m_end-1, K = lda
      const int nrows = min(c.m_end - c.m0, BM);
      ra_base = A + (int64_t)c.m0 * a.lda;
      ra_bytes = (uint32_t)(nrows * a.lda * 2);
      pa.plan_kc(a.lda, [&](int r) { return r < nrows ? r : -1; }, dw);
    } else {
      // K-rows k_begin .. k_end-1, columns m0 ..
      ra_base = A + (int64_t)c.k_begin * a.lda;
      ra_bytes = (uint32_t)((int64_t)(c.k_end - c.k_begin) * a.lda * 2);
      pa.plan_mc(a.lda, c.m0, dw);
    }
    const int nt = c.n0;
    if (LB == KC) {
      rb_base = B;
      rb_bytes = (uint32_t)((int64_t)a.b_next * a.ldb * 2);
      pb.plan_kc(a.ldb, [&](int r) {
        int g;
        if constexpr (Epi::kPaired) g = Epi::template b_row_paired<BN, WN>(ep, nt, r);
        else g = nt * BN + r;
        return g < a.b_next ? g : -1;
      }, dw);
    } else {
      const int b_kend = (MODE == RAGGED_K) ? c.k_end : min(c.k_end, a.b_kend);
      rb_base = B + (int64_t)c.k_begin * a.ldb;
      rb_bytes = (uint32_t)((int64_t)max(b_kend - c.k_begin, 0) * a.ldb * 2);
      pb.plan_mc(a.ldb, nt * BN, dw);
    }
    // K-contiguous operands start at the tile's first K (a split-K part's;
    // row-contiguous ones have it in their base)
    soa = LA == KC ? (uint32_t)(c.k_begin * 2) : 0u;
    sob = LB == KC ? (uint32_t)(c.k_begin * 2) : 0u;
    if constexpr (MX) {
      // lane q = (i ND + w) 64 + lane of instruction i of DMA wave w fetches
      // the slice's scale word of tile row q (A) or of B row q (its weight
      // row), or nothing (an offset outside the range); fp4: word q & 1 of row
      // q >> 1.  In the grouped layout the words of consecutive rows are
      // adjacent: a slice's words for a tile are a few contiguous lines.
      const int nrows = min(c.m_end - c.m0, BM);
      rsa_base = s.A_s;
      rsa_bytes = (uint32_t)(s.a_rows * nb);
      rsb_base = s.B_s + (MODE == RAGGED_M ? (int64_t)c.g * s.b_s_gstride : 0);
      rsb_bytes = (uint32_t)(s.b_rows * nb);
#pragma unroll
      for (int i = 0; i < C::SC_A; ++i) {
        const int q = (i * C::ND + dw) * 64 + lane;
        const int qr = FP4 ? q >> 1 : q;
        const uint32_t ga = FP4 ? (uint32_t)(q & 1) * (uint32_t)s.a_rows * 4 : 0u;
        sa_off[i] = qr < nrows ? (uint32_t)((c.m0 + qr) * 4) + ga : kOffRange;
      }
#pragma unroll
      for (int i = 0; i < C::SC_B; ++i) {
        const int q = (i * C::ND + dw) * 64 + lane;
        const int qr = FP4 ? q >> 1 : q;
        const uint32_t gb = FP4 ? (uint32_t)(q & 1) * (uint32_t)s.b_rows * 4 : 0u;
        int g = -1;
        if (qr < BN) {
          if constexpr (Epi::kPaired) g = Epi::template b_row_paired<BN, WN>(ep, nt, qr);
          else g = nt * BN + qr;
        }
        sb_off[i] = (g >= 0 && g < a.b_next) ? (uint32_t)(g * 4) + gb : kOffRange;
      }
      // the tile's first slice: group (k_begin / BK) * kWordsPerSlice
      const uint32_t g0 = (uint32_t)(c.k_begin / BK) * kWordsPerSlice;
      sosa = g0 * (uint32_t)s.a_rows * 4;
      sosb = g0 * (uint32_t)s.b_rows * 4;
    }
  };
  // MX: a slice's scale words are fetched before its codes (the gathers of
  // the scale lines otherwise complete last, and the wait for the slice waits
  // for them: DeepSeek-V3 SwiGLU forward 1.92 -> 1.81 ms on one box)
  auto issue = [&](int stage) {
    const uint32_t sbase = lds0 + stage * C::STAGE_BYTES;
    if constexpr (MX) {
#if defined(__HIP_DEVICE_COMPILE__)
      const uint32_t sc = sbase + C::A_BYTES + C::B_BYTES;
#pragma unroll
      for (int i = 0; i < C::SC_A; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(rsa_base, rsa_bytes),
                                                 (MOE_LDS void*)(uintptr_t)(sc + (i * C::ND + dw) * 64 * 4), 4,
                                                 sa_off[i], sosa, 0, 0);
#pragma unroll
      for (int i = 0; i < C::SC_B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(rsb_base, rsb_bytes),
                                                 (MOE_LDS void*)(uintptr_t)(sc + (C::SC_WORDS + (i * C::ND + dw) * 64) * 4),
                                                 4, sb_off[i], sosb, 0, 0);
#endif
      sosa += kWordsPerSlice * (uint32_t)s.a_rows * 4;   // the next slice's group(s)
      sosb += kWordsPerSlice * (uint32_t)s.b_rows * 4;
    }
    pa.issue(ra_base, ra_bytes, soa, sbase, dw);
    pb.issue(rb_base, rb_bytes, sob, sbase + C::A_BYTES, dw);
    soa += stride_a;
    sob += stride_b;
  };

  FragPlan<LA, BM, FM> fa;
  FragPlan<LB, BN, FN> fb;
  fa.init(wm * (BM / WM));
  fb.init(wn * (BN / WN));

  floatx16 acc[FM][FN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  };

  // Staged epilogue (bf16 stores): the wave's sub-tile goes out in units of
  // 32 rows x 64 columns, each written to a 4 KB LDS buffer of its own (8-byte
  // pieces, swizzled 128-byte rows) and read back as 16-byte row pieces, so
  // that every store writes whole 128-byte row segments.  The buffers lie in
  // the stage of the tile's last slice, which no DMA targets before the next
  // slice's barrier; a barrier first lets every wave finish reading it.  Stores
  // go through a buffer resource over the tile's valid rows (columns past N
  // get an offset outside it), so every lane issues kEpiStores of them.
  static_assert(!Epi::kStaged || (FN % 2 == 0 && C::NW * 4096 <= C::STAGE_BYTES), "staged epilogue");
  constexpr int kEpiStores = Epi::kStaged ? FM * (FN / 2) * 4 : 0;
  auto epilogue_staged = [&](const TileCoord& c, uint32_t stage_byte) {
    if constexpr (Epi::kStaged) {
      bar();
      const int rows = min(c.m_end - c.m0, BM);
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(ep.C + c.g * ep.c_gstride + (int64_t)c.m0 * ep.ldc, (uint32_t)(rows * ep.ldc * 2));
      MOE_LDS u32x2* w2 = (MOE_LDS u32x2*)(uintptr_t)(stage_byte + wave * 4096);
      const MOE_LDS u32x4* r4 = (const MOE_LDS u32x4*)(uintptr_t)(stage_byte + wave * 4096);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp) {
          const int row = lane & 31;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int j = jp * 2 + jj, chunk = jj * 4 + q;
              const u32x2 v = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                               pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
              w2[(row * 8 + (chunk ^ stage_swz(row))) * 2 + (lane >> 5)] = v;
            }
          const int col = c.n0 * BN + wn * (BN / WN) + jp * 64 + (lane & 7) * 8;
          const uint32_t col_off = col + 8 <= ep.N ? (uint32_t)col * 2 : kOffRange;
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int rr = it * 8 + (lane >> 3), cc = lane & 7;
            const u32x4 v = r4[rr * 8 + (cc ^ stage_swz(rr))];
            const uint32_t off = col_off + (uint32_t)((wm * (BM / WM) + i * 32 + rr) * ep.ldc * 2);
            store_b128<MODE == RAGGED_K>(v, rs, off);
          }
        }
    }
  };

  // epilogue: row = lane%32 of the block, columns 8*(e/4) + 4*(lane/32) + 0..3.
  // Epilogues with a row reduction (kRowDot: the folded-gate gradient) return
  // a term per 4-column vector; a row's terms over the wave's 64 columns are
  // summed in a fixed order (j, q, then the lane pair l, l + 32) into one
  // partial per row and 64-column block.
  static_assert(!Epi::kRowDot || BN / WN == 64, "row partials cover 64 columns per wave");
  auto epilogue = [&](const TileCoord& c) {
    const int nt = c.n0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = c.m0 + wm * (BM / WM) + i * 32 + (lane & 31);
      if constexpr (Epi::kRowDot) {
        float dot = 0.0f;
        if (row < c.m_end) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            // the values as stored (bf16 pairs), for the MX row form of block
            // j (32 columns); only the MX kernels form it
            uint32_t qh[8], qu[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = nt * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
              if constexpr (Epi::kQuant && MX) {
                float dh[4], du[4];
                dot += Epi::at4(ep, c.g, row, col, v, dh, du);
                qh[2 * q] = pack_bf16x2(dh[0], dh[1]);
                qh[2 * q + 1] = pack_bf16x2(dh[2], dh[3]);
                qu[2 * q] = pack_bf16x2(du[0], du[1]);
                qu[2 * q + 1] = pack_bf16x2(du[2], du[3]);
              } else {
                dot += Epi::at4(ep, c.g, row, col, v);
              }
            }
            if constexpr (Epi::kQuant && MX) {
              // (both lanes of a row's pair are here: the row decides)
              const int col0 = nt * BN + wn * (BN / WN) + j * 32;
              if (ep.q_codes && col0 < ep.f) Epi::quant_block(ep, row, col0, qh, qu);
            }
          }
        }
        if (ep.dg_part) {                       // uniform: every lane reaches the shuffle
          dot += __shfl_xor(dot, 32, 64);
          // a tile wider than the rest of the row leaves blocks past its end
          // (dg_ld blocks per row) to no one
          const int blk = (nt * BN + wn * (BN / WN)) / 64;
          if (row < c.m_end && lane < 32 && blk < ep.dg_ld) ep.dg_part[(int64_t)row * ep.dg_ld + blk] = dot;
        }
        continue;
      }
      if (row >= c.m_end) continue;
      if constexpr (Epi::kAccum) {
        float old[FN][4][4];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            Epi::old4(ep, c.g, row, nt * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4, old[j][q]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
            Epi::add4(ep, c.g, row, nt * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4, v, old[j][q]);
          }
        continue;
      }
      if constexpr (Epi::kPaired) {
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          uint32_t qa[8];                       // act as stored (bf16 pairs), for the MX row form
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nt * (BN / 2) + wn * (BN / WN / 2) + j * 32 + q * 8 + (lane >> 5) * 4;
            float h[4], u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              h[e] = acc[i][j][4 * q + e];
              u[e] = acc[i][j + FN / 2][4 * q + e];
            }
            if constexpr (Epi::kQuant && MX) {
              float a[4];
              Epi::at_pair4(ep, row, col, h, u, a);
              qa[2 * q] = pack_bf16x2(a[0], a[1]);
              qa[2 * q + 1] = pack_bf16x2(a[2], a[3]);
            } else {
              Epi::at_pair4(ep, row, col, h, u);
            }
          }
          if constexpr (Epi::kQuant && MX) {
            const int col0 = nt * (BN / 2) + wn * (BN / WN / 2) + j * 32;
            if (ep.q_codes && col0 < ep.f) Epi::quant_block(ep, row, col0, qa);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nt * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
            Epi::at4(ep, c.g, row, col, v);
          }
        }
      }
    }
  };

  // microscaled MFMAs of one slice (codes at sa, sb; scale words after B's)
  auto mx_slice = [&](uint32_t sa, uint32_t sb) {
    if constexpr (MX && FP4) {
      // four 64-deep steps per slice (32 bytes of a row each); lane half h
      // takes 16-byte chunk 2 st + h of its row -- the 32 values of block h
      // of the step -- and passes the scale of that block: byte 2 st + h of
      // the row's two scale words
      const int h = lane >> 5;
      const uint32_t sc = sb + C::B_BYTES;
      u32x2 wa[FM], wb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        wa[i] = *(const MOE_LDS u32x2*)(uintptr_t)(sc + (wm * (BM / WM) + i * 32 + (lane & 31)) * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wb[j] = *(const MOE_LDS u32x2*)(uintptr_t)(sc + C::SC_WORDS * 4 + (wn * (BN / WN) + j * 32 + (lane & 31)) * 8);
      auto chunk = [&](uint32_t base, int row, int c) -> i32x8 {
        const u32x4 v = *(const MOE_LDS u32x4*)(uintptr_t)(base + row * 128 + ((c ^ kc_swz(row)) * 16));
        return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};   // e2m1 uses the low four
      };
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        i32x8 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = chunk(sa, wm * (BM / WM) + i * 32 + (lane & 31), 2 * st + h);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = chunk(sb, wn * (BN / WN) + j * 32 + (lane & 31), 2 * st + h);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int sa_w = (int)(wa[i][st >> 1] >> (8 * h)), sb_w = (int)(wb[j][st >> 1] >> (8 * h));
            if ((st & 1) == 0)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 4, 4, 0, sb_w,
                                                                          0, sa_w);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 4, 4, 2, sb_w,
                                                                          2, sa_w);
          }
      }
    }
    if constexpr (MX && !FP4) {
      // two 64-deep steps per slice; lane half h takes 16-byte chunks
      // 4 st + h and 4 st + 2 + h of its row and passes the scale of block h
      const int h = lane >> 5;
      const uint32_t sc = sb + C::B_BYTES;
      uint32_t wa[FM], wb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        wa[i] = *(const MOE_LDS uint32_t*)(uintptr_t)(sc + (wm * (BM / WM) + i * 32 + (lane & 31)) * 4) >> (8 * h);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        wb[j] = *(const MOE_LDS uint32_t*)(uintptr_t)(sc + C::SC_WORDS * 4 +
                                                      (wn * (BN / WN) + j * 32 + (lane & 31)) * 4) >> (8 * h);
      auto chunk = [&](uint32_t base, int row, int c) -> u32x4 {
        return *(const MOE_LDS u32x4*)(uintptr_t)(base + row * 128 + ((c ^ kc_swz(row)) * 16));
      };
      auto frag = [&](uint32_t base, int row, int st) -> i32x8 {
        const u32x4 lo = chunk(base, row, st * 4 + h), hi = chunk(base, row, st * 4 + 2 + h);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      // step 1's fragments go to a second register set, read before step 0's
      // MFMAs so that the LDS reads can overlap them (iglp_opt(0) below lets
      // the scheduler interleave the two)
      i32x8 af[2][FM], bfr[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[0][i] = frag(sa, wm * (BM / WM) + i * 32 + (lane & 31), 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[0][j] = frag(sb, wn * (BN / WN) + j * 32 + (lane & 31), 0);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st == 0) {
#pragma unroll
          for (int i = 0; i < FM; ++i) af[1][i] = frag(sa, wm * (BM / WM) + i * 32 + (lane & 31), 1);
#pragma unroll
          for (int j = 0; j < FN; ++j) bfr[1][j] = frag(sb, wn * (BN / WN) + j * 32 + (lane & 31), 1);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if (st == 0)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][j], af[0][i], acc[i][j], 0, 0, 0,
                                                                          (int)wb[j], 0, (int)wa[i]);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][j], af[1][i], acc[i][j], 0, 0, 2,
                                                                          (int)wb[j], 2, (int)wa[i]);
          }
      }
      __builtin_amdgcn_iglp_opt(0);
    }
  };

  // bf16 MFMAs of one slice (stage at sa, sb), fragments of K-step kk + 1
  // read while the MFMAs of step kk run
  auto mma_slice = [&](uint32_t sa, uint32_t sb) {
    bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = fa.read(sa, i, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = fb.read(sb, j, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[cur ^ 1][i] = fa.read(sa, i, kk + 1);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[cur ^ 1][j] = fb.read(sb, j, kk + 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
    }
    sched_pipelined_slice<FM * (LA == KC ? 1 : 2) + FN * (LB == KC ? 1 : 2), FM * FN>();
  };

  if constexpr (WS) {
    // Separate loops per role over the same tile / slice sequence, meeting at
    // the same barriers: one per slice, and the staged epilogue's.
    SliceIter cur;
    settle(0, cur);
    if (cur.r < 0) return;
    if (is_load) {
      SliceIter ld = cur;
      plan_tile(ld.c);
      auto advance = [&]() {
        if (++ld.ks >= ld.nk) {
          settle(ld.r + 1, ld);
          if (ld.r >= 0) plan_tile(ld.c);
        }
      };
      int issued = 0;
#pragma unroll
      for (int st = 0; st < STAGES - 1; ++st)
        if (ld.r >= 0) {
          issue(st);
          advance();
          ++issued;
        }
      int n = 0;
      do {
        for (int ks = 0; ks < cur.nk; ++ks, ++n) {
          wait_slices_after<STAGES - 2, DMA_PER_SLICE>(issued - n - 1);
          bar();
          if (ld.r >= 0) {
            issue(issued % STAGES);   // the stage multiplied in the previous iteration
            advance();
            ++issued;
          }
        }
        if constexpr (Epi::kStaged) bar();   // the staged epilogue's barrier
        settle(cur.r + 1, cur);
      } while (cur.r >= 0);
      return;
    }
    int n = 0;
    do {
      zero_acc();
      for (int ks = 0; ks < cur.nk; ++ks, ++n) {
        bar();
        const uint32_t sa = lds0 + (n % STAGES) * C::STAGE_BYTES;
        if constexpr (MX) mx_slice(sa, sa + C::A_BYTES);
        else if (cur.c.m0 + wm * (BM / WM) < cur.c.m_end) mma_slice(sa, sa + C::A_BYTES);
      }
      if constexpr (Epi::kStaged) epilogue_staged(cur.c, lds0 + ((n - 1) % STAGES) * C::STAGE_BYTES);
      else epilogue(cur.c);
      settle(cur.r + 1, cur);
    } while (cur.r >= 0);
    return;
  }

  SliceIter comp, ld;
  settle(0, comp);
  if (comp.r < 0) return;
  ld = comp;
  plan_tile(ld.c);

  auto advance_ld = [&]() {
    if (++ld.ks >= ld.nk) {
      settle(ld.r + 1, ld);
      if (ld.r >= 0) plan_tile(ld.c);
    }
  };

  // epilogues run so far, and that count when each ring stage's slice was
  // issued: the staged epilogue's stores issued after a slice's DMA are
  // counted exactly in the wait for that slice
  int epis = 0;
  int epis_at[STAGES];
  // prologue: the first STAGES-1 slices
  int issued = 0;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    epis_at[s] = 0;
    if (ld.r >= 0) {
      issue(s);
      advance_ld();
      ++issued;
    }
  }
  int n = 0;                      // index of the slice being multiplied
  // tile loop around a slice loop: the accumulators are only touched by MFMAs
  // inside the slice loop, so they stay in place across it
  do {
    zero_acc();
    for (int ks = 0; ks < comp.nk; ++ks, ++n) {
      // wait for slice n: the DMA of the slices issued after it may stay in
      // flight.  Vector memory operations complete in issue order, so the
      // epilogue's stores and loads (issued after every DMA in flight) only
      // make this wait more conservative, never too short.
      if constexpr (Epi::kStaged)
        wait_vmcnt_dyn<0, 63>((issued - n - 1) * DMA_PER_SLICE + (epis - epis_at[n % STAGES]) * kEpiStores);
      else
        wait_slices_after<STAGES - 2, DMA_PER_SLICE>(issued - n - 1);
      bar();
      if (ld.r >= 0) {
        epis_at[issued % STAGES] = epis;
        issue(issued % STAGES);   // the stage multiplied in the previous iteration
        advance_ld();
        ++issued;
      }
      const uint32_t sa = lds0 + (n % STAGES) * C::STAGE_BYTES;
      const uint32_t sb = sa + C::A_BYTES;
      if constexpr (MX) mx_slice(sa, sb);
      if constexpr (!MX) {
        // A wave whose rows of the tile all lie past m_end (the padding of an
        // expert's last tile) skips its reads and MFMAs, which leaves the
        // MFMA pipe to the waves of other workgroups on its SIMD.  Fragments
        // of K-step kk + 1 are read while the MFMAs of step kk run (two
        // register sets), in the order the scheduling groups fix.
        if (comp.c.m0 + wm * (BM / WM) < comp.c.m_end) {
          bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) af[0][i] = fa.read(sa, i, 0);
#pragma unroll
          for (int j = 0; j < FN; ++j) bfr[0][j] = fb.read(sb, j, 0);
#pragma unroll
          for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16) {
#pragma unroll
              for (int i = 0; i < FM; ++i) af[cur ^ 1][i] = fa.read(sa, i, kk + 1);
#pragma unroll
              for (int j = 0; j < FN; ++j) bfr[cur ^ 1][j] = fb.read(sb, j, kk + 1);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
          }
          sched_pipelined_slice<FM * (LA == KC ? 1 : 2) + FN * (LB == KC ? 1 : 2), FM * FN>();
        }
      }
    }
    if constexpr (Epi::kStaged) {
      epilogue_staged(comp.c, lds0 + ((n - 1) % STAGES) * C::STAGE_BYTES);
      ++epis;
    } else {
      epilogue(comp.c);
    }
    settle(comp.r + 1, comp);
  } while (comp.r >= 0);
}

}  // namespace moe
