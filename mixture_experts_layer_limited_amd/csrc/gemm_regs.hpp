// bf16 MFMA grouped-GEMM kernel for gfx950, persistent and register-pipelined:
// it runs the router's weight gradient.
//
// The grid holds two workgroups per CU (256 threads in 2x2 waves, each wave
// owning 64x64 of a 128x128 tile as 2x2 blocks of 32x32 accumulators,
// v_mfma_f32_32x32x16_bf16).
// Global loads of slice k+1 go to registers while slice k is multiplied from
// LDS.  K-contiguous operand rows hold 64 bf16 = eight 16-byte chunks, chunk c
// of row r at position c ^ ((r ^ (r >> 3)) & 7): fragment reads (16
// consecutive rows per cycle on gfx950's 64 banks) and 16-byte writes stay
// free of bank conflicts.  Row-contiguous operands ("MC": both operands of a
// weight gradient) are kept in LDS as they lie in memory and read with
// transposing LDS reads (McFrag).
//
// The MFMA takes the B fragment first, so a lane's accumulator holds four
// consecutive output columns (element e of a block: column 8*(e/4) +
// 4*(lane/32) + e%4, row lane%32) and the epilogue stores 4-column vectors.
#pragma once

#include <type_traits>

#include "gemm.hpp"

namespace moe {

// rows of CH 16-byte chunks: chunk c of row r sits at c ^ ((r ^ (r >> 3)) & (CH - 1))
template <int CH>
__device__ __forceinline__ int rswz_t(int row, int c) { return row * CH + (c ^ ((row ^ (row >> 3)) & (CH - 1))); }

// Global -> register -> LDS staging of one operand slice: ROWS tile rows x BK
// K values (CH = BK / 8 chunks per LDS row).  KC operands load 16 K values of
// one row per lane; MC operands load 4 K-rows x 8 columns per block and
// transpose them on the way to LDS.
template <OpLayout L, int ROWS, int NTHR, int BK = 64>
struct RegLoader {
  static constexpr int CH = BK / 8;
  static constexpr int NB = ROWS / 8, KB = BK / 4;          // MC blocks: 8 columns x 4 K-rows
  static constexpr int NKC = ROWS * CH / NTHR;
  static constexpr int NMC = NB * KB / NTHR;
  static constexpr int NREG = (L == KC) ? NKC : 4 * NMC;
  static_assert(NKC * NTHR == ROWS * CH && NMC * NTHR == NB * KB, "loader split");
  u32x4 r[NREG];

  // block q of an MC slice: column block nb, K-row group kb.  With 8-chunk
  // rows, 8 lanes take 8 column blocks of the same K-rows; with 16-chunk rows
  // 16 lanes take a whole 256-byte K-row piece
  __device__ __forceinline__ static void mc_block(int q, int& nb, int& kb) {
    if constexpr (CH == 8) {
      nb = ((q >> 7) << 3) | (q & 7);
      kb = (q >> 3) & 15;
    } else {
      nb = q % NB;
      kb = q / NB;
    }
  }

  // KC: element (i, k) at base[i * ld + k]; rowv(i) = absolute row or -1; k < kend
  template <class RowFn>
  __device__ __forceinline__ void load_kc(const uint16_t* base, int64_t ld, int k0, int kend, RowFn rowv) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      int q = threadIdx.x + i * NTHR;
      int kk = k0 + (q % CH) * 8;
      int gi = rowv(q / CH);
      u32x4 v = {0, 0, 0, 0};
      if (gi >= 0 && kk < kend) v = *(const u32x4*)(base + (int64_t)gi * ld + kk);
      r[i] = v;
    }
  }
  // MC: element (i, k) at base[k * ld + i]; 8-column groups valid iff i + 8 <= iext; rows k < kend
  __device__ __forceinline__ void load_mc(const uint16_t* base, int64_t ld, int k0, int kend, int i0, int iext) {
#pragma unroll
    for (int b = 0; b < NMC; ++b) {
      int nb, kb;
      mc_block(threadIdx.x + b * NTHR, nb, kb);
      int i = i0 + nb * 8;
      bool ok = i + 8 <= iext;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int kk = k0 + kb * 4 + rr;
        u32x4 v = {0, 0, 0, 0};
        if (ok && kk < kend) v = *(const u32x4*)(base + (int64_t)kk * ld + i);
        r[b * 4 + rr] = v;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* s) const {
    if (L == KC) {
#pragma unroll
      for (int i = 0; i < NKC; ++i) {
        int q = threadIdx.x + i * NTHR;
        s[rswz_t<CH>(q / CH, q % CH)] = r[i];
      }
    } else {
      u32x2* s2 = (u32x2*)s;
#pragma unroll
      for (int b = 0; b < NMC; ++b) {
        int nb, kb;
        mc_block(threadIdx.x + b * NTHR, nb, kb);
        const u32x4* r4 = &r[b * 4];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          int w = m >> 1;
          uint32_t e0, e1, e2, e3;
          if (m & 1) {
            e0 = r4[0][w] >> 16; e1 = r4[1][w] >> 16; e2 = r4[2][w] >> 16; e3 = r4[3][w] >> 16;
          } else {
            e0 = r4[0][w] & 0xFFFFu; e1 = r4[1][w] & 0xFFFFu; e2 = r4[2][w] & 0xFFFFu; e3 = r4[3][w] & 0xFFFFu;
          }
          u32x2 o = {e0 | (e1 << 16), e2 | (e3 << 16)};
          s2[rswz_t<CH>(nb * 8 + m, kb >> 1) * 2 + (kb & 1)] = o;
        }
      }
    }
  }
};

// Row-contiguous operand slice kept as it lies in memory (the layout McFrag
// reads): BK K-rows x ROWS columns, one 16-byte piece of a K-row per lane and
// load, no transposition in registers.
template <int ROWS, int NTHR, int BK>
struct McLoader {
  static constexpr int CPR = ROWS / 8;
  static constexpr int N = BK * CPR / NTHR;
  static_assert(N * NTHR == BK * CPR, "loader split");
  u32x4 r[N];

  // element (i, k) at base[k * ld + i]; columns i0 + 8c .. +7 valid iff
  // i0 + 8c + 8 <= iext; K-rows k0 + k < kend
  __device__ __forceinline__ void load_mc(const uint16_t* base, int64_t ld, int k0, int kend, int i0, int iext) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int q = threadIdx.x + j * NTHR;
      const int k = q / CPR, c = q % CPR;
      const int i = i0 + c * 8, kk = k0 + k;
      u32x4 v = {0, 0, 0, 0};
      if (i + 8 <= iext && kk < kend) v = *(const u32x4*)(base + (int64_t)kk * ld + i);
      r[j] = v;
    }
  }
  __device__ __forceinline__ void store(u32x4* s) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int q = threadIdx.x + j * NTHR;
      const int k = q / CPR, c = q % CPR;
      s[k * CPR + (c ^ mc_mask(k, c))] = r[j];
    }
  }
};

// ---------------------------------------------------------------------------
// Schedule.
//
// The grid holds as many workgroups as fit on the chip (two per CU: their LDS,
// and registers capped at 256 per lane so two waves share a SIMD); the
// workgroups of each XCD stride through one contiguous run of the logical tiles
// (xcd_run_start).  The ragged offsets and tile prefix are copied to LDS once,
// so finding a tile costs no global-memory round trip.  Loads walk the flat
// sequence of (tile, K-slice) pairs one slice ahead of the multiply, crossing
// tile boundaries.  On a tile's last slice the epilogue runs before the
// prefetched slice is written to LDS: the loads of the next tile are issued
// before the epilogue's stores, so waiting for them never waits for the
// stores (vector memory operations complete in issue order), and their
// latency overlaps the multiply and the epilogue.
//
// Two-byte outputs of plain stores are staged through the LDS stage that the
// prefetched slice will fill: each wave writes its 64x64 sub-tile there and
// stores it back 8 columns (16 bytes) per lane, 128 contiguous bytes per row
// (non-temporal for weight gradients, whose output stream would otherwise push
// the operand panels out of L2).
// ---------------------------------------------------------------------------
// BK = 64: two LDS stages (the store of slice n+1 goes to the stage not being
// read).
template <int BK_>
struct PipeCfg {
  static constexpr int BM = 128, BN = 128, WM = 2, WN = 2, BK = BK_, NTHR = 256;
  static constexpr int FM = 2, FN = 2, CH = BK / 8;
  static constexpr int NSTAGE = 2;
  static constexpr int STAGE = (BM + BN) * CH;             // 16-byte chunks per stage
  static constexpr int OFF_INTS = kMaxExperts + 1;
  static constexpr int LDS_BYTES = NSTAGE * STAGE * 16 + 2 * OFF_INTS * 4;
  static_assert(BK == 64, "slice depth");
};

// barrier for LDS traffic only: wait for this wave's LDS operations, then meet
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


template <OpLayout LA, OpLayout LB, GemmMode MODE, class Epi, int BK_>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_pipe_kernel(GemmArgs a, typename Epi::P ep, int NT, int MT) {
  using C = PipeCfg<BK_>;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, BK = C::BK, NTHR = C::NTHR;
  constexpr int FM = C::FM, FN = C::FN, CH = C::CH, NSTAGE = C::NSTAGE;
  extern __shared__ u32x4 smem[];
  int* s_off = (int*)(smem + NSTAGE * C::STAGE);
  int* s_pre = s_off + C::OFF_INTS;

  if (MODE != DENSE && a.offsets)
    for (int i = threadIdx.x; i <= a.G; i += NTHR) s_off[i] = a.offsets[i];
  if (MODE == RAGGED_M)
    for (int i = threadIdx.x; i <= a.G; i += NTHR) s_pre[i] = a.tile_prefix[i];
  __syncthreads();
  const int total = (MODE == RAGGED_M) ? s_pre[a.G] * NT : total_tiles<MODE>(a, NT, MT);
  const int G = gridDim.x, b = blockIdx.x;
  const int X = G < 8 ? G : 8, xcd = b % X, wi = b / X, nx = (G - xcd + X - 1) / X;
  const int run_lo = xcd_run_start<MODE>(a, s_off, total, MT * NT, xcd, X);
  const int run_hi = xcd_run_start<MODE>(a, s_off, total, MT * NT, xcd + 1, X);

  struct It {
    int r;         // step of the tile in this workgroup's stride (-1: done)
    int ks, nk;    // slice within the tile, slices of the tile
    TileCoord c;
  };
  // first step >= r with a tile of this workgroup that has a contraction
  // (tiles without one are zero-filled by the caller)
  auto settle = [&](int r, It& it) {
    for (;; ++r) {
      const int L = run_lo + wi + r * nx;
      if (L >= run_hi) break;
      resolve_tile<MODE, BM>(a, s_off, s_pre, L, NT, MT, it.c);
      it.nk = (it.c.k_end - it.c.k_begin + BK - 1) / BK;
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
  auto advance = [&](It& it) {
    if (++it.ks >= it.nk) settle(it.r + 1, it);
  };

  // K-contiguous operands: rows of CH chunks (rswz_t); row-contiguous ones:
  // the slice as it lies in memory, read with McFrag
  using LdA = std::conditional_t<LA == KC, RegLoader<KC, BM, NTHR, BK>, McLoader<BM, NTHR, BK>>;
  using LdB = std::conditional_t<LB == KC, RegLoader<KC, BN, NTHR, BK>, McLoader<BN, NTHR, BK>>;
  auto load_into = [&](LdA& xa, LdB& xb, const It& it) {
    const TileCoord& c = it.c;
    const int k0 = c.k_begin + it.ks * BK;
    const uint16_t* A = (const uint16_t*)a.A;
    const uint16_t* B = (const uint16_t*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * a.b_gstride : 0);
    if constexpr (LA == KC) {
      xa.load_kc(A, a.lda, k0, c.k_end, [&](int r) -> int { int g = c.m0 + r; return g < c.m_end ? g : -1; });
    } else {
      xa.load_mc(A, a.lda, k0, c.k_end, c.m0, a.a_mext);
    }
    const int nt = c.n0;
    if constexpr (LB == KC) {
      xb.load_kc(B, a.ldb, k0, c.k_end, [&](int r) -> int {
        int g;
        if constexpr (Epi::kPaired) g = Epi::template b_row_paired<BN, WN>(ep, nt, r);
        else g = nt * BN + r;
        return g < a.b_next ? g : -1;
      });
    } else {
      const int b_kend = (MODE == RAGGED_K) ? c.k_end : min(c.k_end, a.b_kend);
      xb.load_mc(B, a.ldb, k0, b_kend, nt * BN, a.b_next);
    }
  };
  auto store_stage = [&](const LdA& xa, const LdB& xb, int stage) {
    u32x4* st = smem + stage * C::STAGE;
    xa.store(st);
    xb.store(st + BM * CH);
  };
  auto stage_of = [](int slice) { return slice & 1; };

  It comp, ld;
  settle(0, comp);
  if (comp.r < 0) return;
  ld = comp;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * (BM / WM) + (lane & 31);
  const int brow0 = wn * (BN / WN) + (lane & 31);
  McFrag<BM, FM> mfa;
  McFrag<BN, FN> mfb;
  if (LA == MC) mfa.init(wm * (BM / WM));
  if (LB == MC) mfb.init(wn * (BN / WN));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(MOE_LDS void*)smem;

  LdA la;
  LdB lb;
  // prologue: slice 0 into LDS stage 0
  load_into(la, lb, ld);
  advance(ld);
  store_stage(la, lb, 0);
  lds_barrier();

  floatx16 acc[FM][FN];

  auto epilogue = [&](const TileCoord& c, int stage) {
    if constexpr (Epi::kStaged) {
      // this wave's 64x64 sub-tile as bf16 rows of 128 bytes in `stage`
      u32x2* w2 = (u32x2*)(smem + stage * C::STAGE + wave * 512);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = i * 32 + (lane & 31), chunk = j * 4 + q;
            const u32x2 v = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                             pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
            w2[(row * 8 + (chunk ^ stage_swz(row))) * 2 + (lane >> 5)] = v;
          }
      // stored through a buffer resource over the tile's valid rows; lanes of
      // columns past N get an offset outside it.  Every lane issues the same
      // stores, so the wait for the prefetched slice counts them exactly.
      // (The launcher only picks this kernel for 16-byte aligned rows.)
      const u32x4* r4 = (const u32x4*)w2;
      const int rows = min(c.m_end - c.m0, BM);
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(ep.C + c.g * ep.c_gstride + (int64_t)c.m0 * ep.ldc, (uint32_t)(rows * ep.ldc * 2));
      const int col = c.n0 * BN + wn * (BN / WN) + (lane & 7) * 8;
      const uint32_t col_off = col + 8 <= ep.N ? (uint32_t)col * 2 : 0x80000000u;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rr = it * 8 + (lane >> 3), cc = lane & 7;
        const u32x4 v = r4[rr * 8 + (cc ^ stage_swz(rr))];
        const uint32_t off = col_off + (uint32_t)((wm * (BM / WM) + rr) * ep.ldc * 2);
        store_b128<MODE == RAGGED_K>(v, rs, off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = c.m0 + wm * (BM / WM) + i * 32 + (lane & 31);
        if (row >= c.m_end) continue;
        if constexpr (Epi::kPaired) {
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = c.n0 * (BN / 2) + wn * (BN / WN / 2) + j * 32 + q * 8 + (lane >> 5) * 4;
              float h[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              float u[4] = {acc[i][j + FN / 2][4 * q], acc[i][j + FN / 2][4 * q + 1],
                            acc[i][j + FN / 2][4 * q + 2], acc[i][j + FN / 2][4 * q + 3]};
              Epi::at_pair4(ep, row, col, h, u);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = c.n0 * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4;
              float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              Epi::at4(ep, c.g, row, col, v);
            }
          }
        }
      }
    }
  };

  // iteration n: load slice n + 1, multiply slice n, store slice n + 1; on a
  // tile's last slice the epilogue comes between the multiply and that store
  int n = 0;
  auto iteration = [&](auto last) {
    bool loaded = false;
    if (ld.r >= 0) {
      load_into(la, lb, ld);
      advance(ld);
      loaded = true;
    }
    const bf16x8* sa = (const bf16x8*)(smem + stage_of(n) * C::STAGE);
    const bf16x8* sb = sa + BM * CH;
    const uint32_t la_byte = lds0 + (uint32_t)(stage_of(n) * C::STAGE * 16);
    const uint32_t lb_byte = la_byte + BM * CH * 16;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (LA == KC) af[i] = sa[rswz_t<CH>(arow0 + i * 32, ch)];
        else af[i] = mfa.read(la_byte, i, kk);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (LB == KC) bfr[j] = sb[rswz_t<CH>(brow0 + j * 32, ch)];
        else bfr[j] = mfb.read(lb_byte, j, kk);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if constexpr (decltype(last)::value) {
      // the stage slice n + 1 goes to is not being read now: stage the tile there
      epilogue(comp.c, stage_of(n + 1));
      if (Epi::kStaged) lds_barrier();   // every wave has read its staged rows
    }
    // stored even when nothing was loaded (the stage is not read again): every
    // path then waits for the loads it issued here, so the compiler never
    // carries them as possibly pending into the next tile, where the first
    // reuse of their registers would wait for everything outstanding,
    // including the epilogue's stores
    store_stage(la, lb, stage_of(n + 1));
    lds_barrier();
    ++n;
  };

  do {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    for (int ks = 0; ks + 1 < comp.nk; ++ks) iteration(std::false_type{});
    iteration(std::true_type{});
    settle(comp.r + 1, comp);
  } while (comp.r >= 0);
}

}  // namespace moe
