// bf16 MFMA grouped-GEMM kernel for gfx950, register-staged variant.
//
// One tile per workgroup (the grid covers every logical tile; surplus
// workgroups of the ragged schedule exit at once), 256 threads in 2x2 waves,
// each wave owning 64x64 of a 128x128 tile as 2x2 blocks of 32x32
// accumulators (v_mfma_f32_32x32x16_bf16), BK = 64.  Global loads of slice
// k+1 go to registers while slice k is multiplied from LDS; two LDS stages, one
// barrier per slice.  Every LDS row holds 64 bf16 = eight 16-byte chunks,
// K-contiguous, chunk c of row r at position c ^ ((r ^ (r >> 3)) & 7): the
// fragment reads (16 consecutive rows per cycle on gfx950's 64 banks), the
// 16-byte K-contiguous writes and the 8-byte transposed writes of
// row-contiguous operands all stay free of bank conflicts.  Row-contiguous
// operands ("MC": the weight in dgrad, both operands in wgrad) are loaded as
// 4 K-rows x 8 columns per thread and transposed in registers on the way in.
//
// Logical tiles are spread with xcd_remap over their exact count, so each XCD
// receives a contiguous run of the expert-major tile order.  The MFMA takes the
// B fragment first, so a lane's accumulator holds four consecutive output
// columns (element e of a block: column 8*(e/4) + 4*(lane/32) + e%4, row
// lane%32) and the epilogue stores 4-column vectors.
#pragma once

#include "gemm.hpp"

namespace moe {

__device__ __forceinline__ int rswz(int row, int c) { return row * 8 + (c ^ ((row ^ (row >> 3)) & 7)); }

struct RegTile {
  static constexpr int BM = 128, BN = 128, WM = 2, WN = 2, BK = 64;
  static constexpr int NTHR = 256;
  static constexpr int FM = 2, FN = 2;
  static constexpr int STAGE = (BM + BN) * 8;              // 16-byte chunks per stage
  static constexpr int LDS_BYTES = 2 * STAGE * 16;
};

template <OpLayout L, int ROWS, int NTHR>
struct RegLoader {
  static constexpr int NKC = ROWS * 8 / NTHR;
  static constexpr int NMC = 16 * (ROWS / 8) / NTHR;
  static constexpr int NREG = (L == KC) ? NKC : 4 * NMC;
  u32x4 r[NREG];

  // KC: element (i, k) at base[i * ld + k]; rowv(i) = absolute row or -1; k < kend
  template <class RowFn>
  __device__ __forceinline__ void load_kc(const uint16_t* base, int64_t ld, int k0, int kend, RowFn rowv) {
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      int q = threadIdx.x + i * NTHR;
      int kk = k0 + (q & 7) * 8;
      int gi = rowv(q >> 3);
      u32x4 v = {0, 0, 0, 0};
      if (gi >= 0 && kk < kend) v = *(const u32x4*)(base + (int64_t)gi * ld + kk);
      r[i] = v;
    }
  }
  // MC: element (i, k) at base[k * ld + i]; 8-column groups valid iff i + 8 <= iext; rows k < kend
  __device__ __forceinline__ void load_mc(const uint16_t* base, int64_t ld, int k0, int kend, int i0, int iext) {
#pragma unroll
    for (int b = 0; b < NMC; ++b) {
      int q = threadIdx.x + b * NTHR;
      int nb = ((q >> 7) << 3) | (q & 7), kb = (q >> 3) & 15;
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
        s[rswz(q >> 3, q & 7)] = r[i];
      }
    } else {
      u32x2* s2 = (u32x2*)s;
#pragma unroll
      for (int b = 0; b < NMC; ++b) {
        int q = threadIdx.x + b * NTHR;
        int nb = ((q >> 7) << 3) | (q & 7), kb = (q >> 3) & 15;
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
          s2[rswz(nb * 8 + m, kb >> 1) * 2 + (kb & 1)] = o;
        }
      }
    }
  }
};

template <OpLayout LA, OpLayout LB, GemmMode MODE, class Epi>
__global__ __launch_bounds__(256) void gemm_regs_kernel(GemmArgs a, typename Epi::P ep, int NT, int MT) {
  using C = RegTile;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, BK = C::BK, NTHR = C::NTHR;
  constexpr int FM = C::FM, FN = C::FN;
  extern __shared__ u32x4 smem[];

  const int total = total_tiles<MODE>(a, NT, MT);
  if ((int)blockIdx.x >= total) return;
  TileCoord c;
  resolve_tile<MODE, BM>(a, xcd_remap(blockIdx.x, total), NT, MT, c);
  if (c.m0 >= c.m_end) return;              // only a mismatched tile prefix could produce this
  const int nt = c.n0;

  const uint16_t* __restrict__ A = (const uint16_t*)a.A;
  const uint16_t* __restrict__ B = (const uint16_t*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * a.b_gstride : 0);
  const int b_kend = (MODE == RAGGED_K) ? c.k_end : min(c.k_end, a.b_kend);

  RegLoader<LA, BM, NTHR> la;
  RegLoader<LB, BN, NTHR> lb;
  auto a_row = [&](int r) -> int { int g = c.m0 + r; return g < c.m_end ? g : -1; };
  auto b_row = [&](int r) -> int {
    int g;
    if constexpr (Epi::kPaired) g = Epi::template b_row_paired<BN, WN>(ep, nt, r);
    else g = nt * BN + r;
    return g < a.b_next ? g : -1;
  };
  auto load = [&](int k0) {
    if (LA == KC) la.load_kc(A, a.lda, k0, c.k_end, a_row);
    else la.load_mc(A, a.lda, k0, c.k_end, c.m0, a.a_mext);
    if (LB == KC) lb.load_kc(B, a.ldb, k0, c.k_end, b_row);
    else lb.load_mc(B, a.ldb, k0, b_kend, nt * BN, a.b_next);
  };
  auto store = [&](int buf) {
    u32x4* s = smem + buf * C::STAGE;
    la.store(s);
    lb.store(s + BM * 8);
  };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (c.k_end - c.k_begin + BK - 1) / BK;
  if (nk > 0) {
    load(c.k_begin);
    store(0);
  }
  __syncthreads();
  const int arow0 = wm * (BM / WM) + (lane & 31);
  const int brow0 = wn * (BN / WN) + (lane & 31);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(c.k_begin + (kt + 1) * BK);
    const bf16x8* sa = (const bf16x8*)(smem + (kt & 1) * C::STAGE);
    const bf16x8* sb = sa + BM * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = sa[rswz(arow0 + i * 32, ch)];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = sb[rswz(brow0 + j * 32, ch)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  // epilogue: row = lane%32 of the block, columns 8*(e/4) + 4*(lane/32) + 0..3
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = c.m0 + wm * (BM / WM) + i * 32 + (lane & 31);
    if (row >= c.m_end) continue;
    if constexpr (Epi::kPaired) {
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * (BN / 2) + wn * (BN / WN / 2) + j * 32 + q * 8 + (lane >> 5) * 4;
          float h[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          float u[4] = {acc[i][j + FN / 2][4 * q], acc[i][j + FN / 2][4 * q + 1], acc[i][j + FN / 2][4 * q + 2],
                        acc[i][j + FN / 2][4 * q + 3]};
          Epi::at_pair4(ep, row, col, h, u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nt * BN + wn * (BN / WN) + j * 32 + q * 8 + (lane >> 5) * 4;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          Epi::at4(ep, c.g, row, col, v);
        }
      }
    }
  }
}

}  // namespace moe
