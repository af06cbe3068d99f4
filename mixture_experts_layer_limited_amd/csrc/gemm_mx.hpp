// MXFP8 grouped-GEMM kernel for gfx950: fp8 e4m3 operands with one e8m0
// scale per 32 consecutive K values, v_mfma_scale_f32_32x32x64_f8f6f4, fp32
// accumulation, the bf16 path's epilogues.
//
// Both operands are K-contiguous codes ([rows][K] bytes) with scales
// ([rows][K/32] bytes); operands the layer contracts along their row index
// reach the kernel as transposed quantised copies.  K is a multiple of 128.
//
// Tiles and staging follow the register-staged bf16 kernel: 256 threads, a
// 128x128 tile, 2x2 waves of 64x64, two LDS stages, one barrier per slice.  A
// slice is 128 K values = 128 bytes per row, i.e. the same eight 16-byte
// chunks per LDS row (and the same conflict-free swizzle) as a 64-deep bf16
// slice, so the bf16 loader moves it unchanged (in 2-byte units).
//
// Operand layout of the scaled MFMA (32 rows x 64 K per step, 32 bytes per
// lane): lane l (h = l / 32) holds row l % 32, bytes 0-15 = 16 K values of the
// step's first 32-block and bytes 16-31 = 16 K values of its second; lanes l
// and l + 32 together cover each block.  Here lane h takes 16-byte chunks h and
// 2 + h of the step's four.  The scale of (row, block b) comes from lane
// row + 32 b, so each lane passes the scale of block h of its own row; the
// scale word of a row holds the slice's four block scales (K/32 bytes per row,
// a multiple of 4), shifted by 8 h per lane, and op_sel picks byte 2 s for
// step s.
#pragma once

#include "gemm.hpp"
#include "gemm_regs.hpp"

namespace moe {

template <GemmMode MODE, class Epi>
__global__ __launch_bounds__(256) void gemm_mx_kernel(GemmArgs a, MxArgs s, typename Epi::P ep, int NT, int MT) {
  using C = RegTile;
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, NTHR = C::NTHR;
  constexpr int FM = C::FM, FN = C::FN;
  constexpr int BKB = 128;                       // K values (bytes) per slice
  extern __shared__ u32x4 smem[];

  const int total = total_tiles<MODE>(a, NT, MT);
  if ((int)blockIdx.x >= total) return;
  TileCoord c;
  resolve_tile<MODE, BM>(a, xcd_remap(blockIdx.x, total), NT, MT, c);
  if (c.m0 >= c.m_end) return;
  const int nt = c.n0;

  // codes in 2-byte units for the bf16 loader; K, ld and offsets are even
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B = (const uint16_t*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * (a.b_gstride / 2) : 0);
  const uint8_t* Bs = s.B_s + (MODE == RAGGED_M ? (int64_t)c.g * s.b_s_gstride : 0);
  const int64_t lda = a.lda / 2, ldb = a.ldb / 2;

  RegLoader<KC, BM, NTHR> la;
  RegLoader<KC, BN, NTHR> lb;
  auto a_row = [&](int r) -> int { int g = c.m0 + r; return g < c.m_end ? g : -1; };
  auto b_row = [&](int r) -> int {
    int g;
    if constexpr (Epi::kPaired) g = Epi::template b_row_paired<BN, WN>(ep, nt, r);
    else g = nt * BN + r;
    return g < a.b_next ? g : -1;
  };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5;
  // absolute rows whose scales this lane passes (or -1)
  int srow_a[FM], srow_b[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) srow_a[i] = a_row(wm * (BM / WM) + i * 32 + (lane & 31));
#pragma unroll
  for (int j = 0; j < FN; ++j) srow_b[j] = b_row(wn * (BN / WN) + j * 32 + (lane & 31));
  uint32_t sa_next[FM], sb_next[FN];

  auto load = [&](int kb) {             // kb: first K byte of the slice
    la.load_kc(A, lda, kb / 2, c.k_end / 2, a_row);
    lb.load_kc(B, ldb, kb / 2, c.k_end / 2, b_row);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa_next[i] = srow_a[i] >= 0 ? *(const uint32_t*)(s.A_s + srow_a[i] * s.a_s_ld + kb / 32) : 0u;
#pragma unroll
    for (int j = 0; j < FN; ++j)
      sb_next[j] = srow_b[j] >= 0 ? *(const uint32_t*)(Bs + srow_b[j] * s.b_s_ld + kb / 32) : 0u;
  };
  auto store = [&](int buf) {
    u32x4* st = smem + buf * C::STAGE;
    la.store(st);
    lb.store(st + BM * 8);
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (c.k_end - c.k_begin + BKB - 1) / BKB;
  uint32_t sa_cur[FM], sb_cur[FN];
  if (nk > 0) {
    load(c.k_begin);
    store(0);
  }
  __syncthreads();
  const int arow0 = wm * (BM / WM) + (lane & 31);
  const int brow0 = wn * (BN / WN) + (lane & 31);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int i = 0; i < FM; ++i) sa_cur[i] = sa_next[i] >> (8 * h);
#pragma unroll
    for (int j = 0; j < FN; ++j) sb_cur[j] = sb_next[j] >> (8 * h);
    if (kt + 1 < nk) load(c.k_begin + (kt + 1) * BKB);
    const u32x4* sa = smem + (kt & 1) * C::STAGE;
    const u32x4* sb = sa + BM * 8;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      i32x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const u32x4 lo = sa[rswz(arow0 + i * 32, st * 4 + h)];
        const u32x4 hi = sa[rswz(arow0 + i * 32, st * 4 + 2 + h)];
        af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const u32x4 lo = sb[rswz(brow0 + j * 32, st * 4 + h)];
        const u32x4 hi = sb[rswz(brow0 + j * 32, st * 4 + 2 + h)];
        bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          // B fragment first (a lane keeps 4 consecutive output columns), each
          // operand with its own scale; formats 0 = fp8 e4m3
          if (st == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 0,
                                                                        (int)sb_cur[j], 0, (int)sa_cur[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 2,
                                                                        (int)sb_cur[j], 2, (int)sa_cur[i]);
        }
    }
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }

  // epilogue: as the bf16 kernel's (row = lane%32 of the block, columns
  // 8*(e/4) + 4*(lane/32) + 0..3)
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
          float hh[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          float u[4] = {acc[i][j + FN / 2][4 * q], acc[i][j + FN / 2][4 * q + 1], acc[i][j + FN / 2][4 * q + 2],
                        acc[i][j + FN / 2][4 * q + 3]};
          Epi::at_pair4(ep, row, col, hh, u);
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
