// Grouped GEMM kernels: the bf16 MFMA path (gfx950 v_mfma_f32_32x32x16_bf16)
// and a plain fp32 path, over the tile schedules of gemm.hpp.
#include "gemm.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Cumulative m-tile counts per group (one workgroup, G <= 256).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_prefix_kernel(const int* __restrict__ offsets, int G,
                                                          int BM, int* __restrict__ prefix) {
  __shared__ int s[kMaxExperts];
  int g = threadIdx.x;
  int v = 0;
  if (g < G) v = (offsets[g + 1] - offsets[g] + BM - 1) / BM;
  s[g] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {     // inclusive Hillis-Steele scan
    int add = (g >= o) ? s[g - o] : 0;
    __syncthreads();
    s[g] += add;
    __syncthreads();
  }
  if (g < G) prefix[g + 1] = s[g];
  if (g == 0) prefix[0] = 0;
}

hipError_t launch_tile_prefix(const int* offsets, int G, int BM, int* prefix, hipStream_t st) {
  tile_prefix_kernel<<<1, 256, 0, st>>>(offsets, G, BM, prefix);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: 256 threads = 4 waves in a 2x2 arrangement, each wave
// owning a 64x64 sub-tile as 2x2 blocks of 32x32 MFMA accumulators.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a, typename Epi::P ep, int NT, int MT) {
  static_assert(BM == 128 && BN == 128, "wave layout assumes 128x128 tiles");
  constexpr int PITCH = BK + 8;                 // bf16 elements per LDS row
  constexpr int KCH = BK / 8;                   // 16-byte chunks per row
  constexpr int A_KC_LOADS = BM * KCH / 256;
  constexpr int B_KC_LOADS = BN * KCH / 256;
  constexpr int A_MC_BLKS = (BK / 4) * (BM / 8) / 256;
  constexpr int B_MC_BLKS = (BK / 4) * (BN / 8) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * PITCH];

  const int total = total_tiles<MODE>(a, NT, MT);
  if ((int)blockIdx.x >= total) return;
  const int L = xcd_remap(blockIdx.x, total);
  TileCoord c;
  resolve_tile<MODE, BM>(a, L, NT, MT, c);
  const int nt = c.n0;

  const uint16_t* __restrict__ A = (const uint16_t*)a.A;
  const uint16_t* __restrict__ B = (const uint16_t*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * a.b_gstride : 0);
  const int tid = threadIdx.x;
  const int b_kend = (MODE == RAGGED_K) ? c.k_end : min(c.k_end, a.b_kend);

  // B tile rows resolved once (KC layout): absolute B row or "invalid"
  int brow[B_KC_LOADS > 0 ? B_KC_LOADS : 1];
  if (LB == KC) {
#pragma unroll
    for (int i = 0; i < B_KC_LOADS; ++i) {
      int q = tid + i * 256;
      int r = q / KCH;
      brow[i] = Epi::b_row(ep, nt, r, BN);
    }
  }

  u32x4 ra[LA == KC ? A_KC_LOADS : 4 * A_MC_BLKS];
  u32x4 rb[LB == KC ? B_KC_LOADS : 4 * B_MC_BLKS];

  auto load_tiles = [&](int k0) {
    if (LA == KC) {
#pragma unroll
      for (int i = 0; i < A_KC_LOADS; ++i) {
        int q = tid + i * 256;
        int r = q / KCH, kc = q % KCH;
        int grow = c.m0 + r, kk = k0 + kc * 8;
        u32x4 v = {0, 0, 0, 0};
        if (grow < c.m_end && kk < c.k_end) v = *(const u32x4*)(A + (int64_t)grow * a.lda + kk);
        ra[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_MC_BLKS; ++i) {
        int q = tid + i * 256;
        int kb = q / (BM / 8), mb = q % (BM / 8);
        int m = c.m0 + mb * 8;
        bool mok = m + 8 <= a.a_mext;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int kk = k0 + kb * 4 + r;
          u32x4 v = {0, 0, 0, 0};
          if (mok && kk < c.k_end) v = *(const u32x4*)(A + (int64_t)kk * a.lda + m);
          ra[i * 4 + r] = v;
        }
      }
    }
    if (LB == KC) {
#pragma unroll
      for (int i = 0; i < B_KC_LOADS; ++i) {
        int q = tid + i * 256;
        int kc = q % KCH;
        int kk = k0 + kc * 8;
        u32x4 v = {0, 0, 0, 0};
        if (brow[i] < a.b_next && kk < c.k_end) v = *(const u32x4*)(B + (int64_t)brow[i] * a.ldb + kk);
        rb[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_MC_BLKS; ++i) {
        int q = tid + i * 256;
        int kb = q / (BN / 8), nb = q % (BN / 8);
        int n = nt * BN + nb * 8;
        bool nok = n + 8 <= a.b_next;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int kk = k0 + kb * 4 + r;
          u32x4 v = {0, 0, 0, 0};
          if (nok && kk < b_kend) v = *(const u32x4*)(B + (int64_t)kk * a.ldb + n);
          rb[i * 4 + r] = v;
        }
      }
    }
  };

  // 4 rows (k..k+3) x 8 columns -> 8 columns x 4 k, written K-contiguous
  auto store_transposed = [&](uint16_t* s, const u32x4* r4, int row0, int kcol) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      int w = m >> 1;
      uint32_t e0 = (m & 1) ? (r4[0][w] >> 16) : (r4[0][w] & 0xFFFFu);
      uint32_t e1 = (m & 1) ? (r4[1][w] >> 16) : (r4[1][w] & 0xFFFFu);
      uint32_t e2 = (m & 1) ? (r4[2][w] >> 16) : (r4[2][w] & 0xFFFFu);
      uint32_t e3 = (m & 1) ? (r4[3][w] >> 16) : (r4[3][w] & 0xFFFFu);
      u32x2 o = {e0 | (e1 << 16), e2 | (e3 << 16)};
      *(u32x2*)(s + (row0 + m) * PITCH + kcol) = o;
    }
  };

  auto store_tiles = [&]() {
    if (LA == KC) {
#pragma unroll
      for (int i = 0; i < A_KC_LOADS; ++i) {
        int q = tid + i * 256;
        int r = q / KCH, kc = q % KCH;
        *(u32x4*)(sA + r * PITCH + kc * 8) = ra[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_MC_BLKS; ++i) {
        int q = tid + i * 256;
        int kb = q / (BM / 8), mb = q % (BM / 8);
        store_transposed(sA, &ra[i * 4], mb * 8, kb * 4);
      }
    }
    if (LB == KC) {
#pragma unroll
      for (int i = 0; i < B_KC_LOADS; ++i) {
        int q = tid + i * 256;
        int r = q / KCH, kc = q % KCH;
        *(u32x4*)(sB + r * PITCH + kc * 8) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_MC_BLKS; ++i) {
        int q = tid + i * 256;
        int kb = q / (BN / 8), nb = q % (BN / 8);
        store_transposed(sB, &rb[i * 4], nb * 8, kb * 4);
      }
    }
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int klen = c.k_end - c.k_begin;
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
    load_tiles(c.k_begin);
    store_tiles();
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_tiles(c.k_begin + (kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        af[mb] = *(const bf16x8*)(sA + (wm * 64 + mb * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bfr[nb] = *(const bf16x8*)(sB + (wn * 64 + nb * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store_tiles();
      __syncthreads();
    }
  }

  // epilogue: accumulator element e of block (mb, nb) sits at
  // row 8*(e/4) + 4*(lane/32) + e%4, column lane%32 of that 32x32 block
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      int lr = wm * 64 + mb * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
      int row = c.m0 + lr;
      if (row >= c.m_end) continue;
      if constexpr (Epi::kPaired) {
        int col = nt * (BN / 2) + wn * 32 + (lane & 31);
        Epi::at_pair(ep, row, col, acc[mb][0][e], acc[mb][1][e]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          int col = nt * BN + wn * 64 + nb * 32 + (lane & 31);
          Epi::at(ep, c.g, row, col, acc[mb][nb][e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: one thread per output element of a 16x16 tile, sequential K.
// ---------------------------------------------------------------------------
template <class T, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi>
__global__ __launch_bounds__(256) void gemm_simple_kernel(GemmArgs a, typename Epi::P ep, int NT, int MT) {
  const int total = total_tiles<MODE>(a, NT, MT);
  if ((int)blockIdx.x >= total) return;
  TileCoord c;
  resolve_tile<MODE, 16>(a, blockIdx.x, NT, MT, c);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = c.m0 + ty;
  if (row >= c.m_end) return;
  const T* __restrict__ A = (const T*)a.A;
  const T* __restrict__ B = (const T*)a.B + (MODE == RAGGED_M ? (int64_t)c.g * a.b_gstride : 0);
  const int b_kend = (MODE == RAGGED_K) ? c.k_end : min(c.k_end, a.b_kend);
  auto Ael = [&](int m, int k) -> float {
    return LA == KC ? to_f32(A[(int64_t)m * a.lda + k]) : to_f32(A[(int64_t)k * a.lda + m]);
  };
  auto Bel = [&](int n, int k) -> float {
    if (k >= b_kend) return 0.0f;
    return LB == KC ? to_f32(B[(int64_t)n * a.ldb + k]) : to_f32(B[(int64_t)k * a.ldb + n]);
  };
  if constexpr (Epi::kPaired) {
    const int col = c.n0 * 16 + tx;
    if (col >= ep.f) return;
    float h = 0.0f, u = 0.0f;
    for (int k = c.k_begin; k < c.k_end; ++k) {
      float xv = Ael(row, k);
      h += xv * Bel(col, k);
      u += xv * Bel((int)ep.f + col, k);
    }
    Epi::at_pair(ep, row, col, h, u);
  } else {
    const int col = c.n0 * 16 + tx;
    if (col >= a.N) return;
    float s = 0.0f;
    for (int k = c.k_begin; k < c.k_end; ++k) s += Ael(row, k) * Bel(col, k);
    Epi::at(ep, c.g, row, col, s);
  }
}

// ---------------------------------------------------------------------------
// Launchers.  `mtiles_bound` = upper bound of m-tiles (RAGGED_M), n = logical
// N (gate columns for the paired SwiGLU epilogue).
// ---------------------------------------------------------------------------
template <class T, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi>
static hipError_t run_gemm(const GemmArgs& a, const typename Epi::P& ep, int rows_total, hipStream_t st) {
  constexpr bool paired = Epi::kPaired;
  int n_logical;
  if constexpr (paired) n_logical = (int)ep.f; else n_logical = a.N;
  if constexpr (sizeof(T) == 2) {
    constexpr int BM = 128, BN = 128, BK = 64;
    const int NT = (n_logical + (paired ? BN / 2 : BN) - 1) / (paired ? BN / 2 : BN);
    const int MT = (MODE == RAGGED_M) ? 0 : (a.M + BM - 1) / BM;
    int64_t grid;
    if (MODE == RAGGED_M) grid = (int64_t)((rows_total + BM - 1) / BM + a.G) * NT;
    else if (MODE == RAGGED_K) grid = (int64_t)a.G * MT * NT;
    else grid = (int64_t)MT * NT;
    if (grid <= 0) return hipSuccess;
    gemm_mfma_kernel<BM, BN, BK, LA, LB, MODE, Epi><<<(unsigned)grid, 256, 0, st>>>(a, ep, NT, MT);
  } else {
    const int NT = (n_logical + 15) / 16;
    const int MT = (MODE == RAGGED_M) ? 0 : (a.M + 15) / 16;
    int64_t grid;
    if (MODE == RAGGED_M) grid = (int64_t)((rows_total + 15) / 16 + a.G) * NT;
    else if (MODE == RAGGED_K) grid = (int64_t)a.G * MT * NT;
    else grid = (int64_t)MT * NT;
    if (grid <= 0) return hipSuccess;
    gemm_simple_kernel<T, LA, LB, MODE, Epi><<<(unsigned)grid, 256, 0, st>>>(a, ep, NT, MT);
  }
  return hipGetLastError();
}

int gemm_tile_rows(bool bf16) { return bf16 ? 128 : 16; }

template <class T>
hipError_t gemm_router_logits(const void* x, const void* w_r, float* logits, int T_, int E, int d,
                              hipStream_t st) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.B = w_r; a.ldb = d; a.M = T_; a.N = E; a.K = d;
  a.b_next = E; a.b_kend = d; a.G = 1;
  EpiStoreF32::P ep{logits, E, 0, T_, E};
  return run_gemm<T, KC, KC, DENSE, EpiStoreF32>(a, ep, T_, st);
}

template <class T>
hipError_t gemm_swiglu_fwd(const void* xin, const int* offsets, const int* tile_prefix, int G,
                           const void* w13, void* hu, void* act, int rows, int d, int f,
                           hipStream_t st) {
  GemmArgs a{};
  a.A = xin; a.lda = d; a.B = w13; a.ldb = d; a.b_gstride = (int64_t)2 * f * d;
  a.M = rows; a.N = 2 * f; a.K = d; a.b_next = 2 * f; a.b_kend = d;
  typename EpiSwiGLU<T>::P ep{(T*)act, (T*)hu, f};
  if (offsets) {
    a.offsets = offsets; a.tile_prefix = tile_prefix; a.G = G;
    return run_gemm<T, KC, KC, RAGGED_M, EpiSwiGLU<T>>(a, ep, rows, st);
  }
  a.G = 1;
  return run_gemm<T, KC, KC, DENSE, EpiSwiGLU<T>>(a, ep, rows, st);
}

template <class T>
hipError_t gemm_down_fwd(const void* act, const int* offsets, const int* tile_prefix, int G,
                         const void* w2, void* y, int rows, int d, int f, hipStream_t st) {
  GemmArgs a{};
  a.A = act; a.lda = f; a.B = w2; a.ldb = f; a.b_gstride = (int64_t)d * f;
  a.M = rows; a.N = d; a.K = f; a.b_next = d; a.b_kend = f;
  typename EpiStore<T>::P ep{(T*)y, d, 0, rows, d};
  if (offsets) {
    a.offsets = offsets; a.tile_prefix = tile_prefix; a.G = G;
    return run_gemm<T, KC, KC, RAGGED_M, EpiStore<T>>(a, ep, rows, st);
  }
  a.G = 1;
  return run_gemm<T, KC, KC, DENSE, EpiStore<T>>(a, ep, rows, st);
}

// dA = dY W2 (B = W2 [d, f] read as (n=f-col, k=d-row): MC), SwiGLU backward epilogue
template <class T>
hipError_t gemm_down_dgrad_swiglu_bwd(const void* dy, const int* offsets, const int* tile_prefix,
                                      int G, const void* w2, const void* hu, void* dhu, int rows,
                                      int d, int f, hipStream_t st) {
  GemmArgs a{};
  a.A = dy; a.lda = d; a.B = w2; a.ldb = f; a.b_gstride = (int64_t)d * f;
  a.M = rows; a.N = f; a.K = d; a.b_next = f; a.b_kend = d;
  typename EpiSwiGLUBwd<T>::P ep{(const T*)hu, (T*)dhu, f};
  if (offsets) {
    a.offsets = offsets; a.tile_prefix = tile_prefix; a.G = G;
    return run_gemm<T, KC, MC, RAGGED_M, EpiSwiGLUBwd<T>>(a, ep, rows, st);
  }
  a.G = 1;
  return run_gemm<T, KC, MC, DENSE, EpiSwiGLUBwd<T>>(a, ep, rows, st);
}

// dX = dHU W13 (K = 2f; B = W13 [2f, d] read as MC); storage or fp32 output
template <class T>
hipError_t gemm_gateup_dgrad(const void* dhu, const int* offsets, const int* tile_prefix, int G,
                             const void* w13, void* dx, bool f32_out, int rows, int d, int f,
                             hipStream_t st) {
  GemmArgs a{};
  a.A = dhu; a.lda = 2 * f; a.B = w13; a.ldb = d; a.b_gstride = (int64_t)2 * f * d;
  a.M = rows; a.N = d; a.K = 2 * f; a.b_next = d; a.b_kend = 2 * f;
  if (f32_out) {
    EpiStoreF32::P ep{(float*)dx, d, 0, rows, d};
    if (offsets) {
      a.offsets = offsets; a.tile_prefix = tile_prefix; a.G = G;
      return run_gemm<T, KC, MC, RAGGED_M, EpiStoreF32>(a, ep, rows, st);
    }
    a.G = 1;
    return run_gemm<T, KC, MC, DENSE, EpiStoreF32>(a, ep, rows, st);
  }
  typename EpiStore<T>::P ep{(T*)dx, d, 0, rows, d};
  if (offsets) {
    a.offsets = offsets; a.tile_prefix = tile_prefix; a.G = G;
    return run_gemm<T, KC, MC, RAGGED_M, EpiStore<T>>(a, ep, rows, st);
  }
  a.G = 1;
  return run_gemm<T, KC, MC, DENSE, EpiStore<T>>(a, ep, rows, st);
}

// dW[g] (M x N) = sum over rows r of group g: P[r, m] Q[r, n]
// (P [rows, M], Q [rows, N] both read with the row as the contraction index)
template <class T>
hipError_t gemm_wgrad(const void* P_, int M, const void* Q_, int N, const int* offsets, int G,
                      int K_dense, void* dw, hipStream_t st) {
  GemmArgs a{};
  a.A = P_; a.lda = M; a.B = Q_; a.ldb = N;
  a.M = M; a.N = N; a.K = K_dense; a.a_mext = M; a.b_next = N; a.b_kend = K_dense;
  a.offsets = offsets; a.G = offsets ? G : 1;
  typename EpiStore<T>::P ep{(T*)dw, N, (int64_t)M * N, M, N};
  return run_gemm<T, MC, MC, RAGGED_K, EpiStore<T>>(a, ep, 0, st);
}

// router backward: dW_r = dl^T x   (dl [T, Ep] with Ep = E rounded up to 8, zero padded)
template <class T>
hipError_t gemm_router_wgrad(const void* dl, int Ep, int E, const void* x, int T_, int d, void* dw_r,
                             hipStream_t st) {
  GemmArgs a{};
  a.A = dl; a.lda = Ep; a.B = x; a.ldb = d;
  a.M = E; a.N = d; a.K = T_; a.a_mext = Ep; a.b_next = d; a.b_kend = T_; a.G = 1;
  typename EpiStore<T>::P ep{(T*)dw_r, d, 0, E, d};
  return run_gemm<T, MC, MC, RAGGED_K, EpiStore<T>>(a, ep, 0, st);
}

// router backward: dx_partial += dl W_r  (K = Ep, rows k >= E of W_r read as 0)
template <class T>
hipError_t gemm_router_dgrad(const void* dl, int Ep, int E, const void* w_r, int T_, int d,
                             float* dx_partial, hipStream_t st) {
  GemmArgs a{};
  a.A = dl; a.lda = Ep; a.B = w_r; a.ldb = d;
  a.M = T_; a.N = d; a.K = Ep; a.b_next = d; a.b_kend = E; a.G = 1;
  EpiAccumF32::P ep{dx_partial, d, 0, T_, d};
  return run_gemm<T, KC, MC, DENSE, EpiAccumF32>(a, ep, T_, st);
}

#define MOE_INSTANTIATE(T)                                                                       \
  template hipError_t gemm_router_logits<T>(const void*, const void*, float*, int, int, int,     \
                                            hipStream_t);                                        \
  template hipError_t gemm_swiglu_fwd<T>(const void*, const int*, const int*, int, const void*,  \
                                         void*, void*, int, int, int, hipStream_t);              \
  template hipError_t gemm_down_fwd<T>(const void*, const int*, const int*, int, const void*,    \
                                       void*, int, int, int, hipStream_t);                       \
  template hipError_t gemm_down_dgrad_swiglu_bwd<T>(const void*, const int*, const int*, int,    \
                                                    const void*, const void*, void*, int, int,   \
                                                    int, hipStream_t);                           \
  template hipError_t gemm_gateup_dgrad<T>(const void*, const int*, const int*, int,             \
                                           const void*, void*, bool, int, int, int,              \
                                           hipStream_t);                                         \
  template hipError_t gemm_wgrad<T>(const void*, int, const void*, int, const int*, int, int,    \
                                    void*, hipStream_t);                                         \
  template hipError_t gemm_router_wgrad<T>(const void*, int, int, const void*, int, int, void*,  \
                                           hipStream_t);                                         \
  template hipError_t gemm_router_dgrad<T>(const void*, int, int, const void*, int, int, float*, \
                                           hipStream_t);

MOE_INSTANTIATE(float)
MOE_INSTANTIATE(bf16)

}  // namespace moe
