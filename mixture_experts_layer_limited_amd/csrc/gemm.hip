// Grouped GEMM kernels: the bf16 MFMA path (gfx950 v_mfma_f32_32x32x16_bf16)
// and a plain fp32 path, over the tile schedules of gemm.hpp.
#include "gemm.hpp"
#include "gemm_band.hpp"
#include "gemm_mfma.hpp"
#include "gemm_regs.hpp"
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
    float s = 0.0f;
    if (col < a.N)
      for (int k = c.k_begin; k < c.k_end; ++k) s += Ael(row, k) * Bel(col, k);
    if constexpr (Epi::kRowDot) {
      // the row's 16 columns sit in 16 consecutive lanes: a fixed tree sums
      // their terms into one partial per row and 16-column block
      float dot = col < a.N ? Epi::at(ep, c.g, row, col, s) : 0.0f;
      if (ep.dg_part) {
        for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 16);
        if (tx == 0 && c.n0 < ep.dg_ld) ep.dg_part[(int64_t)row * ep.dg_ld + c.n0] = dot;
      }
    } else {
      if (col < a.N) Epi::at(ep, c.g, row, col, s);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.  The bf16 path runs the MFMA kernels (gemm_mfma.hpp,
// gemm_band.hpp, gemm_regs.hpp); the fp32 path one 16x16 tile per workgroup.
// For RAGGED_M the tile count is only bounded on the host (sum over experts
// of ceil(n_e/BM) <= rows/BM + G); the kernels read the exact count on the
// device.
// ---------------------------------------------------------------------------

static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int BM, int BN, int WM, int WN, int STAGES, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi,
          int NLW = 0>
static hipError_t launch_mfma(const GemmArgs& a, const typename Epi::P& ep, int n_logical, int rows_total,
                              hipStream_t st, bool persistent) {
  using C = TileCfg<BM, BN, WM, WN, STAGES, false, NLW>;
  constexpr bool paired = Epi::kPaired;
  const int bn_cols = paired ? BN / 2 : BN;
  const int NT = (n_logical + bn_cols - 1) / bn_cols;
  const int MT = (MODE == RAGGED_M) ? 0 : (a.M + BM - 1) / BM;
  int64_t tiles;                          // upper bound of the logical tiles
  if (MODE == RAGGED_M) tiles = (int64_t)((rows_total + BM - 1) / BM + a.G) * NT;
  else if (MODE == RAGGED_K) tiles = (int64_t)a.G * MT * NT;
  else tiles = (int64_t)MT * NT * (a.kchunk > 0 ? (a.K + a.kchunk - 1) / a.kchunk : 1);
  if (tiles <= 0) return hipSuccess;
  constexpr int kLdsPerCU = 160 * 1024;
  const int per_cu = kLdsPerCU / C::LDS_BYTES > 0 ? kLdsPerCU / C::LDS_BYTES : 1;
  int64_t grid = persistent ? (int64_t)device_cus() * per_cu : tiles;
  if (tiles < grid) grid = tiles;
  auto kern = gemm_mfma_kernel<BM, BN, WM, WN, STAGES, LA, LB, MODE, Epi, false, false, NLW>;
  static bool lds_done[kLdsAttrDevices] = {};   // per device, per instantiation
  if (hipError_t e = raise_lds_limit(lds_done, (const void*)kern, C::LDS_BYTES); e != hipSuccess) return e;
  kern<<<(unsigned)grid, C::NTHR, C::LDS_BYTES, st>>>(a, MxArgs{}, ep, NT, MT);
  return hipGetLastError();
}

// Kernel per contraction class, from measurements at the 256-expert,
// d = 7168 shape: forward products and data gradients run on the DMA ring
// (128x256 tiles; 256x256 where experts are large, see big_tiles; data
// gradients read their row-contiguous weight with transposing LDS reads),
// expert weight gradients (short ragged contractions) on the band kernel for
// experts of at most kBandMaxRows rows plus the persistent DMA ring for
// larger ones, and the router's weight gradient on the persistent pipelined
// kernel.

template <OpLayout LA, OpLayout LB, GemmMode MODE, class Epi, int BK>
static hipError_t launch_pipe(const GemmArgs& a, const typename Epi::P& ep, int n_logical, int rows_total,
                              hipStream_t st) {
  using C = PipeCfg<BK>;
  const int bn_cols = Epi::kPaired ? C::BN / 2 : C::BN;
  const int NT = (n_logical + bn_cols - 1) / bn_cols;
  const int MT = (MODE == RAGGED_M) ? 0 : (a.M + C::BM - 1) / C::BM;
  int64_t tiles;                          // upper bound of the logical tiles
  if (MODE == RAGGED_M) tiles = (int64_t)((rows_total + C::BM - 1) / C::BM + a.G) * NT;
  else if (MODE == RAGGED_K) tiles = (int64_t)a.G * MT * NT;
  else tiles = (int64_t)MT * NT;
  if (tiles <= 0) return hipSuccess;
  if (a.G > kMaxExperts) return hipErrorInvalidValue;
  int64_t grid = (int64_t)device_cus() * 2;   // two workgroups fit a CU's LDS
  if (tiles < grid) grid = tiles;
  auto kern = gemm_pipe_kernel<LA, LB, MODE, Epi, BK>;
  static bool lds_done[kLdsAttrDevices] = {};   // per device, per instantiation
  if (hipError_t e = raise_lds_limit(lds_done, (const void*)kern, C::LDS_BYTES); e != hipSuccess) return e;
  kern<<<(unsigned)grid, C::NTHR, C::LDS_BYTES, st>>>(a, ep, NT, MT);
  return hipGetLastError();
}

// Stationary-band weight gradient (gemm_band.hpp) over the experts with
// 1..KMAX rows; false when the shape does not fit it (the caller then runs the
// general kernels on every expert).
template <class Epi>
static bool band_fits(const GemmArgs& a, const typename Epi::P& ep) {
  using S = BandShape<true, true>;          // (the wide unit; the narrow one's limits are within these)
  if (!a.offsets || a.G < 1 || a.G > kMaxExperts) return false;
  // the band on the output's longer side (a multiple of the wide band), the
  // streamed tiles on the other
  const bool pband = a.M > a.N;
  if ((pband ? a.M : a.N) % S::BW != 0 || (pband ? a.N : a.M) % BandCfg<true>::SW != 0) return false;
  if (a.lda != a.M || a.ldb != a.N || ep.ldc != a.N || ep.c_gstride != (int64_t)a.M * a.N) return false;
  if (((uintptr_t)a.A & 15) || ((uintptr_t)a.B & 15) || ((uintptr_t)ep.C & 15)) return false;
  // 32-bit buffer offsets: an expert's rows of either operand and a band's output rows
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)kBandMaxRows * a.lda * 2 < lim && (int64_t)kBandMaxRows * a.ldb * 2 < lim &&
         (int64_t)S::BW * ep.ldc * 2 < lim;   // a tile's output rows (up to the wide band's width)
}

template <class Epi, bool QBAND>
static hipError_t launch_band_kernel(const GemmArgs& a, const typename Epi::P& ep, hipStream_t st) {
  using C = BandCfg<QBAND>;
  auto kern = gemm_band_kernel<Epi, QBAND>;
  static bool lds_done[kLdsAttrDevices] = {};     // per device
  if (hipError_t e = raise_lds_limit(lds_done, (const void*)kern, C::LDS_BYTES); e != hipSuccess) return e;
  // 128-column bands along the band side, 128-wide streamed tiles along the other
  const int UB = (QBAND ? a.N : a.M) / C::SW, TU = (QBAND ? a.M : a.N) / C::SW;
  // each unit walks its tiles starting at its band index (mod the tile count),
  // so neighbouring units read different streamed tiles at any time (3% faster
  // than all starting at tile 0)
  constexpr int rot = 1;
  kern<<<(unsigned)device_cus(), C::NTHR, C::LDS_BYTES, st>>>(a, ep, UB, TU, rot);
  return hipGetLastError();
}

template <class Epi>
static hipError_t launch_band(const GemmArgs& a, const typename Epi::P& ep, hipStream_t st) {
  // the band on the output's longer side: more, shorter units (measured at the
  // 256-expert, d = 7168 shape: the gate/up gradient, 4096 x 7168, with the
  // band along its columns, the down gradient, 7168 x 2048, along its rows).
  // One launch holds both unit shapes: experts of 1 .. kBandWideRows rows take
  // 256-column bands, up to kBandMaxRows 128-column ones (at 128 rows per
  // expert the wide units took gate/up 3.93 -> 3.77 ms, down 2.06 -> 1.96 ms;
  // as a second launch the narrow units cost 0.5 ms more on skewed routing
  // than when they share the persistent grid).
  hipError_t e = a.M > a.N ? launch_band_kernel<Epi, false>(a, ep, st) : launch_band_kernel<Epi, true>(a, ep, st);
  if (e != hipSuccess) return e;
  // experts with more rows: the DMA ring, persistent, skipping the others
  // whole, on 256x256 tiles: a CU's operand traffic per flop is what bounds
  // it, and these take a third less of it than 128x256 tiles (Qwen3, 512 rows
  // per expert: gate/up 2.88 -> 2.36 ms, down 1.49 -> 1.22 ms).  On experts of
  // the band kernel's size the same ring is slower than the band (DeepSeek-V3
  // gate/up 5.13 ms against 3.90).
  GemmArgs big = a;
  big.k_skip = kBandMaxRows;
  return launch_mfma<256, 256, 2, 4, 2, MC, MC, RAGGED_K, Epi>(big, ep, a.N, 0, st, true);
}

// Tile rows of the ragged-row schedule.  The device tile prefix is built with
// this value and the kernel resolves its tiles with its own BM: they must agree.
// Forward products whose experts hold many rows (at least 512 on average: MFMA-bound) run the
// ring on 256x256 tiles, 2x4 waves of 128x64, two stages: half the operand traffic per output
// and a larger wave tile (the Qwen3 and Mixtral gate/up forwards ran 10% faster than on
// 128x256); with fewer rows the 256-row tiles would be mostly padding.
static bool big_tiles(int64_t rows, int G) { return G > 0 && rows >= (int64_t)512 * G; }
// The gate/up data gradient takes the 256x256 tiles under the same rule (on one
// box: Qwen3 2.06 -> 1.86 ms, Mixtral 2.54 -> 2.41, the EP share 2.23 -> 1.87).
// The SwiGLU-backward product (swiglu_bwd = true) always runs on 128x256 tiles:
// its epilogue reads H and U beside the accumulators and spilled at 256x256
// (Qwen3 1.67 ms there, 1.36 ms on 128x256).
int gemm_tile_rows(bool bf16, int64_t rows, int G, bool swiglu_bwd) {
  if (!bf16) return 16;
  return !swiglu_bwd && big_tiles(rows, G) ? 256 : 128;
}

template <class T, OpLayout LA, OpLayout LB, GemmMode MODE, class Epi>
static hipError_t run_gemm(const GemmArgs& a, const typename Epi::P& ep, int rows_total, hipStream_t st) {
  int n_logical;
  if constexpr (Epi::kPaired) n_logical = (int)ep.f; else n_logical = a.N;
  if constexpr (sizeof(T) == 2) {
    // weight gradients (short contractions) run persistent so that a tile's
    // stores overlap the next tile's loads; the rest one tile per workgroup
    const bool persistent = MODE == RAGGED_K;
    // staged epilogues store 16-byte row pieces: the calls' shape checks (d, f,
    // f_shared multiples of 64) and 16-byte aligned outputs guarantee them
    if constexpr (Epi::kStaged)
      if (!(ep.N % 8 == 0 && ep.ldc % 8 == 0 && ep.c_gstride % 8 == 0 && ((uintptr_t)ep.C & 15) == 0))
        return hipErrorInvalidValue;
    // dense products take 256x256 tiles only when those fill every CU: the
    // shared expert's down-projection data gradient (4096 x 2048 outputs,
    // 128 such tiles) runs 0.18 ms on 128x256 tiles against 0.25 ms
    const int64_t big_count = (int64_t)((a.M + 255) / 256) *
                              ((n_logical + (Epi::kPaired ? 127 : 255)) / (Epi::kPaired ? 128 : 256));
    const bool dense_big = a.M >= 1024 && n_logical >= 1024 && big_count >= device_cus();
    if constexpr (MODE != RAGGED_K) {
      // (not the SwiGLU-backward epilogue: see gemm_tile_rows)
      if constexpr (!Epi::kRowDot) {
        const bool big = MODE == RAGGED_M ? big_tiles(rows_total, a.G) : dense_big;
        if (big)
          return launch_mfma<256, 256, 2, 4, 2, LA, LB, MODE, Epi>(a, ep, n_logical, rows_total, st, persistent);
      }
    } else {
      // a weight gradient over one dense contraction of many rows (the
      // shared expert's, K = tokens) is MFMA-bound: 256x256 tiles, one per
      // workgroup, once they cover 7/8 of the CUs (gate/up 448 tiles: 0.35 ->
      // 0.27 ms; down 224 tiles: 0.18 -> 0.14 ms against persistent 128x256)
      if (a.offsets == nullptr && a.K >= 1024 && a.M >= 1024 && n_logical >= 1024 &&
          big_count * 8 >= (int64_t)device_cus() * 7)
        return launch_mfma<256, 256, 2, 4, 2, LA, LB, MODE, Epi>(a, ep, n_logical, rows_total, st, false);
    }
    // ragged-row products (one tile per workgroup): two load waves issue the
    // DMA and wait for it, the eight compute waves only meet them at the
    // barriers (DeepSeek-V3 on one box: down forward 1.84 -> 1.76 ms, down
    // data gradient 1.96 -> 1.85, gate/up data gradient 3.55 -> 3.51, the
    // SwiGLU forward unchanged; four load waves measured the same)
    if constexpr (MODE == RAGGED_M)
      return launch_mfma<128, 256, 2, 4, 3, LA, LB, MODE, Epi, 2>(a, ep, n_logical, rows_total, st, false);
    return launch_mfma<128, 256, 2, 4, 3, LA, LB, MODE, Epi>(a, ep, n_logical, rows_total, st, persistent);
  } else {
    const int NT = (n_logical + 15) / 16;
    const int MT = (MODE == RAGGED_M) ? 0 : (a.M + 15) / 16;
    int64_t grid;
    if (MODE == RAGGED_M) grid = (int64_t)((rows_total + 15) / 16 + a.G) * NT;
    else if (MODE == RAGGED_K) grid = (int64_t)a.G * MT * NT;
    else grid = (int64_t)MT * NT;
    if (grid <= 0) return hipSuccess;
    gemm_simple_kernel<T, LA, LB, MODE, Epi><<<(unsigned)grid, 256, 0, st>>>(a, ep, NT, MT);
    return hipGetLastError();
  }
}

// Weight gradients of experts without rows (or of a dense contraction over
// no rows) are exactly zero; the MFMA kernels skip empty contractions, so
// those outputs are filled here.
__global__ __launch_bounds__(256) void zero_empty_groups_kernel(const int* __restrict__ offsets,
                                                                u32x4* __restrict__ out, int64_t vec_per_group) {
  const int g = blockIdx.y;
  if (offsets && offsets[g + 1] != offsets[g]) return;    // NULL offsets: one empty group
  u32x4* o = out + g * vec_per_group;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vec_per_group; i += (int64_t)gridDim.x * blockDim.x)
    o[i] = z;
}

// The router logits have few output tiles (T / 128 x E / 256: 32 for 4096
// tokens and 256 experts) and a long contraction (d): split along d into
// parts that fill the CUs (at most 8, each at least 512 deep), each part's
// fp32 result in a block of its own, summed in part order afterwards (no
// atomics: the sum is the same on every run).
int router_logit_parts(bool bf16, int64_t T, int E, int d, int* kchunk) {
  *kchunk = d;
  if (!bf16 || d < 1024 || T <= 0) return 1;
  const int64_t tiles = ((T + 127) / 128) * ((E + 255) / 256);
  int64_t s = (256 + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > d / 512) s = d / 512;
  if (s <= 1) return 1;
  const int kc = (int)(((d + s - 1) / s + 63) / 64 * 64);
  *kchunk = kc;
  return (d + kc - 1) / kc;
}

// out[i] = storage(part[0][i] + part[1][i] + ...), in part order
template <class TO>
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int parts, int64_t n,
                                                        TO* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = part[i];
    for (int p = 1; p < parts; ++p) s += part[p * n + i];
    out[i] = from_f32<TO>(s);
  }
}

template <class TO>
static hipError_t launch_sum_parts(const float* part, int parts, int64_t n, TO* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  sum_parts_kernel<TO><<<(unsigned)blocks, 256, 0, st>>>(part, parts, n, out);
  return hipGetLastError();
}

template <class T>
hipError_t gemm_router_logits(const void* x, const void* w_r, float* logits, int T_, int E, int d, float* part,
                              hipStream_t st) {
  GemmArgs a{};
  a.A = x; a.lda = d; a.B = w_r; a.ldb = d; a.M = T_; a.N = E; a.K = d;
  a.b_next = E; a.b_kend = d; a.G = 1;
  int kchunk;
  const int parts = router_logit_parts(sizeof(T) == 2, T_, E, d, &kchunk);
  if (parts <= 1) {
    EpiStoreF32::P ep{logits, E, 0, T_, E};
    return run_gemm<T, KC, KC, DENSE, EpiStoreF32>(a, ep, T_, st);
  }
  a.kchunk = kchunk;
  const int64_t n = (int64_t)T_ * E;
  EpiStoreF32::P ep{part, E, n, T_, E};
  if (hipError_t e = run_gemm<T, KC, KC, DENSE, EpiStoreF32>(a, ep, T_, st); e != hipSuccess) return e;
  return launch_sum_parts<float>(part, parts, n, logits, st);
}

template <class T>
hipError_t gemm_swiglu_fwd(const void* xin, const int* offsets, const int* tile_prefix, int G,
                           const void* w13, void* hu, void* act, int rows, int d, int f,
                           const float* row_gates, bool from_stored, hipStream_t st) {
  GemmArgs a{};
  a.A = xin; a.lda = d; a.B = w13; a.ldb = d; a.b_gstride = (int64_t)2 * f * d;
  a.M = rows; a.N = 2 * f; a.K = d; a.b_next = 2 * f; a.b_kend = d;
  typename EpiSwiGLU<T>::P ep{(T*)act, (T*)hu, f, row_gates, from_stored ? 1 : 0};
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

// Gate-gradient partials per row of the down-projection data gradient: one
// per 64-column block on the MFMA path, per 16-column block on the fp32 one.
int gemm_dg_parts(bool bf16, int f) { return bf16 ? (f + 63) / 64 : (f + 15) / 16; }

// d_gates[n] = sum over p < P, in order, of part[row_id_map[n] * P + p]
__global__ __launch_bounds__(256) void gate_grad_sum_kernel(const float* __restrict__ part, int P,
                                                            const int32_t* __restrict__ row_id_map,
                                                            int64_t n_total, float* __restrict__ d_gates) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= n_total) return;
  const float* q = part + (int64_t)row_id_map[n] * P;
  float s = 0.0f;
  for (int i = 0; i < P; ++i) s += q[i];
  d_gates[n] = s;
}

hipError_t launch_gate_grad_sum(const float* part, int P, const int32_t* row_id_map, int64_t n_total,
                                float* d_gates, hipStream_t st) {
  if (n_total == 0) return hipSuccess;
  gate_grad_sum_kernel<<<(unsigned)((n_total + 255) / 256), 256, 0, st>>>(part, P, row_id_map, n_total, d_gates);
  return hipGetLastError();
}

// dA = dY W2 (B = W2 [d, f] read as (n=f-col, k=d-row): MC), SwiGLU backward
// epilogue (folded gates: row_gates with the gate-gradient partials dg_part
// [rows, gemm_dg_parts]; act recomputation: act_out)
template <class T>
hipError_t gemm_down_dgrad_swiglu_bwd(const void* dy, const int* offsets, const int* tile_prefix,
                                      int G, const void* w2, const void* hu, void* dhu, int rows,
                                      int d, int f, const float* row_gates, float* dg_part, void* act_out,
                                      hipStream_t st) {
  GemmArgs a{};
  a.A = dy; a.lda = d; a.B = w2; a.ldb = f; a.b_gstride = (int64_t)d * f;
  a.M = rows; a.N = f; a.K = d; a.b_next = f; a.b_kend = d;
  typename EpiSwiGLUBwd<T>::P ep{(const T*)hu, (T*)dhu, f, row_gates, row_gates ? dg_part : nullptr,
                                 gemm_dg_parts(sizeof(T) == 2, f), (T*)act_out};
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
// (P [rows, M], Q [rows, N] both read with the row as the contraction index).
// `site` (0..3) selects a distinct kernel symbol per call site.
template <class T, int kSite>
static hipError_t wgrad_site(const GemmArgs& a, void* dw, int M, int N, hipStream_t st) {
  typename EpiStore<T, kSite>::P ep{(T*)dw, N, (int64_t)M * N, M, N};
  if constexpr (sizeof(T) == 2)
    if (band_fits<EpiStore<T, kSite>>(a, ep)) return launch_band<EpiStore<T, kSite>>(a, ep, st);
  return run_gemm<T, MC, MC, RAGGED_K, EpiStore<T, kSite>>(a, ep, 0, st);
}

template <class T>
hipError_t gemm_wgrad(const void* P_, int M, const void* Q_, int N, const int* offsets, int G,
                      int K_dense, void* dw, int site, hipStream_t st) {
  GemmArgs a{};
  a.A = P_; a.lda = M; a.B = Q_; a.ldb = N;
  a.M = M; a.N = N; a.K = K_dense; a.a_mext = M; a.b_next = N; a.b_kend = K_dense;
  a.offsets = offsets; a.G = offsets ? G : 1;
  if (sizeof(T) == 2 && (offsets || K_dense == 0)) {
    // the bf16 kernels skip tiles without a contraction: zero those outputs
    const int64_t vec = (int64_t)M * N * sizeof(T) / 16;   // M*N is a multiple of 64
    zero_empty_groups_kernel<<<dim3(64, offsets ? G : 1), 256, 0, st>>>(offsets, (u32x4*)dw, vec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (site) {
    case 1: return wgrad_site<T, 1>(a, dw, M, N, st);
    case 2: return wgrad_site<T, 2>(a, dw, M, N, st);
    case 3: return wgrad_site<T, 3>(a, dw, M, N, st);
    default: return wgrad_site<T, 0>(a, dw, M, N, st);
  }
}

// The router weight gradient has E x d outputs (1 x 32 tiles of 128 x 128 for
// 128 experts and d = 4096) and a contraction over all T tokens: split the
// tokens into parts that fill both workgroup slots of every CU (at most 8,
// each at least 256 tokens), fp32 parts summed in part order and rounded once.
int router_wgrad_parts(bool bf16, int64_t T, int E, int d, int* kchunk) {
  *kchunk = (int)T;
  if (!bf16 || T < 512) return 1;
  const int64_t tiles = (int64_t)((E + 127) / 128) * ((d + 127) / 128);
  int64_t s = (512 + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > T / 256) s = T / 256;
  if (s <= 1) return 1;
  const int kc = (int)(((T + s - 1) / s + 63) / 64 * 64);
  *kchunk = kc;
  return (int)((T + kc - 1) / kc);
}

// router backward: dW_r = dl^T x   (dl [T, Ep] with Ep = E rounded up to 8, zero padded)
template <class T>
hipError_t gemm_router_wgrad(const void* dl, int Ep, int E, const void* x, int T_, int d, void* dw_r, float* part,
                             hipStream_t st) {
  GemmArgs a{};
  a.A = dl; a.lda = Ep; a.B = x; a.ldb = d;
  a.M = E; a.N = d; a.K = T_; a.a_mext = Ep; a.b_next = d; a.b_kend = T_; a.G = 1;
  typename EpiStore<T, 4>::P ep{(T*)dw_r, d, 0, E, d};
  // E output rows: the persistent 128x128 kernel (the ring's 128x256 tiles are
  // few and mostly padding: 4 experts, 32768 tokens, d = 7168 took 0.29 ms on
  // the ring, 0.16 here; 256 experts, 4096 tokens 0.081 and 0.070)
  if constexpr (sizeof(T) == 2) {
    if (d % 8 == 0 && ((uintptr_t)dw_r & 15) == 0) {
      int kchunk;
      const int parts = router_wgrad_parts(true, T_, E, d, &kchunk);
      if (parts > 1) {
        a.G = parts;
        a.kchunk = kchunk;
        const int64_t n = (int64_t)E * d;
        EpiStoreF32::P pp{part, d, n, E, d};
        if (hipError_t e = launch_pipe<MC, MC, RAGGED_K, EpiStoreF32, 64>(a, pp, d, 0, st); e != hipSuccess) return e;
        return launch_sum_parts<T>(part, parts, n, (T*)dw_r, st);
      }
      return launch_pipe<MC, MC, RAGGED_K, EpiStore<T, 4>, 64>(a, ep, d, 0, st);
    }
  }
  return run_gemm<T, MC, MC, RAGGED_K, EpiStore<T, 4>>(a, ep, 0, st);
}

// router backward: dx_partial += dl W_r  (K = Ep, rows k >= E of W_r read as 0)
template <class T>
hipError_t gemm_router_dgrad(const void* dl, int Ep, int E, const void* w_r, int T_, int d,
                             float* dx_partial, hipStream_t st) {
  GemmArgs a{};
  a.A = dl; a.lda = Ep; a.B = w_r; a.ldb = d;
  a.M = T_; a.N = d; a.K = Ep; a.b_next = d; a.b_kend = E; a.G = 1;
  EpiAccumF32::P ep{dx_partial, d, 0, T_, d};
  // a short contraction (Ep) and an fp32 read-modify-write of every output:
  // persistent 128x256 tiles, so that a tile's epilogue overlaps the next
  // tile's loads
  if constexpr (sizeof(T) == 2) return launch_mfma<128, 256, 2, 4, 3, KC, MC, DENSE, EpiAccumF32>(a, ep, d, T_, st, true);
  return run_gemm<T, KC, MC, DENSE, EpiAccumF32>(a, ep, T_, st);
}

#define MOE_INSTANTIATE(T)                                                                       \
  template hipError_t gemm_router_logits<T>(const void*, const void*, float*, int, int, int,     \
                                            float*, hipStream_t);                                \
  template hipError_t gemm_swiglu_fwd<T>(const void*, const int*, const int*, int, const void*,  \
                                         void*, void*, int, int, int, const float*, bool,        \
                                         hipStream_t);                                           \
  template hipError_t gemm_down_fwd<T>(const void*, const int*, const int*, int, const void*,    \
                                       void*, int, int, int, hipStream_t);                       \
  template hipError_t gemm_down_dgrad_swiglu_bwd<T>(const void*, const int*, const int*, int,    \
                                                    const void*, const void*, void*, int, int,   \
                                                    int, const float*, float*, void*,            \
                                                    hipStream_t);                                \
  template hipError_t gemm_gateup_dgrad<T>(const void*, const int*, const int*, int,             \
                                           const void*, void*, bool, int, int, int,              \
                                           hipStream_t);                                         \
  template hipError_t gemm_wgrad<T>(const void*, int, const void*, int, const int*, int, int,    \
                                    void*, int, hipStream_t);                                         \
  template hipError_t gemm_router_wgrad<T>(const void*, int, int, const void*, int, int, void*,  \
                                           float*, hipStream_t);                                 \
  template hipError_t gemm_router_dgrad<T>(const void*, int, int, const void*, int, int, float*, \
                                           hipStream_t);

MOE_INSTANTIATE(float)
MOE_INSTANTIATE(bf16)

}  // namespace moe
