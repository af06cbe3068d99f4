// Grouped GEMM machinery for the expert, shared-expert and router contractions.
//
// Every contraction of the layer is C[m,n] = sum_k A(m,k) B(n,k) over groups:
//   RAGGED_M  groups split the rows of A and C (expert g owns rows
//             offsets[g]..offsets[g+1]-1 of the permuted buffer) and each group
//             has its own B (the expert's weight): forward GEMMs and dgrads.
//   RAGGED_K  groups split the contraction (an expert's rows again) and each
//             group writes its own C (that expert's weight gradient): wgrads.
//   DENSE     one group (router, shared expert).
// Operands are stored either K-contiguous ("KC": element (i,k) at p[i*ld+k]) or
// row-index-contiguous ("MC": element (i,k) at p[k*ld+i]).  Tiles are staged in
// LDS K-contiguous per row, so MC operands are transposed in registers on the
// way in; the MFMA fragments are then read identically for every layout.
#pragma once

#include "common.hpp"

namespace moe {

enum OpLayout { KC = 0, MC = 1 };
enum GemmMode { DENSE = 0, RAGGED_M = 1, RAGGED_K = 2 };

struct GemmArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int64_t b_gstride;       // element offset between groups' B (RAGGED_M experts)
  int M, N, K;             // DENSE: all three; RAGGED_M: N, K; RAGGED_K: M, N
  int a_mext;              // MC A: valid extent of the row index for loads (>= M, mult. of 8)
  int b_next;              // valid extent of B's n index for loads
  int b_kend;              // rows k >= b_kend of an MC B read as 0 (DENSE), else K
  const int* offsets;      // [G+1] ragged offsets (RAGGED_*); NULL + G=1 means [0,K)
  const int* tile_prefix;  // RAGGED_M: [G+1] cumulative m-tiles per group
  int G;
};

struct TileCoord {
  int g;        // group
  int m0;       // first row of the tile (absolute row of A/C for RAGGED_M)
  int m_end;    // rows >= m_end are outside the group
  int n0;       // first column (tile-local meaning for paired epilogues)
  int k_begin;  // contraction range of this group
  int k_end;
};

// Resolve a logical tile index.  Returns false when the tile is empty.
template <GemmMode MODE, int BM>
__device__ __forceinline__ bool resolve_tile(const GemmArgs& a, int L, int NT, int MT, TileCoord& c) {
  if (MODE == DENSE) {
    int mt = L % MT, nt = L / MT;
    c.g = 0; c.m0 = mt * BM; c.m_end = a.M; c.n0 = nt; c.k_begin = 0; c.k_end = a.K;
    return true;
  } else if (MODE == RAGGED_M) {
    // expert-major order: all tiles of group g, n-tile major, m-tile fastest
    int lo = 0, hi = a.G;  // find g with tile_prefix[g]*NT <= L < tile_prefix[g+1]*NT
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (a.tile_prefix[mid] * NT <= L) lo = mid; else hi = mid;
    }
    int g = lo;
    int first = a.tile_prefix[g], mt_g = a.tile_prefix[g + 1] - first;
    int local = L - first * NT;
    int nt = local / mt_g, mi = local % mt_g;
    int row0 = a.offsets[g];
    c.g = g; c.m0 = row0 + mi * BM; c.m_end = a.offsets[g + 1]; c.n0 = nt;
    c.k_begin = 0; c.k_end = a.K;
    return true;
  } else {
    int per = MT * NT;
    int g = L / per, r = L % per;
    int mt = r % MT, nt = r / MT;
    c.g = g; c.m0 = mt * BM; c.m_end = a.M; c.n0 = nt;
    c.k_begin = a.offsets ? a.offsets[g] : 0;
    c.k_end = a.offsets ? a.offsets[g + 1] : a.K;
    return true;
  }
}

// Total logical tiles (device side; RAGGED_M depends on the expert sizes).
template <GemmMode MODE>
__device__ __forceinline__ int total_tiles(const GemmArgs& a, int NT, int MT) {
  if (MODE == RAGGED_M) return a.tile_prefix[a.G] * NT;
  if (MODE == RAGGED_K) return a.G * MT * NT;
  return MT * NT;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// Give each XCD a contiguous run of logical tiles so that tiles sharing a
// weight panel or an activation panel meet in the same L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  int q = total >> 3, r = total & 7;
  int x = b & 7, i = b >> 3;
  return x * q + (x < r ? x : r) + i;
}

// ---------------------------------------------------------------------------
// Epilogues.  Each receives fp32 results at absolute (row, col) positions.
// ---------------------------------------------------------------------------
template <class T>
struct EpiStore {                       // C[row, col] = storage(v)
  struct P { T* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) p.C[g * p.c_gstride + (int64_t)row * p.ldc + col] = from_f32<T>(v);
  }
};

struct EpiStoreF32 {                    // C[row, col] = v   (fp32 output)
  struct P { float* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) p.C[g * p.c_gstride + (int64_t)row * p.ldc + col] = v;
  }
};

struct EpiAccumF32 {                    // C[row, col] += v  (fp32, one writer per element)
  struct P { float* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) {
      float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
      *c = *c + v;
    }
  }
};

// SwiGLU forward: the tile's B rows interleave 32 gate rows and the matching
// 32 up rows, so one lane holds H and U of the same (row, col).
template <class T>
struct EpiSwiGLU {
  struct P { T* act; T* hu; int64_t f; };  // act [rows, f], hu [rows, 2f] or NULL
  static constexpr bool kPaired = true;
  // tile-row r in [0, BN): wave half wn = r/64; r%64 < 32 -> gate, else up
  __device__ static int b_row(const P& p, int nt, int r, int BN) {
    int wn = r / 64, half = (r % 64) / 32, i = r % 32;
    int col = nt * (BN / 2) + wn * 32 + i;
    if (col >= p.f) return 1 << 30;
    return half ? (int)p.f + col : col;
  }
  __device__ static void at_pair(const P& p, int row, int col, float h, float u) {
    if (col >= p.f) return;
    float a = h / (1.0f + expf(-h)) * u;
    p.act[(int64_t)row * p.f + col] = from_f32<T>(a);
    if (p.hu) {
      p.hu[(int64_t)row * 2 * p.f + col] = from_f32<T>(h);
      p.hu[(int64_t)row * 2 * p.f + p.f + col] = from_f32<T>(u);
    }
  }
};

// SwiGLU backward inside the down-projection dgrad: v = dA[row, col]
template <class T>
struct EpiSwiGLUBwd {
  struct P { const T* hu; T* dhu; int64_t f; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int, int row, int col, float dA) {
    if (col >= p.f) return;
    int64_t base = (int64_t)row * 2 * p.f;
    float h = to_f32(p.hu[base + col]);
    float u = to_f32(p.hu[base + p.f + col]);
    float sg = 1.0f / (1.0f + expf(-h));
    float dh = dA * u * sg * (1.0f + h * (1.0f - sg));
    float du = dA * h * sg;
    p.dhu[base + col] = from_f32<T>(dh);
    p.dhu[base + p.f + col] = from_f32<T>(du);
  }
};

}  // namespace moe
