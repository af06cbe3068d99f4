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
// Epilogues.  Each receives fp32 results at absolute (row, col) positions:
// `at` for one element (fp32 kernel), `at4` for four consecutive columns
// col..col+3 (MFMA kernel; col is a multiple of 4).
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void store4(T* p, const float v[4], bool vec) {
  if constexpr (sizeof(T) == 2) {
    if (vec) {
      u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *(u32x2*)p = w;
      return;
    }
  } else {
    if (vec) {
      floatx4 w = {v[0], v[1], v[2], v[3]};
      *(floatx4*)p = w;
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = from_f32<T>(v[i]);
}

template <class T>
__device__ __forceinline__ void load4(const T* p, float v[4]) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w = *(const u32x2*)p;
    v[0] = bf16_bits_lo(w[0]); v[1] = bf16_bits_hi(w[0]);
    v[2] = bf16_bits_lo(w[1]); v[3] = bf16_bits_hi(w[1]);
  } else {
    floatx4 w = *(const floatx4*)p;
    v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
  }
}

template <class T>
struct EpiStore {                       // C[row, col] = storage(v)
  struct P { T* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) p.C[g * p.c_gstride + (int64_t)row * p.ldc + col] = from_f32<T>(v);
  }
  __device__ static void at4(const P& p, int g, int row, int col, const float v[4]) {
    T* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
    if (col + 4 <= p.N) {
      store4<T>(c, v, (p.ldc & 3) == 0);
    } else {
      for (int i = 0; i < 4 && col + i < p.N; ++i) c[i] = from_f32<T>(v[i]);
    }
  }
};

template <int kUnused>
struct EpiStoreF32T {                   // C[row, col] = v   (fp32 output)
  struct P { float* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) p.C[g * p.c_gstride + (int64_t)row * p.ldc + col] = v;
  }
  __device__ static void at4(const P& p, int g, int row, int col, const float v[4]) {
    float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
    if (col + 4 <= p.N) {
      store4<float>(c, v, (p.ldc & 3) == 0);
    } else {
      for (int i = 0; i < 4 && col + i < p.N; ++i) c[i] = v[i];
    }
  }
};

template <int kUnused>
struct EpiAccumF32T {                   // C[row, col] += v  (fp32, one writer per element)
  struct P { float* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void at(const P& p, int g, int row, int col, float v) {
    if (col < p.N) {
      float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
      *c = *c + v;
    }
  }
  __device__ static void at4(const P& p, int g, int row, int col, const float v[4]) {
    float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
    if (col + 4 <= p.N && (p.ldc & 3) == 0) {
      float o[4];
      load4<float>(c, o);
      float w[4] = {o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]};
      store4<float>(c, w, true);
    } else {
      for (int i = 0; i < 4 && col + i < p.N; ++i) c[i] = c[i] + v[i];
    }
  }
};

// (class templates: kernel instantiations over plain-struct epilogues lose
// their host launch stubs with this compiler)
using EpiStoreF32 = EpiStoreF32T<0>;
using EpiAccumF32 = EpiAccumF32T<0>;

// SwiGLU forward.  In the MFMA kernel each wave's B rows hold its gate
// columns followed by the matching up columns, so one lane holds H and U of
// the same (row, col).  The fp32 kernel reads gate row col and up row f+col.
template <class T>
struct EpiSwiGLU {
  struct P { T* act; T* hu; int64_t f; };  // act [rows, f], hu [rows, 2f] or NULL
  static constexpr bool kPaired = true;
  // tile-row r of a BN-row tile split over WN waves: wave part w = r / (BN/WN);
  // its first half are gate rows, its second half the matching up rows
  template <int BN, int WN>
  __device__ static int b_row_paired(const P& p, int nt, int r) {
    constexpr int PART = BN / WN, HALF = PART / 2;
    int w = r / PART, o = r % PART;
    int col = nt * (BN / 2) + w * HALF + (o % HALF);
    if (col >= p.f) return 1 << 30;
    return o >= HALF ? (int)p.f + col : col;
  }
  __device__ static void act_of(float h, float u, float& a) { a = h / (1.0f + expf(-h)) * u; }
  __device__ static void at_pair(const P& p, int row, int col, float h, float u) {
    if (col >= p.f) return;
    float a;
    act_of(h, u, a);
    p.act[(int64_t)row * p.f + col] = from_f32<T>(a);
    if (p.hu) {
      p.hu[(int64_t)row * 2 * p.f + col] = from_f32<T>(h);
      p.hu[(int64_t)row * 2 * p.f + p.f + col] = from_f32<T>(u);
    }
  }
  __device__ static void at_pair4(const P& p, int row, int col, const float h[4], const float u[4]) {
    if (col + 4 > p.f) {
      for (int i = 0; i < 4; ++i) at_pair(p, row, col + i, h[i], u[i]);
      return;
    }
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) act_of(h[i], u[i], a[i]);
    const bool vec = (p.f & 3) == 0;
    store4<T>(p.act + (int64_t)row * p.f + col, a, vec);
    if (p.hu) {
      store4<T>(p.hu + (int64_t)row * 2 * p.f + col, h, vec);
      store4<T>(p.hu + (int64_t)row * 2 * p.f + p.f + col, u, vec);
    }
  }
};

// SwiGLU backward inside the down-projection dgrad: v = dA[row, col]
template <class T>
struct EpiSwiGLUBwd {
  struct P { const T* hu; T* dhu; int64_t f; };
  static constexpr bool kPaired = false;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void grad(float dA, float h, float u, float& dh, float& du) {
    float sg = 1.0f / (1.0f + expf(-h));
    dh = dA * u * sg * (1.0f + h * (1.0f - sg));
    du = dA * h * sg;
  }
  __device__ static void at(const P& p, int, int row, int col, float dA) {
    if (col >= p.f) return;
    int64_t base = (int64_t)row * 2 * p.f;
    float dh, du;
    grad(dA, to_f32(p.hu[base + col]), to_f32(p.hu[base + p.f + col]), dh, du);
    p.dhu[base + col] = from_f32<T>(dh);
    p.dhu[base + p.f + col] = from_f32<T>(du);
  }
  __device__ static void at4(const P& p, int g, int row, int col, const float v[4]) {
    if (col + 4 > p.f || (p.f & 3) != 0) {
      for (int i = 0; i < 4; ++i) at(p, g, row, col + i, v[i]);
      return;
    }
    int64_t base = (int64_t)row * 2 * p.f;
    float h[4], u[4], dh[4], du[4];
    load4<T>(p.hu + base + col, h);
    load4<T>(p.hu + base + p.f + col, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) grad(v[i], h[i], u[i], dh[i], du[i]);
    store4<T>(p.dhu + base + col, dh, true);
    store4<T>(p.dhu + base + p.f + col, du, true);
  }
};

}  // namespace moe
