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

constexpr int kRawBufferFlags = 0x00020000;   // raw (unformatted) buffer, gfx9 family

// buffer resource over `bytes` bytes from `base`: accesses past the range are
// dropped (stores) or read as zero (loads)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}
enum GemmMode { DENSE = 0, RAGGED_M = 1, RAGGED_K = 2 };

// Position of the 16-byte chunk c of row r in an epilogue staging buffer of
// 128-byte rows: 16 consecutive rows written 8 bytes per lane, or 8 lanes
// reading each row's eight chunks, stay free of bank conflicts.
__device__ __forceinline__ int stage_swz(int r) { return (r ^ (r >> 3)) & 7; }

// 16-byte buffer store (device pass only: in the host pass a device builtin
// inside a helper makes the compiler drop later kernels' launch stubs).
// NT = true marks the store non-temporal (cache-policy bit 1, "nt" on gfx950):
// the line is not kept for reuse, so an output stream does not push operand
// panels out of L2.
template <bool NT = false>
__device__ __forceinline__ void store_b128(u32x4 v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, NT ? 2 : 0);
#endif
}

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
  int k_skip;              // RAGGED_K: groups with at most this many rows are left to another kernel
  int kchunk;              // split-K (bf16 kernels; DENSE, or RAGGED_K without offsets and G parts): output
                           // tile (m, n) is computed once per part s, over K range [s kchunk, (s+1) kchunk),
                           // into output block g = s (DENSE: kchunk a multiple of 64); 0: no split
};

// Persistent schedule over XCDs.  Workgroups are dispatched round-robin over
// the XCDs (block b -> XCD b % 8), so with X = min(G, 8) workgroup b is the
// (b / X)-th of the workgroups of XCD b % X.  Each XCD owns one contiguous run
// [lo, hi) of logical tiles for the whole launch and its workgroups stride
// through it: the tiles one L2 serves are neighbours at any time, and later
// tiles reuse the panels earlier ones brought in.  Runs split the work evenly:
// by tile count, except for ragged contractions, where a tile of group g costs
// kSplitAlpha + (off[g+1] - off[g]) (its store plus its contraction).
constexpr int kSplitAlpha = 64;

template <GemmMode MODE>
__device__ __forceinline__ int xcd_run_start(const GemmArgs& a, const int* off, int total, int P, int x, int X) {
  if (x >= X) return total;
  const int G = a.G;
  if (MODE == RAGGED_K && a.offsets && a.k_skip > 0) {
    // groups of at most k_skip rows cost nothing here.  Wave-parallel over
    // the groups (G <= 256): lane l owns groups 4l .. 4l+3, the lane sums are
    // scanned across the wave, and the run starts in the first group whose
    // cumulative cost passes W x / X (every wave computes the same value).
    // The first run starts at the first group that is not skipped, and with
    // no such group every run is empty.
    const int lane = threadIdx.x & 63;
    int64_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      const int n = e < G ? off[e + 1] - off[e] : 0;
      c[i] = n > a.k_skip ? (int64_t)P * (kSplitAlpha + n) : 0;
      sum += c[i];
    }
    auto shfl64 = [](int64_t v, int src) -> int64_t {
      const int lo = __shfl((int)(uint32_t)v, src, 64), hi = __shfl((int)(v >> 32), src, 64);
      return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    };
    int64_t incl = sum;                                   // inclusive scan over lanes
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t v = shfl64(incl, lane >= o ? lane - o : lane);
      if (lane >= o) incl += v;
    }
    const int64_t W = shfl64(incl, 63);
    const int64_t T = W * x / X;
    int64_t before = incl - sum;
    int found = -1;
    int64_t found_before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (found < 0 && before + c[i] > T) {
        found = 4 * lane + i;
        found_before = before;
      }
      before += c[i];
    }
    const uint64_t m = __ballot(found >= 0);
    if (m == 0) return total;
    const int src = __ffsll((unsigned long long)m) - 1;
    const int e = __shfl(found, src, 64);
    const int64_t b = shfl64(found_before, src);
    const int64_t ce = kSplitAlpha + (off[e + 1] - off[e]);   // one tile of group e
    const int64_t in = (T - b + ce - 1) / ce;
    return e * P + (int)(in < P ? in : P);
  }
  if (x <= 0) return 0;
  if (MODE != RAGGED_K || !a.offsets) return (int)((int64_t)total * x / X);
  auto cum = [&](int e) -> int64_t { return (int64_t)e * kSplitAlpha + (off[e] - off[0]); };
  const int64_t T = (int64_t)P * cum(G) * x / X;             // work before the run, in tile units
  int lo = 0, hi = G;                                        // last e < G with P cum(e) <= T
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)P * cum(mid) <= T) lo = mid; else hi = mid;
  }
  const int64_t ce = kSplitAlpha + (off[lo + 1] - off[lo]);
  const int64_t in = (T - (int64_t)P * cum(lo)) / ce;
  return lo * P + (int)(in < P ? in : P);
}

// Scales of MXFP8 operands (e8m0 bytes, one per 32 K values, K/32 per row).
//
// Operand layout of the scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (32 rows
// x 64 K per step, 32 bytes per lane), as a probe on the GPU fixed it: lane l
// (h = l / 32) holds row l % 32, bytes 0-15 = 16 K values of the step's first
// 32-block and bytes 16-31 = 16 K values of its second; lanes l and l + 32
// together cover each block.  With a 128-value slice as eight 16-byte chunks
// per row, lane half h takes chunks 4 s + h and 4 s + 2 + h in step s.  The
// scale of (row, block b) comes from lane row + 32 b, so each lane passes the
// scale of block h of its own row; a row's scale word holds the slice's four
// block scales, shifted by 8 h per lane, and op_sel picks byte 2 s for step s.
// Scale layouts of a quantised matrix of R rows with nb blocks (of 32 values)
// per row.  Plain: the scale of block b of row r at byte r nb + b.  Grouped
// (nb a multiple of 4): the scales of blocks 4q .. 4q+3 of a row form one
// 4-byte word, and the words of group q for rows 0 .. R-1 are consecutive:
// byte 4 (q R + r) + b % 4.  A GEMM slice of 128 fp8 (or 256 fp4) values then
// needs one (two) such words per row, and the words of a tile's rows are
// adjacent in memory.
__host__ __device__ __forceinline__ int64_t mx_scale_at(int64_t r, int b, int64_t R, int nb, bool grouped) {
  return grouped ? ((int64_t)(b >> 2) * R + r) * 4 + (b & 3) : r * nb + b;
}

struct MxArgs {
  const uint8_t* A_s;      // A scales, grouped over a_rows rows
  const uint8_t* B_s;      // B scales, grouped over b_rows rows (per group: + g * b_s_gstride)
  int64_t a_rows, b_rows;
  int64_t b_s_gstride;
};

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

struct TileCoord {
  int g;        // group
  int m0;       // first row of the tile (absolute row of A/C for RAGGED_M)
  int m_end;    // rows >= m_end are outside the group
  int n0;       // first column (tile-local meaning for paired epilogues)
  int k_begin;  // contraction range of this group
  int k_end;
};

// Resolve a logical tile index.  `off` / `pre` are the ragged offsets and the
// tile prefix (a copy in LDS or the global arrays of `a`).
template <GemmMode MODE, int BM>
__device__ __forceinline__ void resolve_tile(const GemmArgs& a, const int* off, const int* pre, int L, int NT,
                                             int MT, TileCoord& c) {
  if (MODE == DENSE) {
    // split-K: part s of every output tile, then part s + 1
    const int s = L / (MT * NT), r = L % (MT * NT);
    int mt = r % MT, nt = r / MT;
    c.g = s; c.m0 = mt * BM; c.m_end = a.M; c.n0 = nt;
    c.k_begin = a.kchunk > 0 ? s * a.kchunk : 0;
    c.k_end = a.kchunk > 0 ? min(a.K, c.k_begin + a.kchunk) : a.K;
  } else if (MODE == RAGGED_M) {
    // expert-major order: all tiles of group g, n-tile major, m-tile fastest
    int lo = 0, hi = a.G;  // find g with pre[g]*NT <= L < pre[g+1]*NT
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (pre[mid] * NT <= L) lo = mid; else hi = mid;
    }
    int g = lo;
    int first = pre[g], mt_g = pre[g + 1] - first;
    int local = L - first * NT;
    int nt = local / mt_g, mi = local % mt_g;
    int row0 = off[g];
    c.g = g; c.m0 = row0 + mi * BM; c.m_end = off[g + 1]; c.n0 = nt;
    c.k_begin = 0; c.k_end = a.K;
  } else {
    // group-major; inside a group, bands of kBandM m-tiles walked n-tile by
    // n-tile (m fastest inside the band).  64 consecutive tiles (what the
    // workgroups of one XCD hold at a time) are then about 8 x 8 tiles: they
    // read 8 row blocks of each operand once and reuse each 8 times from L2,
    // instead of re-reading one operand's whole panel for every row of tiles.
    constexpr int kBandM = 8;
    int per = MT * NT;
    int g = L / per, r = L % per;
    int band = r / (kBandM * NT), in = r % (kBandM * NT);
    int bm = min(kBandM, MT - band * kBandM);
    int mt = band * kBandM + in % bm, nt = in / bm;
    c.g = g; c.m0 = mt * BM; c.m_end = a.M; c.n0 = nt;
    // no offsets: one contraction [0, K), or with kchunk > 0 group g's part
    // [g kchunk, (g+1) kchunk) of it (split-K)
    c.k_begin = a.offsets ? off[g] : a.kchunk > 0 ? g * a.kchunk : 0;
    c.k_end = a.offsets ? off[g + 1] : a.kchunk > 0 ? min(a.K, (g + 1) * a.kchunk) : a.K;
  }
}

template <GemmMode MODE, int BM>
__device__ __forceinline__ void resolve_tile(const GemmArgs& a, int L, int NT, int MT, TileCoord& c) {
  resolve_tile<MODE, BM>(a, a.offsets, a.tile_prefix, L, NT, MT, c);
}

// ---------------------------------------------------------------------------
// LDS slices of row-contiguous ("MC") operands.  A slice is kept as it lies in
// memory: K-rows of ROWS values (ROWS/8 16-byte chunks each), logical chunk c
// of K-row k at position c ^ mc_mask(k, c).  MFMA fragments are read with
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i%4
// of the 8-byte piece addressed by lane i/4 + 4j (j = 0..3).  Pointing lane q
// at K-row k0 + q/4, columns n0 + 4(q%4) .. +3 hands lane i the four K values
// k0..k0+3 of column n0 + i.  A cycle's 32 lanes touch 4 K-rows x 4 chunks,
// which the XOR spreads over all 16 chunk positions of the 64 banks; 16 lanes
// writing one K-row's 16 chunks also land on distinct positions.
// ---------------------------------------------------------------------------
#define MOE_LDS __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4i16;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short v8i16;

__device__ __forceinline__ int mc_mask(int k, int c) { return ((k & 3) << 1) | (((c >> 1) & 1) << 3); }

// Fragment reads of NF fragments of 32 tile rows (row0 + 32 f) from an MC
// slice of ROWS columns; per-lane byte offsets are computed once.
template <int ROWS, int NF>
struct McFrag {
  static constexpr int CPR = ROWS / 8;
  uint32_t off[NF];

  __device__ __forceinline__ void init(int row0) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, q = lane & 15;
    const int klane = 8 * (g >> 1) + (q >> 2);             // K-row within a 16-step
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = row0 + 32 * f + 16 * (g & 1) + 4 * (q & 3);
      const int c = n >> 3, half = q & 1;
      off[f] = (uint32_t)(klane * CPR * 16 + ((c ^ mc_mask(klane, c)) * 16) + half * 8);
    }
  }
  // fragment f, K-step kk; `base` = LDS byte address of the slice
  __device__ __forceinline__ bf16x8 read(uint32_t base, int f, int kk) const {
#if defined(__HIP_DEVICE_COMPILE__)
    // K-rows kk*16 + {0..3} and kk*16 + {4..7}: k & 3 is unchanged, so the XOR is too
    const uint32_t a = base + off[f] + (uint32_t)(kk * 16 * CPR * 16);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS v4i16*)(uintptr_t)a);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS v4i16*)(uintptr_t)(a + 4 * CPR * 16));
    v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
#else
    return bf16x8{};
#endif
  }
};

// Total logical tiles (device side; RAGGED_M depends on the expert sizes).
template <GemmMode MODE>
__device__ __forceinline__ int total_tiles(const GemmArgs& a, int NT, int MT) {
  if (MODE == RAGGED_M) return a.tile_prefix[a.G] * NT;
  if (MODE == RAGGED_K) return a.G * MT * NT;
  return MT * NT * (a.kchunk > 0 ? (a.K + a.kchunk - 1) / a.kchunk : 1);
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

// kSite only tells launch sites apart (distinct kernel symbols for profiles)
template <class T, int kSite = 0>
struct EpiStore {                       // C[row, col] = storage(v)
  struct P { T* C; int64_t ldc; int64_t c_gstride; int M; int N; };
  static constexpr bool kPaired = false;
  static constexpr bool kRowDot = false;
  // 2-byte outputs may be staged through LDS and stored 8 columns at a time
  static constexpr bool kStaged = sizeof(T) == 2;
  static constexpr bool kAccum = false;
  static constexpr bool kQuant = false;
  __device__ static void store8(const P& p, int g, int row, int col, u32x4 v) {
    uint16_t* c = (uint16_t*)(p.C + g * p.c_gstride + (int64_t)row * p.ldc + col);
    if (col + 8 <= p.N && (p.ldc & 7) == 0) {
      *(u32x4*)c = v;
    } else {
      for (int i = 0; i < 8 && col + i < p.N; ++i) c[i] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
    }
  }
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
  static constexpr bool kRowDot = false;
  static constexpr bool kStaged = false;
  static constexpr bool kAccum = false;
  static constexpr bool kQuant = false;
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
  static constexpr bool kRowDot = false;
  static constexpr bool kStaged = false;
  // the MFMA kernel reads a 32-row fragment's old values (old4) before it
  // writes any of them (add4), so the reads' latency is paid once per fragment
  static constexpr bool kAccum = true;
  static constexpr bool kQuant = false;
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
  __device__ static void old4(const P& p, int g, int row, int col, float o[4]) {
    const float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
    if (col + 4 <= p.N && (p.ldc & 3) == 0) {
      load4<float>(c, o);
    } else {
      for (int i = 0; i < 4; ++i) o[i] = col + i < p.N ? c[i] : 0.0f;
    }
  }
  __device__ static void add4(const P& p, int g, int row, int col, const float v[4], const float o[4]) {
    float* c = p.C + g * p.c_gstride + (int64_t)row * p.ldc + col;
    const float w[4] = {o[0] + v[0], o[1] + v[1], o[2] + v[2], o[3] + v[3]};
    if (col + 4 <= p.N && (p.ldc & 3) == 0) {
      store4<float>(c, w, true);
    } else {
      for (int i = 0; i < 4 && col + i < p.N; ++i) c[i] = w[i];
    }
  }
};

// (class templates: kernel instantiations over plain-struct epilogues lose
// their host launch stubs with this compiler)
using EpiStoreF32 = EpiStoreF32T<0>;
using EpiAccumF32 = EpiAccumF32T<0>;

// ---- MX block quantisation (one e8m0 scale per 32 consecutive values) -----
// The rule itself is stated where the quantisation kernels are (mxfp8.hip);
// these are its per-block steps, shared with the GEMM epilogues that emit the
// row form of their output.
// smallest e with 448 * 2^e >= amax, clamped to [-127, 127]
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0x1.cp-119f)) return -127;            // amax <= 448 * 2^-127 (or 0)
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFF) - 127;         // amax = m 2^E, m in [1, 2)
  const int e = (b & 0x7FFFFFu) <= 0x600000u ? E - 8 : E - 7;   // m <= 1.75 : 1.75 2^E >= amax
  return e > 127 ? 127 : e;
}

// smallest e with 6 * 2^e >= amax, clamped to [-127, 127]
__device__ __forceinline__ int mx4_exponent(float amax) {
  if (!(amax > 0x1.8p-125f)) return -127;            // amax <= 6 * 2^-127 (or 0)
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFF) - 127;         // amax = m 2^E, m in [1, 2)
  const int e = (b & 0x7FFFFFu) <= 0x400000u ? E - 2 : E - 1;   // m <= 1.5 : 1.5 2^E >= amax
  return e > 127 ? 127 : e;
}

// e2m1 codes of v0 (low nibble) and v1 (high nibble) into byte SEL of `old`:
// each the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with v's sign, ties to the
// even code, saturating at 6.  gfx950's scaled conversion with scale 1 rounds
// exactly so (compared value by value, ties and saturation included).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pk(uint32_t old, float v0, float v1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, v0, v1, 1.0f, SEL);
}

// 16 bf16 values from 8 pairs (element 2i in the low half of word i)
__device__ __forceinline__ void unpack_bf16x16(const uint32_t w[8], float v[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_bits_lo(w[i]);
    v[2 * i + 1] = bf16_bits_hi(w[i]);
  }
}

// One block of 32 values of a row held by the lane pair (l, l ^ 32) of a wave,
// as an MFMA accumulator row holds them: the lane of half h = (l >> 5) & 1 has
// v[4q + e] = value 8q + 4h + e of the block (q, e = 0..3).  Writes the
// block's codes at `codes` (fp8: 32 bytes; fp4: 16, element 2i in the low
// nibble) and, from half 0, its scale byte at `scale`: the codes and scale the
// row quantiser gives the same 32 values.  Both lanes of the pair must run it.
__device__ __forceinline__ void mx_quant_pair(const float v[16], bool fp4, uint8_t* codes, uint8_t* scale) {
  const int h = (int)((threadIdx.x >> 5) & 1);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  // each lane ends with 16 contiguous code bytes (fp4: 8): half 0 the first
  // 16 values of the block, half 1 the rest, swapping the pieces it lacks
  if (!fp4) {
    const int e = mx_exponent(amax);
    uint32_t w[4];                                     // codes of values 8q + 4h .. +3
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * q], -e), ldexpf(v[4 * q + 1], -e), 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * q + 2], -e), ldexpf(v[4 * q + 3], -e), word, true);
      w[q] = (uint32_t)word;
    }
    const uint32_t r0 = (uint32_t)__shfl_xor((int)(h ? w[0] : w[2]), 32, 64);
    const uint32_t r1 = (uint32_t)__shfl_xor((int)(h ? w[1] : w[3]), 32, 64);
    *(u32x4*)(codes + 16 * h) = h ? u32x4{r0, w[2], r1, w[3]} : u32x4{w[0], r0, w[1], r1};
    if (h == 0) *scale = (uint8_t)(e + 127);
  } else {
    const int e = mx4_exponent(amax);
    uint32_t hw[4];                                    // 16 bits: values 8q + 4h .. +3
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x = e2m1_pk<0>(0u, ldexpf(v[4 * q], -e), ldexpf(v[4 * q + 1], -e));
      hw[q] = e2m1_pk<1>(x, ldexpf(v[4 * q + 2], -e), ldexpf(v[4 * q + 3], -e));
    }
    const uint32_t r = (uint32_t)__shfl_xor((int)(h ? (hw[0] | hw[1] << 16) : (hw[2] | hw[3] << 16)), 32, 64);
    *(u32x2*)(codes + 8 * h) = h ? u32x2{(r & 0xFFFFu) | hw[2] << 16, (r >> 16) | hw[3] << 16}
                                 : u32x2{hw[0] | (r & 0xFFFFu) << 16, hw[1] | (r >> 16) << 16};
    if (h == 0) *scale = (uint8_t)(e + 127);
  }
}

// SwiGLU output of one element: silu(h) * u, times the row's gate g when gates
// are folded.  The forward (with act formed from the stored H, U) and the
// backward that forms act again both go through this one function, so the two
// are the same instructions on the same inputs and agree bit for bit.
__device__ __forceinline__ float swiglu_act(float h, float u, float g) { return g * (h / (1.0f + expf(-h)) * u); }

// value of v after a round trip through storage type T (identity for fp32)
template <class T>
__device__ __forceinline__ float through(float v) { return to_f32(from_f32<T>(v)); }

// SwiGLU forward.  In the MFMA kernel each wave's B rows hold its gate
// columns followed by the matching up columns, so one lane holds H and U of
// the same (row, col).  The fp32 kernel reads gate row col and up row f+col.
// row_gates (folded gates, [rows] fp32) multiplies act; from_stored forms act
// from H and U as stored (rounded to T) rather than from the fp32 results.
template <class T>
struct EpiSwiGLU {
  struct P {
    T* act; T* hu; int64_t f;             // act [rows, f], hu [rows, 2f] or NULL
    const float* row_gates = nullptr;     // gate of each row (folded gates) or NULL
    int from_stored = 0;
    // the MX row form of act as stored, or NULL: codes [rows, f] (fp4:
    // [rows, f/2]) and scales [rows, f/32] (MFMA kernel only)
    uint8_t* q_codes = nullptr;
    uint8_t* q_scales = nullptr;          // grouped over q_rows rows
    int q_fp4 = 0;
    int64_t q_rows = 0;
  };
  static constexpr bool kPaired = true;
  static constexpr bool kStaged = false;
  static constexpr bool kAccum = false;
  static constexpr bool kRowDot = false;
  static constexpr bool kQuant = true;
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
  __device__ static float act_of(const P& p, float h, float u, float g) {
    if (p.from_stored) return swiglu_act(through<T>(h), through<T>(u), g);
    return swiglu_act(h, u, g);
  }
  __device__ static float gate_of(const P& p, int row) { return p.row_gates ? p.row_gates[row] : 1.0f; }
  __device__ static void at_pair(const P& p, int row, int col, float h, float u) {
    if (col >= p.f) return;
    const float a = act_of(p, h, u, gate_of(p, row));
    p.act[(int64_t)row * p.f + col] = from_f32<T>(a);
    if (p.hu) {
      p.hu[(int64_t)row * 2 * p.f + col] = from_f32<T>(h);
      p.hu[(int64_t)row * 2 * p.f + p.f + col] = from_f32<T>(u);
    }
  }
  // Q: a_st receives the four act values as stored (zeros past f)
  template <bool Q>
  __device__ __forceinline__ static void at_pair4_impl(const P& p, int row, int col, const float h[4],
                                                       const float u[4], float* a_st) {
    if constexpr (Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a_st[i] = 0.0f;
    }
    if (col + 4 > p.f) {
      for (int i = 0; i < 4; ++i) at_pair(p, row, col + i, h[i], u[i]);
      return;
    }
    float a[4];
    const float g = gate_of(p, row);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = act_of(p, h[i], u[i], g);
    const bool vec = (p.f & 3) == 0;
    store4<T>(p.act + (int64_t)row * p.f + col, a, vec);
    if (p.hu) {
      store4<T>(p.hu + (int64_t)row * 2 * p.f + col, h, vec);
      store4<T>(p.hu + (int64_t)row * 2 * p.f + p.f + col, u, vec);
    }
    if constexpr (Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a_st[i] = through<T>(a[i]);
    }
  }
  __device__ static void at_pair4(const P& p, int row, int col, const float h[4], const float u[4], float a_st[4]) {
    at_pair4_impl<true>(p, row, col, h, u, a_st);
  }
  __device__ static void at_pair4(const P& p, int row, int col, const float h[4], const float u[4]) {
    at_pair4_impl<false>(p, row, col, h, u, nullptr);
  }
  // the MX block of act at columns col0 .. col0 + 31 of `row`: the lane's 16
  // values of it (mx_quant_pair's layout) as bf16 pairs
  __device__ static void quant_block(const P& p, int row, int col0, const uint32_t a_st[8]) {
    float v[16];
    unpack_bf16x16(a_st, v);
    uint8_t* codes = p.q_codes + (p.q_fp4 ? (int64_t)row * (p.f / 2) + col0 / 2 : (int64_t)row * p.f + col0);
    mx_quant_pair(v, p.q_fp4 != 0, codes, p.q_scales + mx_scale_at(row, col0 / 32, p.q_rows, (int)(p.f / 32), true));
  }
};

// SwiGLU backward inside the down-projection dgrad: v = dA[row, col].
// Folded gates (row_gates): the product gives dA of g*act, so the row's gate
// gradient gets the term dA * silu(h) u (returned by at / at4, summed by the
// kernel over each 64-column block of the row into dg_part) and dH, dU use
// g * dA.  act_out (act formed again from the stored H, U, times g) is written
// when the backward recomputes act.
template <class T>
struct EpiSwiGLUBwd {
  struct P {
    const T* hu; T* dhu; int64_t f;
    const float* row_gates = nullptr;     // folded gates [rows] or NULL
    float* dg_part = nullptr;             // [rows, dg_ld] gate-gradient partials (with row_gates)
    int dg_ld = 0;
    T* act_out = nullptr;                 // [rows, f] act formed again, or NULL
    // the MX row form of dHU as stored (blocks along its 2f columns), or
    // NULL: codes [rows, 2f] (fp4: [rows, f]) and scales grouped over q_rows rows
    uint8_t* q_codes = nullptr;
    uint8_t* q_scales = nullptr;
    int q_fp4 = 0;
    int64_t q_rows = 0;
  };
  static constexpr bool kPaired = false;
  static constexpr bool kStaged = false;
  static constexpr bool kAccum = false;
  static constexpr bool kRowDot = true;   // the kernels reduce at's return value when dg_part is set
  static constexpr bool kQuant = true;
  __device__ static int b_row(const P&, int nt, int r, int BN) { return nt * BN + r; }
  __device__ static void grad(float dA, float h, float u, float& dh, float& du) {
    float sg = 1.0f / (1.0f + expf(-h));
    dh = dA * u * sg * (1.0f + h * (1.0f - sg));
    du = dA * h * sg;
  }
  __device__ static float at(const P& p, int, int row, int col, float dA) {
    if (col >= p.f) return 0.0f;
    int64_t base = (int64_t)row * 2 * p.f;
    const float h = to_f32(p.hu[base + col]), u = to_f32(p.hu[base + p.f + col]);
    const float g = p.row_gates ? p.row_gates[row] : 1.0f;
    float dot = 0.0f;
    if (p.row_gates) dot = dA * swiglu_act(h, u, 1.0f);
    if (p.act_out) p.act_out[(int64_t)row * p.f + col] = from_f32<T>(swiglu_act(h, u, g));
    float dh, du;
    grad(g * dA, h, u, dh, du);
    p.dhu[base + col] = from_f32<T>(dh);
    p.dhu[base + p.f + col] = from_f32<T>(du);
    return dot;
  }
  // Q: dh_st, du_st receive the dH and dU values as stored (zeros past f)
  template <bool Q>
  __device__ __forceinline__ static float at4_impl(const P& p, int g_, int row, int col, const float v[4],
                                                   float* dh_st, float* du_st) {
    if constexpr (Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dh_st[i] = du_st[i] = 0.0f;
    }
    if (col + 4 > p.f || (p.f & 3) != 0) {
      float dot = 0.0f;
      for (int i = 0; i < 4; ++i) dot += at(p, g_, row, col + i, v[i]);
      return dot;
    }
    int64_t base = (int64_t)row * 2 * p.f;
    float h[4], u[4], dh[4], du[4];
    load4<T>(p.hu + base + col, h);
    load4<T>(p.hu + base + p.f + col, u);
    const float g = p.row_gates ? p.row_gates[row] : 1.0f;
    float dot = 0.0f;
    if (p.row_gates) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dot += v[i] * swiglu_act(h[i], u[i], 1.0f);
    }
    if (p.act_out) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = swiglu_act(h[i], u[i], g);
      store4<T>(p.act_out + (int64_t)row * p.f + col, a, true);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) grad(g * v[i], h[i], u[i], dh[i], du[i]);
    store4<T>(p.dhu + base + col, dh, true);
    store4<T>(p.dhu + base + p.f + col, du, true);
    if constexpr (Q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dh_st[i] = through<T>(dh[i]);
        du_st[i] = through<T>(du[i]);
      }
    }
    return dot;
  }
  __device__ static float at4(const P& p, int g_, int row, int col, const float v[4], float dh_st[4],
                              float du_st[4]) {
    return at4_impl<true>(p, g_, row, col, v, dh_st, du_st);
  }
  __device__ static float at4(const P& p, int g_, int row, int col, const float v[4]) {
    return at4_impl<false>(p, g_, row, col, v, nullptr, nullptr);
  }
  // the MX blocks of dH and dU at columns col0 .. col0 + 31 of `row` (each
  // lane's 16 values of each as bf16 pairs)
  __device__ static void quant_block(const P& p, int row, int col0, const uint32_t dh_st[8], const uint32_t du_st[8]) {
    const int64_t f2 = 2 * p.f;
    uint8_t* cr = p.q_codes + (p.q_fp4 ? (int64_t)row * p.f : (int64_t)row * f2);
    const bool fp4 = p.q_fp4 != 0;
    const int nb = (int)(f2 / 32);
    float v[16];
    unpack_bf16x16(dh_st, v);
    mx_quant_pair(v, fp4, cr + (fp4 ? col0 / 2 : col0), p.q_scales + mx_scale_at(row, col0 / 32, p.q_rows, nb, true));
    unpack_bf16x16(du_st, v);
    mx_quant_pair(v, fp4, cr + (fp4 ? (p.f + col0) / 2 : p.f + col0),
                  p.q_scales + mx_scale_at(row, (int)((p.f + col0) / 32), p.q_rows, nb, true));
  }
};

}  // namespace moe
