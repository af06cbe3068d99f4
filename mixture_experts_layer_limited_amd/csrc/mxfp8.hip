// MXFP8 / MXFP4 path: quantisation of bf16 tensors to fp8 e4m3 (or fp4
// e2m1) codes with one e8m0 scale per 32 consecutive values, and the
// scaled-MFMA grouped GEMMs.
//
// MXFP4 follows the same rule with e2m1 elements (largest magnitude 6: e is
// the smallest integer with 6 * 2^e >= amax) and stores two codes per byte,
// element 2i in the low nibble; a 128-byte slice row then holds 256 values.
//
// Quantisation rule (block of 32 values, amax = largest magnitude): the scale
// is 2^e with e the smallest integer such that 448 * 2^e >= amax, clamped to
// [-127, 127] (amax = 0 gives e = -127 and zero codes); it is stored as the
// byte e + 127.  Each value v becomes the e4m3fn code nearest to v / 2^e
// (ties to the even code), saturating at +-448.  Both steps are exact integer
// and power-of-two arithmetic on the fp32 image of the bf16 input.
//
// Layouts:
//   rows  : codes [R][C], scales [R][C/32]   (blocks along the contiguous C)
//   cols  : codes [C][R], scales [C][R/32]   (transposed copy, blocks along R:
//           the weights for the products that contract over their rows)
// Scales come plain (as above) or grouped (mx_scale_at in gemm.hpp: four
// block scales of a row per word, the words of consecutive rows adjacent),
// the layout the microscaled GEMMs read; codes are the same in both.
// The weight gradients contract over the token rows: their operands are
// quantised along the rows (32-row blocks restarting at each expert's first
// row) and widened back to bf16 (mx_qdq_rows).
#include <stdint.h>

#include "common.hpp"
#include "gemm.hpp"
#include "gemm_mfma.hpp"
#include "gemm_regs.hpp"
#include "kernels.hpp"

namespace moe {

// quantise 32 fp32 values; returns the scale byte
__device__ __forceinline__ uint32_t mx_block(const float v[32], uint32_t out[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  // v_cvt_pk_fp8_f32: the nearest e4m3fn code, ties to the even code (|v| / 2^e
  // <= 448 by the choice of e, so nothing reaches the saturation)
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w], -e), ldexpf(v[4 * w + 1], -e), 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * w + 2], -e), ldexpf(v[4 * w + 3], -e), word, true);
    out[w] = (uint32_t)word;
  }
  return (uint32_t)(e + 127);
}

// quantise 32 fp32 values to e2m1 (16 bytes, element 2i in the low nibble);
// returns the scale byte
__device__ __forceinline__ uint32_t mx4_block(const float v[32], uint32_t out[4]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx4_exponent(amax);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float* x = v + 8 * w;
    uint32_t word = e2m1_pk<0>(0u, ldexpf(x[0], -e), ldexpf(x[1], -e));
    word = e2m1_pk<1>(word, ldexpf(x[2], -e), ldexpf(x[3], -e));
    word = e2m1_pk<2>(word, ldexpf(x[4], -e), ldexpf(x[5], -e));
    out[w] = e2m1_pk<3>(word, ldexpf(x[6], -e), ldexpf(x[7], -e));
  }
  return (uint32_t)(e + 127);
}

// ---------------------------------------------------------------------------
// Row form: one thread per 32-block.  src [batch][R][ld] bf16 ->
// codes [batch][R][C], scales [batch][R][C/32].
// ---------------------------------------------------------------------------
template <bool FP4>
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const uint16_t* __restrict__ src, int64_t ld,
                                                            int64_t src_bstride, int R, int C,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, bool grouped) {
  const int nb = C / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)R * nb) return;
  const int64_t bt = blockIdx.y;
  const int r = (int)(t / nb), b = (int)(t % nb);
  const u32x4* p = (const u32x4*)(src + bt * src_bstride + (int64_t)r * ld + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 w = p[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_bits_lo(w[j]);
      v[8 * i + 2 * j + 1] = bf16_bits_hi(w[j]);
    }
  }
  uint32_t sb;
  if constexpr (FP4) {
    uint32_t out[4];
    sb = mx4_block(v, out);
    *(u32x4*)(codes + (bt * R + r) * (int64_t)(C / 2) + b * 16) = u32x4{out[0], out[1], out[2], out[3]};
  } else {
    uint32_t out[8];
    sb = mx_block(v, out);
    u32x4* q = (u32x4*)(codes + (bt * R + r) * (int64_t)C + b * 32);
    q[0] = u32x4{out[0], out[1], out[2], out[3]};
    q[1] = u32x4{out[4], out[5], out[6], out[7]};
  }
  scales[bt * R * (int64_t)nb + mx_scale_at(r, b, R, nb, grouped)] = (uint8_t)sb;
}

hipError_t launch_mx_quant_rows(const void* src, int64_t ld, int64_t src_bstride, int batch, int R, int C,
                                uint8_t* codes, uint8_t* scales, bool fp4, bool grouped, hipStream_t st) {
  const int64_t n = (int64_t)R * (C / 32);
  if (n == 0 || batch == 0) return hipSuccess;
  if (grouped && C % 128) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + 255) / 256), batch);
  if (fp4)
    mx_quant_rows_kernel<true><<<grid, 256, 0, st>>>((const uint16_t*)src, ld, src_bstride, R, C, codes, scales,
                                                     grouped);
  else
    mx_quant_rows_kernel<false><<<grid, 256, 0, st>>>((const uint16_t*)src, ld, src_bstride, R, C, codes, scales,
                                                      grouped);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column form (the weights' transposed copies): a workgroup takes 128 rows
// (four 32-row blocks) by 64 columns.  The tile is read with 16-byte row loads
// into LDS; thread (column c, block b) then quantises its 32 values and writes
// 32 contiguous code bytes, so the four blocks of a column (four adjacent
// lanes) fill one 128-byte line.  src [rows][ld] bf16, codes [C][ldq],
// scales [C][ldq/32]; rows past `rows` below rp_limit are zero codes, rows at
// or past rp_limit are not written.
// ---------------------------------------------------------------------------
constexpr int kQcRows = 128, kQcCols = 64;

// FP4: codes [C][ldq / 2] (two per byte), 16 bytes per block
// ROWS_TOO: the same launch also writes the row form of the tile (codes_r
// [R][C], scales_r [R][C/32] per matrix; rows = rp_limit = R, a multiple of
// 32, C of 32), so a weight is read once for both forms.
template <bool FP4, bool ROWS_TOO = false>
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(const uint16_t* __restrict__ src, int64_t ld,
                                                            int rows, int C, int64_t ldq,
                                                            int rp_limit, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t z_src,
                                                            int64_t z_codes, bool grouped,
                                                            uint8_t* __restrict__ codes_r = nullptr,
                                                            uint8_t* __restrict__ scales_r = nullptr) {
  __shared__ uint16_t tile[kQcRows][kQcCols];
  // grid z: independent matrices (a batch of weights), z_src elements and
  // z_codes values apart (z_codes code bytes for fp8, half that for fp4;
  // z_codes / 32 scale bytes)
  src += blockIdx.z * z_src;
  codes += blockIdx.z * (FP4 ? z_codes / 2 : z_codes);
  scales += blockIdx.z * (z_codes / 32);
  const int rp0 = blockIdx.x * kQcRows;
  const int c0 = blockIdx.y * kQcCols;
  // every tile below rp_limit is written (rows past `rows` as zero codes)
  if (rp0 >= rp_limit) return;
  const int src0 = rp0;                                 // source rows of this tile: src0 .. src0+n-1
  int n = rows - rp0;
  n = n < 0 ? 0 : (n > kQcRows ? kQcRows : n);
  // 128 rows x 8 chunks of 16 bytes; columns past C and rows past n read as 0
  for (int q = threadIdx.x; q < kQcRows * (kQcCols / 8); q += 256) {
    const int r = q >> 3, ch = q & 7;
    const int c = c0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < n && c + 8 <= C) v = *(const u32x4*)(src + (int64_t)(src0 + r) * ld + c);
    *(u32x4*)&tile[r][(ch ^ ((r >> 5) << 1)) * 8] = v;  // block b's chunks XOR 2b
  }
  __syncthreads();
  if constexpr (ROWS_TOO) {
    // thread t: row t / 2 of the tile, its 32-column block t % 2
    const int r = threadIdx.x >> 1, bb = threadIdx.x & 1, cb = c0 + 32 * bb;
    if (r < n && cb + 32 <= C) {
      float v[32];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 w = *(const u32x4*)&tile[r][((4 * bb + k) ^ ((r >> 5) << 1)) * 8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * k + 2 * j] = bf16_bits_lo(w[j]);
          v[8 * k + 2 * j + 1] = bf16_bits_hi(w[j]);
        }
      }
      const int64_t row = (int64_t)blockIdx.z * rows + src0 + r;
      uint32_t sb;
      if constexpr (FP4) {
        uint32_t out[4];
        sb = mx4_block(v, out);
        *(u32x4*)(codes_r + row * (C / 2) + cb / 2) = u32x4{out[0], out[1], out[2], out[3]};
      } else {
        uint32_t out[8];
        sb = mx_block(v, out);
        u32x4* q = (u32x4*)(codes_r + row * C + cb);
        q[0] = u32x4{out[0], out[1], out[2], out[3]};
        q[1] = u32x4{out[4], out[5], out[6], out[7]};
      }
      scales_r[(int64_t)blockIdx.z * rows * (C / 32) + mx_scale_at(src0 + r, cb / 32, rows, C / 32, grouped)] =
          (uint8_t)sb;
    }
  }
  // wave w takes columns 16w .. 16w+15 and lane (4j + b) block b of column
  // 16w + j: the four blocks of a column, one 128-byte code line, come from
  // adjacent lanes; the XOR puts the 4 x 16 columns on 32 distinct banks
  const int c = 16 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 2), b = threadIdx.x & 3;
  const int rb = rp0 + 32 * b;
  if (c0 + c >= C || rb >= rp_limit) return;
  const int pc = (((c >> 3) ^ (b << 1)) << 3) | (c & 7);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = bf16_bits_lo(tile[32 * b + i][pc]);
  uint32_t sb;
  if constexpr (FP4) {
    uint32_t out[4];
    sb = mx4_block(v, out);
    *(u32x4*)(codes + (int64_t)(c0 + c) * (ldq / 2) + rb / 2) = u32x4{out[0], out[1], out[2], out[3]};
  } else {
    uint32_t out[8];
    sb = mx_block(v, out);
    u32x4* q = (u32x4*)(codes + (int64_t)(c0 + c) * ldq + rb);
    q[0] = u32x4{out[0], out[1], out[2], out[3]};
    q[1] = u32x4{out[4], out[5], out[6], out[7]};
  }
  // (the column form's rows are the C columns, blocks along ldq)
  scales[mx_scale_at(c0 + c, rb / 32, C, (int)(ldq / 32), grouped)] = (uint8_t)sb;
}

hipError_t launch_mx_quant_both(const void* src, int batch, int R, int C, uint8_t* codes_r, uint8_t* scales_r,
                                uint8_t* codes_c, uint8_t* scales_c, bool fp4, bool grouped, hipStream_t st) {
  if (batch == 0 || R == 0 || C == 0) return hipSuccess;
  if (R % 32 || C % 32 || (grouped && (R % 128 || C % 128))) return hipErrorInvalidValue;
  const dim3 grid((R + kQcRows - 1) / kQcRows, (C + kQcCols - 1) / kQcCols, batch);
  const int64_t z = (int64_t)R * C;
  if (fp4)
    mx_quant_cols_kernel<true, true><<<grid, 256, 0, st>>>((const uint16_t*)src, C, R, C, R, R, codes_c, scales_c, z, z,
                                                           grouped, codes_r, scales_r);
  else
    mx_quant_cols_kernel<false, true><<<grid, 256, 0, st>>>((const uint16_t*)src, C, R, C, R, R, codes_c, scales_c, z,
                                                            z, grouped, codes_r, scales_r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantise-dequantise along rows: dst [rows][ld] bf16 holds the microscaled
// value (code x 2^e) of each src value, the blocks being 32 consecutive rows of
// one column; group g's blocks start at its first row off[g] (NULL: one group
// of `rows` rows), a group's last block holding the rows that remain (the
// missing ones count as zeros, which leaves the block's amax unchanged).  An
// e4m3 or e2m1 value times 2^e has at most four significant bits, so it is a
// bf16 value (except where 2^e is clamped at 2^-127 and the block's values lie
// below 2^-118, among bf16's subnormals): a product over two such operands in
// bf16 MFMAs with fp32 accumulation is the microscaled product.  bpre [G+1] =
// cumulative 32-row block counts of the groups (tile prefix of 32-row tiles).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t E = (c >> 1) & 3, m = c & 1;          // 0, .5 | 1, 1.5 | 2, 3 | 4, 6
  const float a = E == 0 ? 0.5f * (float)m : ldexpf((float)(2 + m), (int)E - 2);
  return (c & 8u) ? -a : a;
}

template <bool FP4>
__device__ __forceinline__ void qdq_block(float v[32]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = FP4 ? mx4_exponent(amax) : mx_exponent(amax);
  if constexpr (FP4) {
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const uint32_t b = e2m1_pk<0>(0u, ldexpf(v[i], -e), ldexpf(v[i + 1], -e));
      v[i] = ldexpf(e2m1_value(b & 15u), e);
      v[i + 1] = ldexpf(e2m1_value((b >> 4) & 15u), e);
    }
  } else {
    // to the e4m3fn grid and back with the hardware conversions (nearest
    // code, ties to even)
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[i], -e), ldexpf(v[i + 1], -e), 0, false);
      v[i] = ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 0), e);
      v[i + 1] = ldexpf(__builtin_amdgcn_cvt_f32_fp8(w, 1), e);
    }
  }
}

// A workgroup takes one 32-row block by 256 columns: 16-byte row loads into
// LDS, thread c quantises column c's 32 values there, 16-byte row stores.
template <bool FP4>
__global__ __launch_bounds__(256) void mx_qdq_rows_kernel(const uint16_t* __restrict__ src, int64_t ld, int rows,
                                                          int C, const int* __restrict__ off,
                                                          const int* __restrict__ bpre, int G,
                                                          uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ uint16_t tile[32][256];
  const int blk = blockIdx.x;
  int r0, n;
  if (off) {
    if (blk >= bpre[G]) return;
    int lo = 0, hi = G;                                 // group g with bpre[g] <= blk < bpre[g+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (bpre[mid] <= blk) lo = mid; else hi = mid;
    }
    r0 = off[lo] + 32 * (blk - bpre[lo]);
    n = off[lo + 1] - r0;
  } else {
    r0 = 32 * blk;
    n = rows - r0;
  }
  if (n <= 0) return;
  if (n > 32) n = 32;
  const int c0 = blockIdx.y * 256;
  // 32 rows x 32 chunks of 8 columns; rows past n and columns past C read as 0
  for (int q = threadIdx.x; q < 32 * 32; q += 256) {
    const int r = q >> 5, ch = q & 31, c = c0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < n && c + 8 <= C) v = *(const u32x4*)(src + (int64_t)(r0 + r) * ld + c);
    *(u32x4*)&tile[r][ch * 8] = v;
  }
  __syncthreads();
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = bf16_bits_lo(tile[r][threadIdx.x]);
  qdq_block<FP4>(v);
#pragma unroll
  for (int r = 0; r < 32; ++r) tile[r][threadIdx.x] = (uint16_t)(pack_bf16x2(v[r], 0.0f) & 0xFFFFu);
  __syncthreads();
  for (int q = threadIdx.x; q < 32 * 32; q += 256) {
    const int r = q >> 5, ch = q & 31, c = c0 + ch * 8;
    if (r < n && c + 8 <= C) *(u32x4*)(dst + (int64_t)(r0 + r) * ldd + c) = *(const u32x4*)&tile[r][ch * 8];
  }
}

hipError_t launch_mx_qdq_rows(const void* src, int64_t ld, int rows, int C, const int* off, const int* bpre, int G,
                              void* dst, int64_t ldd, bool fp4, hipStream_t st) {
  if (rows <= 0 || C <= 0) return hipSuccess;
  if (C % 8 != 0 || ld % 8 != 0 || ldd % 8 != 0 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return hipErrorInvalidValue;
  const int64_t blocks = (rows + 31) / 32 + (off ? G : 0);   // upper bound of the groups' 32-row blocks
  const dim3 grid((unsigned)blocks, (unsigned)((C + 255) / 256));
  if (fp4)
    mx_qdq_rows_kernel<true><<<grid, 256, 0, st>>>((const uint16_t*)src, ld, rows, C, off, bpre, G,
                                                   (uint16_t*)dst, ldd);
  else
    mx_qdq_rows_kernel<false><<<grid, 256, 0, st>>>((const uint16_t*)src, ld, rows, C, off, bpre, G,
                                                    (uint16_t*)dst, ldd);
  return hipGetLastError();
}

// batched transposed form for weights: src [batch][R][C] -> codes [batch][C][R],
// one launch with the batch in the grid's z dimension (one launch per matrix
// took 8.9 ms for 256 matrices of 4096 x 7168, dominated by launch and drain)
hipError_t launch_mx_quant_cols_batched(const void* src, int batch, int R, int C, uint8_t* codes,
                                        uint8_t* scales, bool fp4, bool grouped, hipStream_t st) {
  if (batch == 0 || R == 0 || C == 0) return hipSuccess;
  if (grouped && R % 128) return hipErrorInvalidValue;
  const int tiles = (R + kQcRows - 1) / kQcRows;
  const dim3 grid(tiles, (C + kQcCols - 1) / kQcCols, batch);
  if (fp4)
    mx_quant_cols_kernel<true><<<grid, 256, 0, st>>>((const uint16_t*)src, C, R, C, R, R,
                                                     codes, scales, (int64_t)R * C, (int64_t)R * C, grouped);
  else
    mx_quant_cols_kernel<false><<<grid, 256, 0, st>>>((const uint16_t*)src, C, R, C, R, R,
                                                      codes, scales, (int64_t)R * C, (int64_t)R * C, grouped);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP8 / MXFP4 GEMM launchers.  Callers give K, leading dimensions and group
// strides in values; the kernels count them in 2-byte units of the code
// bytes (two fp8 values or four fp4 values per unit).
// ---------------------------------------------------------------------------
template <bool FP4>
static void to_units(GemmArgs& a) {
  constexpr int per = FP4 ? 4 : 2;        // values per 2-byte unit
  a.lda /= per; a.ldb /= per; a.K /= per; a.b_kend /= per; a.b_gstride /= per;
}

// DMA-fed LDS ring (gemm_mfma_kernel in its microscaled form): 128x256 tiles,
// 2x4 compute waves and two load waves, three stages; one tile per workgroup.
// The load waves took the skewed DeepSeek-V3 MXFP8 step from 15.6 to 15.0 ms
// (gate/up data gradient 1.93 -> 1.72 ms, down forward 1.13 -> 0.97 ms).  The
// MXFP4 SwiGLU forward keeps every wave loading: with its fused quantisation
// the epilogue needs more than the registers three waves per SIMD leave (it
// spilled and ran 8.4 ms instead of 1.12).
template <GemmMode MODE, class Epi, bool FP4>
static hipError_t launch_mx_dma(GemmArgs a, const MxArgs& s, const typename Epi::P& ep, int n_logical,
                                int rows_total, hipStream_t st) {
  constexpr int BM = 128, BN = 256, WM = 2, WN = 4, STAGES = 3, NLW = (FP4 && Epi::kPaired) ? 0 : 2;
  using C = TileCfg<BM, BN, WM, WN, STAGES, true, NLW, FP4>;
  const int bn_cols = Epi::kPaired ? BN / 2 : BN;
  const int NT = (n_logical + bn_cols - 1) / bn_cols;
  const int MT = (MODE == RAGGED_M) ? 0 : (a.M + BM - 1) / BM;
  int64_t tiles;
  if (MODE == RAGGED_M) tiles = (int64_t)((rows_total + BM - 1) / BM + a.G) * NT;
  else tiles = (int64_t)MT * NT;
  if (tiles <= 0) return hipSuccess;
  to_units<FP4>(a);
  auto kern = gemm_mfma_kernel<BM, BN, WM, WN, STAGES, KC, KC, MODE, Epi, true, FP4, NLW>;
  static bool lds_done[kLdsAttrDevices] = {};   // per device, per instantiation
  if (hipError_t e = raise_lds_limit(lds_done, (const void*)kern, C::LDS_BYTES); e != hipSuccess) return e;
  kern<<<(unsigned)tiles, C::NTHR, C::LDS_BYTES, st>>>(a, s, ep, NT, MT);
  return hipGetLastError();
}

// Z[rows, N] = Q[rows, K] . W[g][N, K]^T over ragged row groups (or dense when
// offsets is NULL): the operands are quantised row forms.
template <class Epi>
static hipError_t mx_rows_gemm(const MxQ& q, const int* offsets, const int* prefix, int G, const MxQ& w,
                               int64_t w_gstride, int rows, int N, int K, const typename Epi::P& ep,
                               int n_logical, bool fp4, hipStream_t st) {
  GemmArgs a{};
  a.A = q.codes; a.lda = K; a.B = w.codes; a.ldb = K; a.b_gstride = w_gstride;
  a.M = rows; a.N = N; a.K = K; a.b_next = N; a.b_kend = K;
  // grouped scales: A's over its `rows` rows, each group's B over its N rows
  MxArgs s{q.scales, w.scales, rows, N, w_gstride / 32};
  // staged epilogues store 16-byte row pieces (the call's shape checks and
  // 16-byte aligned outputs guarantee them)
  if constexpr (Epi::kStaged)
    if (!(ep.N % 8 == 0 && ep.ldc % 8 == 0 && ep.c_gstride % 8 == 0 && ((uintptr_t)ep.C & 15) == 0))
      return hipErrorInvalidValue;
  if (offsets) {
    a.offsets = offsets; a.tile_prefix = prefix; a.G = G;
    return fp4 ? launch_mx_dma<RAGGED_M, Epi, true>(a, s, ep, n_logical, rows, st)
               : launch_mx_dma<RAGGED_M, Epi, false>(a, s, ep, n_logical, rows, st);
  }
  a.G = 1;
  return fp4 ? launch_mx_dma<DENSE, Epi, true>(a, s, ep, n_logical, rows, st)
             : launch_mx_dma<DENSE, Epi, false>(a, s, ep, n_logical, rows, st);
}

hipError_t gemm_mx_swiglu_fwd(const MxQ& x, const int* off, const int* prefix, int G, const MxQ& w13, void* hu,
                              void* act, int rows, int d, int f, const float* row_gates, bool from_stored, bool fp4,
                              uint8_t* act_codes, uint8_t* act_scales, hipStream_t st) {
  typename EpiSwiGLU<bf16>::P ep{(bf16*)act, (bf16*)hu, f, row_gates, from_stored ? 1 : 0,
                                 act_codes, act_scales, fp4 ? 1 : 0, rows};
  return mx_rows_gemm<EpiSwiGLU<bf16>>(x, off, prefix, G, w13, (int64_t)2 * f * d, rows, 2 * f, d, ep, f, fp4, st);
}

hipError_t gemm_mx_down_fwd(const MxQ& act, const int* off, const int* prefix, int G, const MxQ& w2, void* y,
                            int rows, int d, int f, bool fp4, hipStream_t st) {
  typename EpiStore<bf16, 5>::P ep{(bf16*)y, d, 0, rows, d};
  return mx_rows_gemm<EpiStore<bf16, 5>>(act, off, prefix, G, w2, (int64_t)d * f, rows, d, f, ep, d, fp4, st);
}

// dA = dY W2 with W2 quantised along d (w2t [g][f][d]); SwiGLU backward epilogue
hipError_t gemm_mx_down_dgrad_swiglu_bwd(const MxQ& dy, const int* off, const int* prefix, int G,
                                         const MxQ& w2t, const void* hu, void* dhu, int rows, int d, int f,
                                         const float* row_gates, float* dg_part, void* act_out, bool fp4,
                                         uint8_t* dhu_codes, uint8_t* dhu_scales, hipStream_t st) {
  typename EpiSwiGLUBwd<bf16>::P ep{(const bf16*)hu, (bf16*)dhu, f, row_gates, row_gates ? dg_part : nullptr,
                                    gemm_dg_parts(true, f), (bf16*)act_out, dhu_codes, dhu_scales, fp4 ? 1 : 0,
                                    rows};
  return mx_rows_gemm<EpiSwiGLUBwd<bf16>>(dy, off, prefix, G, w2t, (int64_t)f * d, rows, f, d, ep, f, fp4, st);
}

// dX = dHU W13 with W13 quantised along 2f (w13t [g][d][2f]); bf16 or fp32 out
hipError_t gemm_mx_gateup_dgrad(const MxQ& dhu, const int* off, const int* prefix, int G, const MxQ& w13t,
                                void* dx, bool f32_out, int rows, int d, int f, bool fp4, hipStream_t st) {
  if (f32_out) {
    EpiStoreF32T<1>::P ep{(float*)dx, d, 0, rows, d};
    return mx_rows_gemm<EpiStoreF32T<1>>(dhu, off, prefix, G, w13t, (int64_t)d * 2 * f, rows, d, 2 * f, ep, d, fp4,
                                         st);
  }
  typename EpiStore<bf16, 6>::P ep{(bf16*)dx, d, 0, rows, d};
  return mx_rows_gemm<EpiStore<bf16, 6>>(dhu, off, prefix, G, w13t, (int64_t)d * 2 * f, rows, d, 2 * f, ep, d, fp4,
                                         st);
}

}  // namespace moe
