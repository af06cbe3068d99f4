// Internal launchers of libmoe_gfx950 (host side).  Every launcher only
// enqueues work on `st` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// A kernel's dynamic-LDS limit (hipFuncAttributeMaxDynamicSharedMemorySize)
// is set per device: `done`, one array per kernel instantiation, records the
// devices on which it has been raised to `bytes`.
constexpr int kLdsAttrDevices = 64;
inline hipError_t raise_lds_limit(bool (&done)[kLdsAttrDevices], const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kLdsAttrDevices) return hipErrorInvalidDevice;
  if (done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done[dev] = true;
  return e;
}

struct RouterParams {
  int T, E, k;
  int score;        // 0 softmax, 1 sigmoid
  int n_group, topk_group;
  int renorm;
  float scale;
  float aux_coeff;
  int balanced;     // force-balanced routing: choice j of token t is expert (t k + j) mod E
};

constexpr int kRouterTokensPerBlock = 16;
constexpr int kPermTokensPerRange = 64;

// router.hip
hipError_t launch_router_topk(const float* logits, const float* bias, const RouterParams& p,
                              int32_t* idx, float* gates, int* cnt_part, float* colsum_part,
                              hipStream_t st);
hipError_t launch_router_finalize(const int* cnt_part, float* colsum_part, int nblk, const RouterParams& p,
                                  int32_t* counts, hipStream_t st);
hipError_t launch_router_aux(const int32_t* counts, const float* colsum, const RouterParams& p, float* aux,
                             hipStream_t st);
hipError_t launch_router_bias_update(const int32_t* counts, int E, int64_t Tk, float rate, float* bias,
                                     hipStream_t st);
template <class T>
hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gates,
                             const float* d_gates, const int32_t* counts, const RouterParams& p,
                             float d_aux, float* d_logits, T* dl_store, int Ep, hipStream_t st);

// permute.hip
hipError_t launch_perm_hist(const int32_t* idx, int T, int k, int E, int* hist, hipStream_t st);
hipError_t launch_perm_scan(int* hist, int R, int E, int rows, int32_t* offsets, hipStream_t st);
// gates / row_gates (optional pair): row_gates[row_id_map[n]] = gates[n]
hipError_t launch_perm_rank(const int32_t* idx, int T, int k, int E, int* base, int32_t* row_id_map,
                            int32_t* src_token, const float* gates, float* row_gates, hipStream_t st);
hipError_t launch_scatter_rows(const void* x, const int32_t* row_id_map, int T_, int k, int row_bytes,
                               void* out, hipStream_t st);
template <class T>
hipError_t launch_combine(const T* y_perm, const int32_t* rmap, const float* gates, const T* y_shared,
                          T* y, int T_, int k, int d, hipStream_t st);
template <class T>
hipError_t launch_combine_bwd(const T* dy, const T* y_perm, const int32_t* rmap, const float* gates,
                              T* dy_perm, float* d_gates, int T_, int k, int d, hipStream_t st);
template <class T>
hipError_t launch_unpermute_sum(const T* dx_perm, const int32_t* rmap, const float* partial, T* dx,
                                int T_, int k, int d, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);

// gemm.hip
hipError_t launch_tile_prefix(const int* offsets, int G, int BM, int* prefix, hipStream_t st);
// rows of the ragged tiles of the forward and gate/up data-gradient products
// (swiglu_bwd = false) or of the SwiGLU-backward product; the device tile
// prefix must be built with it
int gemm_tile_rows(bool bf16, int64_t rows, int G, bool swiglu_bwd);
// Split-K parts of the router logits GEMM (1: none) and the K range of each
// (*kchunk, a multiple of 64); the parts need [parts][T][E] fp32 of workspace.
int router_logit_parts(bool bf16, int64_t T, int E, int d, int* kchunk);
// logits = x w_r^T; with parts > 1 (router_logit_parts) the parts go to `part`
// and are summed in part order into logits
template <class T>
hipError_t gemm_router_logits(const void* x, const void* w_r, float* logits, int T_, int E, int d, float* part,
                              hipStream_t st);
// row_gates: folded gates (act = g silu(H) U) or NULL; from_stored: act from H, U as stored
template <class T>
hipError_t gemm_swiglu_fwd(const void* xin, const int* offsets, const int* tile_prefix, int G,
                           const void* w13, void* hu, void* act, int rows, int d, int f,
                           const float* row_gates, bool from_stored, hipStream_t st);
template <class T>
hipError_t gemm_down_fwd(const void* act, const int* offsets, const int* tile_prefix, int G,
                         const void* w2, void* y, int rows, int d, int f, hipStream_t st);
// row_gates (folded gates) with dg_part [rows, gemm_dg_parts] gate-gradient
// partials, or NULL; act_out: act formed again from hu (recomputation) or NULL
template <class T>
hipError_t gemm_down_dgrad_swiglu_bwd(const void* dy, const int* offsets, const int* tile_prefix,
                                      int G, const void* w2, const void* hu, void* dhu, int rows,
                                      int d, int f, const float* row_gates, float* dg_part, void* act_out,
                                      hipStream_t st);
int gemm_dg_parts(bool bf16, int f);
hipError_t launch_gate_grad_sum(const float* part, int P, const int32_t* row_id_map, int64_t n_total,
                                float* d_gates, hipStream_t st);
template <class T>
hipError_t gemm_gateup_dgrad(const void* dhu, const int* offsets, const int* tile_prefix, int G,
                             const void* w13, void* dx, bool f32_out, int rows, int d, int f,
                             hipStream_t st);
template <class T>
hipError_t gemm_wgrad(const void* P_, int M, const void* Q_, int N, const int* offsets, int G,
                      int K_dense, void* dw, int site, hipStream_t st);
// Split-K parts of the router weight gradient (contraction over the T tokens)
// and the rows of each (*kchunk); [parts][E][d] fp32 of workspace.
int router_wgrad_parts(bool bf16, int64_t T, int E, int d, int* kchunk);
template <class T>
hipError_t gemm_router_wgrad(const void* dl, int Ep, int E, const void* x, int T_, int d, void* dw_r, float* part,
                             hipStream_t st);
template <class T>
hipError_t gemm_router_dgrad(const void* dl, int Ep, int E, const void* w_r, int T_, int d,
                             float* dx_partial, hipStream_t st);

// mxfp8.hip (MXFP8 and MXFP4: `fp4` selects e2m1 codes, two per byte)
struct MxQ {                            // codes and e8m0 scales of one quantised tensor
  const uint8_t* codes;
  const uint8_t* scales;
};
// grouped: scales in the grouped layout (mx_scale_at; the blocked dimension
// a multiple of 128), else plain
hipError_t launch_mx_quant_rows(const void* src, int64_t ld, int64_t src_bstride, int batch, int R, int C,
                                uint8_t* codes, uint8_t* scales, bool fp4, bool grouped, hipStream_t st);
hipError_t launch_mx_quant_cols_batched(const void* src, int batch, int R, int C, uint8_t* codes,
                                        uint8_t* scales, bool fp4, bool grouped, hipStream_t st);
// both forms of [batch][R][C] in one pass (R and C multiples of 32)
hipError_t launch_mx_quant_both(const void* src, int batch, int R, int C, uint8_t* codes_r, uint8_t* scales_r,
                                uint8_t* codes_c, uint8_t* scales_c, bool fp4, bool grouped, hipStream_t st);
// dst [rows][ldd] bf16 = the microscaled values of src [rows][ld] with 32-row
// blocks per column, restarting at each group's first row (bpre: cumulative
// 32-row block counts, launch_tile_prefix with 32; off NULL: one group)
hipError_t launch_mx_qdq_rows(const void* src, int64_t ld, int rows, int C, const int* off, const int* bpre, int G,
                              void* dst, int64_t ldd, bool fp4, hipStream_t st);
// act_codes / act_scales: the row form of act (blocks of 32 along f) written by
// the epilogue from the stored act, or NULL
hipError_t gemm_mx_swiglu_fwd(const MxQ& x, const int* off, const int* prefix, int G, const MxQ& w13, void* hu,
                              void* act, int rows, int d, int f, const float* row_gates, bool from_stored, bool fp4,
                              uint8_t* act_codes, uint8_t* act_scales, hipStream_t st);
hipError_t gemm_mx_down_fwd(const MxQ& act, const int* off, const int* prefix, int G, const MxQ& w2, void* y,
                            int rows, int d, int f, bool fp4, hipStream_t st);
// dhu_codes / dhu_scales: the row form of dHU (blocks of 32 along 2f), or NULL
hipError_t gemm_mx_down_dgrad_swiglu_bwd(const MxQ& dy, const int* off, const int* prefix, int G,
                                         const MxQ& w2t, const void* hu, void* dhu, int rows, int d, int f,
                                         const float* row_gates, float* dg_part, void* act_out, bool fp4,
                                         uint8_t* dhu_codes, uint8_t* dhu_scales, hipStream_t st);
hipError_t gemm_mx_gateup_dgrad(const MxQ& dhu, const int* off, const int* prefix, int G, const MxQ& w13t,
                                void* dx, bool f32_out, int rows, int d, int f, bool fp4, hipStream_t st);

}  // namespace moe
