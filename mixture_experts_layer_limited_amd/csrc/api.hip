// C ABI of libmoe_gfx950: host-side validation and orchestration of the
// kernels.  Nothing here allocates device memory or synchronises; every call
// checks its arguments before the first launch and reports failures through
// moe_status and moe_last_error().
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status ok() {
  g_err.clear();
  return MOE_OK;
}

// ---- device check (cached per device) --------------------------------------
constexpr int kMaxDevices = 64;
struct DevInfo {
  bool checked = false;
  bool gfx950 = false;
  int cus = 0;
};
DevInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

moe_status check_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_INVALID_ARGUMENT, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& di = g_dev[dev];
  if (!di.checked) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    di.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    di.cus = prop.multiProcessorCount;
    di.checked = true;
    if (!di.gfx950) {
      return fail(MOE_ERR_UNSUPPORTED, "device %d is %s, this library is built for gfx950", dev,
                  prop.gcnArchName);
    }
  }
  if (!di.gfx950) return fail(MOE_ERR_UNSUPPORTED, "device %d is not a gfx950 GPU", dev);
  return MOE_OK;
}

moe_status check_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  return check_device(dev);
}

// ---- argument validation ---------------------------------------------------
moe_status check_cfg(const moe_cfg* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg is NULL");
  if (c->flags & ~(MOE_FLAG_FORCE_BALANCED | MOE_FLAG_FOLD_GATES | MOE_FLAG_RECOMPUTE_ACT))
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.flags = 0x%x has unknown bits", (unsigned)c->flags);
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16 && c->dtype != MOE_MXFP8 && c->dtype != MOE_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "cfg.dtype %d not supported", c->dtype);
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.T = %lld < 0", (long long)c->T);
  if (c->E < 1 || c->E > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.E = %lld outside [1, %d]", (long long)c->E, kMaxExperts);
  if (c->k < 1 || c->k > c->E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.k = %lld outside [1, E=%lld]", (long long)c->k,
                (long long)c->E);
  if (c->d < 8 || c->d % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.d = %lld must be a positive multiple of 8", (long long)c->d);
  if (c->f < 8 || c->f % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.f = %lld must be a positive multiple of 8", (long long)c->f);
  if (c->f_shared < 0 || c->f_shared % 8)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.f_shared = %lld must be 0 or a multiple of 8", (long long)c->f_shared);
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.score = %d unknown", c->score);
  if (c->n_group < 1 || c->E % c->n_group)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.n_group = %d must divide E = %lld", c->n_group, (long long)c->E);
  if (c->topk_group < 1 || c->topk_group > c->n_group)
    return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.topk_group = %d outside [1, n_group=%d]", c->topk_group, c->n_group);
  if ((int64_t)c->topk_group * (c->E / c->n_group) < c->k)
    return fail(MOE_ERR_INVALID_ARGUMENT, "topk_group * E / n_group = %lld < k = %lld",
                (long long)c->topk_group * (c->E / c->n_group), (long long)c->k);
  if (c->renorm != 0 && c->renorm != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.renorm must be 0 or 1");
  if (c->aux_coeff != 0.0f && c->score != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_UNSUPPORTED, "the aux loss is defined for the softmax score only");
  const int64_t lim = (int64_t)1 << 31;
  if (c->T * c->k >= lim || c->d >= lim / 8 || c->f >= lim / 8 || c->f_shared >= lim / 8)
    return fail(MOE_ERR_INVALID_ARGUMENT, "shape too large (T*k, d, f must stay below 2^31 / 8)");
  return MOE_OK;
}

// The MFMA kernels address an operand through a buffer resource with a 32-bit
// byte range and 32-bit per-lane offsets: one expert's (or the dense
// products') rows of any operand or output, and one expert's weight matrix,
// must span fewer than 2^31 bytes.  Expert sizes are only known on the
// device, so the bound is taken with all T*k rows in one expert.
moe_status check_offsets_32bit(const moe_cfg* c, int64_t elt_bytes) {
  const int64_t lim = (int64_t)1 << 31;
  int64_t width = c->d;                              // widest row of any operand or output
  if (2 * c->f > width) width = 2 * c->f;
  if (2 * c->f_shared > width) width = 2 * c->f_shared;
  if (c->E > width) width = c->E;
  const int64_t rows = c->T * c->k > c->T ? c->T * c->k : c->T;
  const int64_t wmax = 2 * (c->f > c->f_shared ? c->f : c->f_shared) * c->d;
  if (rows * width * elt_bytes >= lim || wmax * elt_bytes >= lim)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "shape too large for 32-bit buffer offsets: T*k rows x %lld columns and one expert's "
                "2f x d weight must each stay below 2^31 bytes", (long long)width);
  return MOE_OK;
}

// the bf16 GEMM path streams K-contiguous operands in 64-wide slices
moe_status check_gemm_shapes(const moe_cfg* c) {
  if (c->dtype != MOE_F32 && (c->d % 64 || c->f % 64 || c->f_shared % 64))
    return fail(MOE_ERR_INVALID_ARGUMENT, "bf16 GEMMs need d, f and f_shared to be multiples of 64");
  if (c->dtype != MOE_F32) return check_offsets_32bit(c, 2);
  return MOE_OK;
}

inline bool is_mx(const moe_cfg* c) { return c->dtype == MOE_MXFP8 || c->dtype == MOE_MXFP4; }
inline bool is_fp4(const moe_cfg* c) { return c->dtype == MOE_MXFP4; }

// expert GEMM calls of the bf16 / fp32 path
moe_status check_not_mx(const moe_cfg* c) {
  if (is_mx(c))
    return fail(MOE_ERR_UNSUPPORTED, "cfg.dtype is MXFP8 / MXFP4: use the *_mxfp8 / *_mxfp4 expert GEMM calls");
  return MOE_OK;
}

// the microscaled GEMMs contract in slices of 128 code bytes per row: 128 fp8
// or 256 fp4 values
moe_status check_mx_shapes(const moe_cfg* c, int32_t want) {
  const char* name = want == MOE_MXFP4 ? "MXFP4" : "MXFP8";
  if (c->dtype != want) return fail(MOE_ERR_INVALID_ARGUMENT, "cfg.dtype must be MOE_%s for this call", name);
  const int64_t m = want == MOE_MXFP4 ? 256 : 128;
  if (c->d % m || c->f % m || c->f_shared % m)
    return fail(MOE_ERR_INVALID_ARGUMENT, "%s GEMMs need d, f and f_shared to be multiples of %lld", name, (long long)m);
  return check_offsets_32bit(c, 2);               // bf16 operands and outputs beside the codes
}

#define REQ(p)                                                                          \
  do {                                                                                  \
    if (!(p)) return fail(MOE_ERR_INVALID_ARGUMENT, "argument '%s' must not be NULL", #p); \
  } while (0)
#define ALIGNED(p)                                                                            \
  do {                                                                                        \
    if ((p) && ((uintptr_t)(p) & 15))                                                         \
      return fail(MOE_ERR_INVALID_ARGUMENT, "argument '%s' must be 16-byte aligned", #p);      \
  } while (0)
#define CHECK(call)                                                                     \
  do {                                                                                  \
    moe_status s_ = (call);                                                             \
    if (s_ != MOE_OK) return s_;                                                        \
  } while (0)
// ---- kernel timing trace -----------------------------------------------------
struct Trace {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;          // 2 per kernel: before, after
  std::vector<const char*> names;
};
thread_local Trace g_trace;

inline void trace_pre(hipStream_t st) {
  if (g_trace.on && g_trace.n < g_trace.cap) hipEventRecord(g_trace.ev[2 * g_trace.n], st);
}
inline void trace_post(const char* name, hipStream_t st) {
  if (g_trace.on && g_trace.n < g_trace.cap) {
    hipEventRecord(g_trace.ev[2 * g_trace.n + 1], st);
    g_trace.names[g_trace.n++] = name;
  }
}

// every launcher enqueues exactly one kernel (or none for empty work)
#define LAUNCH_NAMED(name, call)                                                                      \
  do {                                                                                                \
    trace_pre(st);                                                                                    \
    hipError_t e_ = (call);                                                                           \
    trace_post(name, st);                                                                             \
    if (e_ != hipSuccess) return fail(MOE_ERR_DEVICE, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)
#define LAUNCH(call) LAUNCH_NAMED(#call, call)

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t ranges(int64_t T) { return (T + kPermTokensPerRange - 1) / kPermTokensPerRange; }
inline int64_t router_blocks(int64_t T) { return (T + kRouterTokensPerBlock - 1) / kRouterTokensPerBlock; }
inline int64_t pad64(int64_t e) { return (e + 63) & ~int64_t(63); }
inline size_t elt(const moe_cfg* c) { return c->dtype == MOE_F32 ? 4 : 2; }
inline bool fold(const moe_cfg* c) { return (c->flags & MOE_FLAG_FOLD_GATES) != 0; }
inline bool recompute(const moe_cfg* c) { return (c->flags & MOE_FLAG_RECOMPUTE_ACT) != 0; }

// Workspace regions of the grouped-GEMM calls beyond their own first region
// (the tile prefix, or the MXFP8 buffers): act formed again from hu_save
// (recomputation; the routed experts' rows and later the shared expert's, so
// one region of the larger size) and the folded gates' gradient partials.
struct GemmExtra {
  size_t act, dg, bytes;       // offsets from the region start, total size
};
GemmExtra gemm_extra(const moe_cfg* c, size_t at, bool bf16_gemms) {
  GemmExtra w;
  const int64_t rows = c->T * c->k;
  size_t o = at;
  w.act = o;
  if (recompute(c)) {
    const int64_t n = rows * c->f > c->T * c->f_shared ? rows * c->f : c->T * c->f_shared;
    o += align256((size_t)n * elt(c));
  }
  w.dg = o;
  if (fold(c)) o += align256((size_t)rows * gemm_dg_parts(bf16_gemms, (int)c->f) * 4);
  w.bytes = o - at;
  return w;
}

// MXFP8 workspace: two int arrays (tile prefix, padded offsets), one row-form
// quantised activation (codes + scales) and two column-form ones
struct MxWs {
  int64_t rows_max, cmax_rows, cmax_cols;
  size_t ints, qa, qt;            // region sizes (qa: one activation's row form; qt: one
                                  // weight-gradient operand, bf16)
  GemmExtra extra;                // recomputed act, gate-gradient partials (after the others)
  size_t total() const { return ints + 2 * qa + 2 * qt + extra.bytes; }
};
MxWs mx_ws(const moe_cfg* c) {
  MxWs w;
  const int64_t rows = c->T * c->k;
  w.rows_max = rows > c->T ? rows : c->T;
  int64_t cm = c->d;
  if (2 * c->f > cm) cm = 2 * c->f;
  if (2 * c->f_shared > cm) cm = 2 * c->f_shared;
  w.cmax_rows = cm;
  w.cmax_cols = cm;
  // (row-form codes sized for fp8: an fp4 form takes half the region)
  w.ints = 2 * align256((size_t)(c->E + 2) * 4);
  w.qa = align256((size_t)(w.rows_max * w.cmax_rows)) + align256((size_t)(w.rows_max * w.cmax_rows / 32));
  w.qt = align256((size_t)(w.rows_max * w.cmax_cols * 2));
  w.extra = gemm_extra(c, w.ints + 2 * w.qa + 2 * w.qt, true);
  return w;
}

// router workspace: per-block counts and column sums, then the split-K parts
// of the logits GEMM
size_t router_parts_bytes(const moe_cfg* c) {
  int kchunk;
  const int parts = router_logit_parts(c->dtype != MOE_F32, c->T, (int)c->E, (int)c->d, &kchunk);
  return parts > 1 ? align256((size_t)parts * c->T * c->E * 4) : 0;
}

size_t ws_bytes_for(const moe_cfg* c) {
  size_t router = 2 * align256((size_t)router_blocks(c->T) * c->E * 4) + router_parts_bytes(c);
  size_t perm = align256((size_t)ranges(c->T) * c->E * 4);
  const size_t prefix = align256((size_t)(c->E + 2) * 4);
  size_t gemm = prefix + gemm_extra(c, prefix, c->dtype != MOE_F32).bytes;
  int wchunk;
  const int wparts = router_wgrad_parts(c->dtype != MOE_F32, c->T, (int)c->E, (int)c->d, &wchunk);
  size_t rbwd = align256((size_t)c->T * pad64(c->E) * elt(c)) +
                (wparts > 1 ? align256((size_t)wparts * c->E * c->d * 4) : 0);
  size_t m = router;
  if (perm > m) m = perm;
  if (gemm > m) m = gemm;
  if (rbwd > m) m = rbwd;
  if (is_mx(c) && mx_ws(c).total() > m) m = mx_ws(c).total();
  return m < 256 ? 256 : m;
}

moe_status check_ws(const moe_cfg* c, void* ws, size_t bytes) {
  size_t need = ws_bytes_for(c);
  if (!ws) return fail(MOE_ERR_INVALID_ARGUMENT, "argument 'workspace' must not be NULL");
  ALIGNED(ws);
  if (bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", bytes, need);
  return MOE_OK;
}

RouterParams router_params(const moe_cfg* c) {
  RouterParams p;
  p.T = (int)c->T; p.E = (int)c->E; p.k = (int)c->k; p.score = c->score;
  p.n_group = c->n_group; p.topk_group = c->topk_group; p.renorm = c->renorm;
  p.scale = c->scale; p.aux_coeff = c->aux_coeff;
  p.balanced = (c->flags & MOE_FLAG_FORCE_BALANCED) ? 1 : 0;
  return p;
}

template <class T>
moe_status router_topk_impl(const moe_cfg* c, const void* x, const void* w_router, const float* bias,
                            float* logits, int32_t* idx, float* gates, int32_t* counts, float* aux,
                            void* ws, hipStream_t st) {
  RouterParams p = router_params(c);
  const int nblk = (int)router_blocks(c->T);
  char* w = (char*)ws;
  int* cnt_part = (int*)w;
  float* colsum_part = (float*)(w + align256((size_t)nblk * c->E * 4));
  float* logit_parts = (float*)(w + 2 * align256((size_t)nblk * c->E * 4));
  if (x) LAUNCH_NAMED("gemm_router_logits", gemm_router_logits<T>(x, w_router, logits, (int)c->T, (int)c->E, (int)c->d,
                                                                  logit_parts, st));
  const bool want_colsum = c->aux_coeff != 0.0f;
  LAUNCH_NAMED("router_topk", launch_router_topk(logits, bias, p, idx, gates, cnt_part, want_colsum ? colsum_part : nullptr, st));
  LAUNCH_NAMED("router_finalize", launch_router_finalize(cnt_part, want_colsum ? colsum_part : nullptr, nblk, p, counts, st));
  if (want_colsum && aux) LAUNCH_NAMED("router_aux", launch_router_aux(counts, colsum_part, p, aux, st));
  return ok();
}

template <class T>
moe_status gemm_fwd_impl(const moe_cfg* c, const void* x_perm, const int32_t* off, const float* row_gates,
                         const void* w13, const void* w2, void* hu, void* act, void* y_perm, const void* x,
                         const void* ws13, const void* ws2, void* hu_s, void* act_s, void* y_s,
                         void* ws, hipStream_t st) {
  const bool bf = sizeof(T) == 2;
  const int E = (int)c->E, rows = (int)(c->T * c->k), d = (int)c->d, f = (int)c->f;
  const bool rc = recompute(c);
  int* prefix = (int*)ws;
  if (rows > 0) {
    LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, gemm_tile_rows(bf, rows, E, false), prefix, st));
    LAUNCH_NAMED("gemm_swiglu_fwd", gemm_swiglu_fwd<T>(x_perm, off, prefix, E, w13, hu, act, rows, d, f,
                                                       fold(c) ? row_gates : nullptr, rc, st));
    LAUNCH_NAMED("gemm_down_fwd", gemm_down_fwd<T>(act, off, prefix, E, w2, y_perm, rows, d, f, st));
  }
  if (c->f_shared > 0 && c->T > 0) {
    const int fs = (int)c->f_shared, T_ = (int)c->T;
    LAUNCH_NAMED("gemm_swiglu_fwd_shared", gemm_swiglu_fwd<T>(x, nullptr, nullptr, 1, ws13, hu_s, act_s, T_, d, fs,
                                                              nullptr, rc, st));
    LAUNCH_NAMED("gemm_down_fwd_shared", gemm_down_fwd<T>(act_s, nullptr, nullptr, 1, ws2, y_s, T_, d, fs, st));
  }
  return ok();
}

template <class T>
moe_status gemm_bwd_impl(const moe_cfg* c, const void* dy_perm, const void* x_perm, const int32_t* off,
                         const float* row_gates, const int32_t* row_id_map, const void* hu, const void* act,
                         const void* w13, const void* w2, void* dhu, void* dx_perm, void* dw13, void* dw2,
                         float* d_gates, const void* dy, const void* x, const void* hu_s, const void* act_s,
                         const void* ws13, const void* ws2, void* dhu_s, float* dx_partial, void* dws13,
                         void* dws2, void* ws, hipStream_t st) {
  const bool bf = sizeof(T) == 2;
  const int E = (int)c->E, rows = (int)(c->T * c->k), d = (int)c->d, f = (int)c->f, T_ = (int)c->T;
  int* prefix = (int*)ws;
  const size_t prefix_bytes = align256((size_t)(c->E + 2) * 4);
  const GemmExtra X = gemm_extra(c, prefix_bytes, bf);
  // recomputation: the down-projection dgrad forms act again into the workspace
  void* act_rec = recompute(c) ? (char*)ws + X.act : nullptr;
  float* dg_part = fold(c) ? (float*)((char*)ws + X.dg) : nullptr;
  const float* rg = fold(c) ? row_gates : nullptr;
  // the SwiGLU-backward product and the gate/up data gradient may take
  // different tile heights: the prefix is built again between them if so
  const int bm_swiglu_bwd = gemm_tile_rows(bf, rows, E, true), bm_dgrad = gemm_tile_rows(bf, rows, E, false);
  if (rows > 0) LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, bm_swiglu_bwd, prefix, st));
  if (rows > 0)
    LAUNCH_NAMED("gemm_down_dgrad_swiglu_bwd", gemm_down_dgrad_swiglu_bwd<T>(dy_perm, off, prefix, E, w2, hu, dhu, rows, d, f,
                                                                             rg, dg_part, act_rec, st));
  if (rg && rows > 0)
    LAUNCH_NAMED("gate_grad_sum", launch_gate_grad_sum(dg_part, gemm_dg_parts(bf, f), row_id_map, rows, d_gates, st));
  // weight gradients cover every expert (empty experts get zeros)
  LAUNCH_NAMED("gemm_wgrad_down", gemm_wgrad<T>(dy_perm, d, act_rec ? act_rec : act, f, off, E, 0, dw2, 1, st));
  if (rows > 0 && bm_dgrad != bm_swiglu_bwd)
    LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, bm_dgrad, prefix, st));
  if (rows > 0) LAUNCH_NAMED("gemm_gateup_dgrad", gemm_gateup_dgrad<T>(dhu, off, prefix, E, w13, dx_perm, false, rows, d, f, st));
  LAUNCH_NAMED("gemm_wgrad_gateup", gemm_wgrad<T>(dhu, 2 * f, x_perm, d, off, E, 0, dw13, 0, st));
  if (c->f_shared > 0) {
    const int fs = (int)c->f_shared;
    // (the routed experts are done with act_rec: the shared expert's act goes there)
    if (T_ > 0) LAUNCH_NAMED("gemm_down_dgrad_swiglu_bwd_shared", gemm_down_dgrad_swiglu_bwd<T>(dy, nullptr, nullptr, 1, ws2, hu_s, dhu_s, T_, d, fs,
                                                                                               nullptr, nullptr, act_rec, st));
    LAUNCH_NAMED("gemm_wgrad_down_shared", gemm_wgrad<T>(dy, d, act_rec ? act_rec : act_s, fs, nullptr, 1, T_, dws2, 3, st));
    if (T_ > 0) LAUNCH_NAMED("gemm_gateup_dgrad_shared", gemm_gateup_dgrad<T>(dhu_s, nullptr, nullptr, 1, ws13, dx_partial, true, T_, d, fs, st));
    LAUNCH_NAMED("gemm_wgrad_gateup_shared", gemm_wgrad<T>(dhu_s, 2 * fs, x, d, nullptr, 1, T_, dws13, 2, st));
  } else {
    LAUNCH_NAMED("fill_f32", launch_fill_f32(dx_partial, (int64_t)T_ * d, 0.0f, st));
  }
  return ok();
}

template <class T>
moe_status router_bwd_impl(const moe_cfg* c, const void* x, const void* w_router, const float* logits,
                           const int32_t* idx, const float* gates, const int32_t* counts,
                           const float* d_gates, float d_aux, float* d_logits, void* dw_router,
                           float* dx_partial, void* ws, hipStream_t st) {
  RouterParams p = router_params(c);
  const int T_ = (int)c->T, E = (int)c->E, d = (int)c->d;
  const bool bf = sizeof(T) == 2;
  const int Ep = bf ? (int)pad64(E) : E;   // K of the router dgrad: a multiple of 64
  T* dl_store = bf ? (T*)ws : nullptr;
  LAUNCH_NAMED("router_bwd", launch_router_bwd<T>(logits, idx, gates, d_gates, counts, p, d_aux, d_logits, dl_store, Ep, st));
  const void* dl = bf ? (const void*)dl_store : (const void*)d_logits;
  float* wparts = (float*)((char*)ws + align256((size_t)T_ * Ep * sizeof(T)));
  LAUNCH_NAMED("gemm_router_wgrad", gemm_router_wgrad<T>(dl, Ep, E, x, T_, d, dw_router, wparts, st));
  if (T_ > 0) LAUNCH_NAMED("gemm_router_dgrad", gemm_router_dgrad<T>(dl, Ep, E, w_router, T_, d, dx_partial, st));
  return ok();
}


// ---- MXFP8 expert GEMMs --------------------------------------------------------
struct MxBufs {
  int* prefix;
  int* bpre;            // 32-row block prefix of the weight gradients' operands
  uint8_t *qa_c, *qa_s;  // row form of a GEMM's activation operand
  uint8_t *qb_c, *qb_s;  // row form of act / dHU, written by the product that forms them
  void *qd1, *qd2;      // weight-gradient operands, quantised and widened to bf16
  void* act_rec;        // act formed again (recomputation) or NULL
  float* dg_part;       // folded gates' gradient partials or NULL
};
MxBufs mx_bufs(const moe_cfg* c, void* ws) {
  const MxWs w = mx_ws(c);
  uint8_t* p = (uint8_t*)ws;
  MxBufs b;
  b.prefix = (int*)p;
  b.bpre = (int*)(p + w.ints / 2);
  p += w.ints;
  b.qa_c = p;
  b.qa_s = p + align256((size_t)(w.rows_max * w.cmax_rows));
  p += w.qa;
  b.qb_c = p;
  b.qb_s = p + align256((size_t)(w.rows_max * w.cmax_rows));
  p += w.qa;
  b.qd1 = p;
  p += w.qt;
  b.qd2 = p;
  b.act_rec = recompute(c) ? (uint8_t*)ws + w.extra.act : nullptr;
  b.dg_part = fold(c) ? (float*)((uint8_t*)ws + w.extra.dg) : nullptr;
  return b;
}
inline MxQ mxq(const uint8_t* c, const uint8_t* s) { return MxQ{c, s}; }
inline MxQ mxq(const moe_mx_tensor& t) { return MxQ{t.codes, t.scales}; }

moe_status mx_fwd_impl(const moe_cfg* c, const void* x_perm, const int32_t* off, const float* row_gates,
                       const moe_mx_weights* w, void* hu, void* act, void* y_perm, const void* x, void* hu_s,
                       void* act_s, void* y_s, void* ws, hipStream_t st) {
  const bool rc = recompute(c), fp4 = is_fp4(c);
  const float* rg = fold(c) ? row_gates : nullptr;
  const int E = (int)c->E, rows = (int)(c->T * c->k), d = (int)c->d, f = (int)c->f, T_ = (int)c->T;
  MxBufs b = mx_bufs(c, ws);
  const MxQ qa = mxq(b.qa_c, b.qa_s), qb = mxq(b.qb_c, b.qb_s);
  if (rows > 0) {
    LAUNCH_NAMED("mx_quant_rows", launch_mx_quant_rows(x_perm, d, 0, 1, rows, d, b.qa_c, b.qa_s, fp4, true, st));
    LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, 128, b.prefix, st));
    // the SwiGLU epilogue writes act's row form beside act
    LAUNCH_NAMED("gemm_mx_swiglu_fwd", gemm_mx_swiglu_fwd(qa, off, b.prefix, E, mxq(w->w13), hu, act, rows, d, f, rg, rc,
                                                          fp4, b.qb_c, b.qb_s, st));
    LAUNCH_NAMED("gemm_mx_down_fwd", gemm_mx_down_fwd(qb, off, b.prefix, E, mxq(w->w2), y_perm, rows, d, f, fp4, st));
  }
  if (c->f_shared > 0 && T_ > 0) {
    const int fs = (int)c->f_shared;
    LAUNCH_NAMED("mx_quant_rows", launch_mx_quant_rows(x, d, 0, 1, T_, d, b.qa_c, b.qa_s, fp4, true, st));
    LAUNCH_NAMED("gemm_mx_swiglu_fwd_shared",
                 gemm_mx_swiglu_fwd(qa, nullptr, nullptr, 1, mxq(w->ws13), hu_s, act_s, T_, d, fs, nullptr, rc, fp4,
                                    b.qb_c, b.qb_s, st));
    LAUNCH_NAMED("gemm_mx_down_fwd_shared",
                 gemm_mx_down_fwd(qb, nullptr, nullptr, 1, mxq(w->ws2), y_s, T_, d, fs, fp4, st));
  }
  return ok();
}

moe_status mx_bwd_impl(const moe_cfg* c, const void* dy_perm, const void* x_perm, const int32_t* off,
                       const float* row_gates, const int32_t* row_id_map, const void* hu, const void* act,
                       const moe_mx_weights* w, void* dhu, void* dx_perm, void* dw13, void* dw2, float* d_gates,
                       const void* dy, const void* x, const void* hu_s, const void* act_s, void* dhu_s,
                       float* dx_partial, void* dws13, void* dws2, void* ws, hipStream_t st) {
  const int E = (int)c->E, rows = (int)(c->T * c->k), d = (int)c->d, f = (int)c->f, T_ = (int)c->T;
  MxBufs b = mx_bufs(c, ws);
  const bool fp4 = is_fp4(c);
  const float* rg = fold(c) ? row_gates : nullptr;
  if (b.act_rec) {                  // recomputation: the backward reads the act it forms again
    act = b.act_rec;
    act_s = b.act_rec;              // (the shared expert's, after the routed experts are done with it)
  }
  const MxQ qa = mxq(b.qa_c, b.qa_s), qb = mxq(b.qb_c, b.qb_s);
  // Weight gradients contract over the rows: both operands are quantised along
  // the rows (32-row blocks restarting at each expert's first row) and widened
  // back to bf16, where every microscaled value is exact, and multiplied by the
  // bf16 weight-gradient kernels.  These products are bound by writing their
  // bf16 outputs, which the stationary-band kernel does best; the products are
  // the microscaled ones (exact in either form, fp32 accumulation).
  auto wgrad = [&](const void* P, int M, const void* Q, int N, const int* offs, int G, int rows_k, void* dw,
                   int site) -> moe_status {
    LAUNCH_NAMED("mx_qdq_rows", launch_mx_qdq_rows(P, M, rows_k, M, offs, b.bpre, G, b.qd1, M, fp4, st));
    LAUNCH_NAMED("mx_qdq_rows", launch_mx_qdq_rows(Q, N, rows_k, N, offs, b.bpre, G, b.qd2, N, fp4, st));
    static const char* const kName[4] = {"gemm_mx_wgrad_gateup", "gemm_mx_wgrad_down", "gemm_mx_wgrad_gateup_shared",
                                         "gemm_mx_wgrad_down_shared"};
    LAUNCH_NAMED(kName[site], gemm_wgrad<bf16>(b.qd1, M, b.qd2, N, offs, G, offs ? 0 : rows_k, dw, site, st));
    return ok();
  };
  if (rows > 0) {
    LAUNCH_NAMED("mx_quant_rows", launch_mx_quant_rows(dy_perm, d, 0, 1, rows, d, b.qa_c, b.qa_s, fp4, true, st));
    LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, 128, b.prefix, st));
    LAUNCH_NAMED("gemm_mx_down_dgrad_swiglu_bwd",
                 gemm_mx_down_dgrad_swiglu_bwd(qa, off, b.prefix, E, mxq(w->w2_t), hu, dhu, rows, d, f, rg, b.dg_part,
                                               b.act_rec, fp4, b.qb_c, b.qb_s, st));
    if (rg)
      LAUNCH_NAMED("gate_grad_sum", launch_gate_grad_sum(b.dg_part, gemm_dg_parts(true, f), row_id_map, rows, d_gates, st));
  }
  // weight gradients cover every expert: experts without rows get zeros
  LAUNCH_NAMED("tile_prefix", launch_tile_prefix(off, E, 32, b.bpre, st));
  CHECK(wgrad(dy_perm, d, act, f, off, E, rows, dw2, 1));
  if (rows > 0) {
    // (dHU's row form was written by the SwiGLU-backward epilogue)
    LAUNCH_NAMED("gemm_mx_gateup_dgrad",
                 gemm_mx_gateup_dgrad(qb, off, b.prefix, E, mxq(w->w13_t), dx_perm, false, rows, d, f, fp4, st));
  }
  CHECK(wgrad(dhu, 2 * f, x_perm, d, off, E, rows, dw13, 0));
  if (c->f_shared > 0) {
    const int fs = (int)c->f_shared;
    if (T_ > 0) {
      LAUNCH_NAMED("mx_quant_rows", launch_mx_quant_rows(dy, d, 0, 1, T_, d, b.qa_c, b.qa_s, fp4, true, st));
      LAUNCH_NAMED("gemm_mx_down_dgrad_swiglu_bwd_shared",
                   gemm_mx_down_dgrad_swiglu_bwd(qa, nullptr, nullptr, 1, mxq(w->ws2_t), hu_s, dhu_s, T_, d, fs, nullptr,
                                                 nullptr, b.act_rec, fp4, b.qb_c, b.qb_s, st));
    }
    CHECK(wgrad(dy, d, act_s, fs, nullptr, 1, T_, dws2, 3));
    if (T_ > 0) {
      LAUNCH_NAMED("gemm_mx_gateup_dgrad_shared",
                   gemm_mx_gateup_dgrad(qb, nullptr, nullptr, 1, mxq(w->ws13_t), dx_partial, true, T_, d, fs, fp4, st));
    }
    CHECK(wgrad(dhu_s, 2 * fs, x, d, nullptr, 1, T_, dws13, 2));
  } else {
    LAUNCH_NAMED("fill_f32", launch_fill_f32(dx_partial, (int64_t)T_ * d, 0.0f, st));
  }
  return ok();
}

// ---- the grouped-GEMM forward without a caller workspace ----------------------
// Its one scratch buffer, the device-built tile prefix (E + 2 <= 258 ints), lives
// in this file-scope device array instead: every GPU the library runs on holds
// its own copy until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address of each
// GPU's copy is looked up once, with that device current, and kept per device.
constexpr int kNoAllocScratchInts = 1024;            // 4 KiB
static __device__ __align__(256) int g_noalloc_scratch[kNoAllocScratchInts];
void* g_noalloc_ptr[kMaxDevices] = {};
std::mutex g_noalloc_mu;

moe_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_INVALID_ARGUMENT, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_noalloc_scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return MOE_OK;
}

moe_status check_mx_tensor(const moe_mx_tensor& t, const char* name) {
  if (!t.codes || !t.scales) return fail(MOE_ERR_INVALID_ARGUMENT, "weights.%s: codes and scales must not be NULL", name);
  if (((uintptr_t)t.codes & 15) || ((uintptr_t)t.scales & 3))
    return fail(MOE_ERR_INVALID_ARGUMENT, "weights.%s: codes must be 16-byte and scales 4-byte aligned", name);
  return MOE_OK;
}
}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_trace_begin(int capacity) {
  if (capacity < 1 || capacity > (1 << 20))
    return fail(MOE_ERR_INVALID_ARGUMENT, "trace capacity %d outside [1, 2^20]", capacity);
  if (g_trace.on) return fail(MOE_ERR_INVALID_ARGUMENT, "a trace is already active on this thread");
  g_trace.ev.assign(2 * (size_t)capacity, nullptr);
  g_trace.names.assign(capacity, nullptr);
  for (auto& e : g_trace.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (auto& q : g_trace.ev)
        if (q) hipEventDestroy(q);
      g_trace.ev.clear();
      return fail(MOE_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorString(r));
    }
  }
  g_trace.cap = capacity;
  g_trace.n = 0;
  g_trace.on = true;
  return ok();
}

int moe_trace_end(const char** names, float* ms, int capacity) {
  if (!g_trace.on) return 0;
  g_trace.on = false;
  int n = g_trace.n, rc = n;
  for (int i = 0; i < n && i < capacity; ++i) {
    float t = 0.0f;
    if (hipEventSynchronize(g_trace.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess)
      rc = -1;
    if (names) names[i] = g_trace.names[i];
    if (ms) ms[i] = t;
  }
  for (auto& e : g_trace.ev) hipEventDestroy(e);
  g_trace.ev.clear();
  g_trace.names.clear();
  return rc;
}

moe_status moe_init(int device) {
  CHECK(check_device(device));
  return ok();
}

size_t moe_workspace_size(const moe_cfg* cfg) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  g_err.clear();
  return ws_bytes_for(cfg);
}

moe_status moe_router_topk(const moe_cfg* cfg, const void* x, const void* w_router, const float* bias,
                           float* logits, int32_t* topk_idx, float* topk_gates, int32_t* expert_counts,
                           float* aux_loss, void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  if ((x == nullptr) != (w_router == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x and w_router must both be given or both be NULL");
  if (x) CHECK(check_gemm_shapes(cfg));
  REQ(logits); REQ(topk_idx); REQ(topk_gates); REQ(expert_counts);
  if (cfg->aux_coeff != 0.0f) REQ(aux_loss);
  ALIGNED(x); ALIGNED(w_router); ALIGNED(logits);
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  if (cfg->dtype != MOE_F32)
    return router_topk_impl<bf16>(cfg, x, w_router, bias, logits, topk_idx, topk_gates, expert_counts,
                                  aux_loss, workspace, st);
  return router_topk_impl<float>(cfg, x, w_router, bias, logits, topk_idx, topk_gates, expert_counts,
                                 aux_loss, workspace, st);
}

moe_status moe_router_bias_update(const moe_cfg* cfg, const int32_t* expert_counts, float rate, float* bias,
                                  void* stream) {
  CHECK(check_cfg(cfg));
  REQ(expert_counts); REQ(bias);
  if (!(rate >= 0.0f && rate <= 3.0e38f)) return fail(MOE_ERR_INVALID_ARGUMENT, "rate must be finite and >= 0");
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  LAUNCH_NAMED("router_bias_update",
               launch_router_bias_update(expert_counts, (int)cfg->E, cfg->T * cfg->k, rate, bias, st));
  return ok();
}

moe_status moe_permute(const moe_cfg* cfg, const void* x, const int32_t* topk_idx, const float* topk_gates,
                       int32_t* expert_offsets, int32_t* row_id_map, int32_t* src_token, float* row_gates,
                       void* x_perm, void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  REQ(x); REQ(topk_idx); REQ(expert_offsets); REQ(row_id_map); REQ(src_token); REQ(x_perm);
  if (fold(cfg)) { REQ(topk_gates); REQ(row_gates); }
  if ((topk_gates == nullptr) != (row_gates == nullptr))
    return fail(MOE_ERR_INVALID_ARGUMENT, "topk_gates and row_gates must both be given or both be NULL");
  ALIGNED(x); ALIGNED(x_perm);
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  const int T_ = (int)cfg->T, k = (int)cfg->k, E = (int)cfg->E, rows = T_ * k;
  int* hist = (int*)workspace;
  LAUNCH_NAMED("perm_hist", launch_perm_hist(topk_idx, T_, k, E, hist, st));
  LAUNCH_NAMED("perm_scan", launch_perm_scan(hist, (int)ranges(T_), E, rows, expert_offsets, st));
  LAUNCH_NAMED("perm_rank", launch_perm_rank(topk_idx, T_, k, E, hist, row_id_map, src_token, topk_gates, row_gates,
                                             st));
  LAUNCH_NAMED("scatter_rows", launch_scatter_rows(x, row_id_map, T_, k, (int)(cfg->d * elt(cfg)), x_perm, st));
  return ok();
}

moe_status moe_grouped_gemm_swiglu(const moe_cfg* cfg, const void* x_perm, const int32_t* expert_offsets,
                                   const float* row_gates, const void* w13, const void* w2, void* hu_save,
                                   void* act, void* y_perm, const void* x, const void* ws13, const void* ws2,
                                   void* hu_shared_save, void* act_shared, void* y_shared, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_not_mx(cfg));
  CHECK(check_gemm_shapes(cfg));
  REQ(x_perm); REQ(expert_offsets); REQ(w13); REQ(w2); REQ(act); REQ(y_perm);
  if (fold(cfg)) REQ(row_gates);
  ALIGNED(x_perm); ALIGNED(w13); ALIGNED(w2); ALIGNED(hu_save); ALIGNED(act); ALIGNED(y_perm);
  if (cfg->f_shared > 0) {
    REQ(x); REQ(ws13); REQ(ws2); REQ(act_shared); REQ(y_shared);
    ALIGNED(x); ALIGNED(ws13); ALIGNED(ws2); ALIGNED(hu_shared_save); ALIGNED(act_shared); ALIGNED(y_shared);
  }
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  if (cfg->dtype != MOE_F32)
    return gemm_fwd_impl<bf16>(cfg, x_perm, expert_offsets, row_gates, w13, w2, hu_save, act, y_perm, x, ws13,
                               ws2, hu_shared_save, act_shared, y_shared, workspace, st);
  return gemm_fwd_impl<float>(cfg, x_perm, expert_offsets, row_gates, w13, w2, hu_save, act, y_perm, x, ws13,
                              ws2, hu_shared_save, act_shared, y_shared, workspace, st);
}

moe_status moe_grouped_gemm_swiglu_noalloc(const moe_cfg* cfg, const void* x_perm,
                                           const int32_t* expert_offsets, const float* row_gates,
                                           const void* w13, const void* w2, void* hu_save, void* act,
                                           void* y_perm, const void* x, const void* ws13, const void* ws2,
                                           void* hu_shared_save, void* act_shared, void* y_shared,
                                           void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_not_mx(cfg));
  CHECK(check_gemm_shapes(cfg));
  REQ(x_perm); REQ(expert_offsets); REQ(w13); REQ(w2); REQ(act); REQ(y_perm);
  if (fold(cfg)) REQ(row_gates);
  ALIGNED(x_perm); ALIGNED(w13); ALIGNED(w2); ALIGNED(hu_save); ALIGNED(act); ALIGNED(y_perm);
  if (cfg->f_shared > 0) {
    REQ(x); REQ(ws13); REQ(ws2); REQ(act_shared); REQ(y_shared);
    ALIGNED(x); ALIGNED(ws13); ALIGNED(ws2); ALIGNED(hu_shared_save); ALIGNED(act_shared); ALIGNED(y_shared);
  }
  // the forward's scratch is the tile prefix: E + 2 ints
  if (cfg->E + 2 > kNoAllocScratchInts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "E = %lld needs %lld scratch ints, the static scratch holds %d",
                (long long)cfg->E, (long long)cfg->E + 2, kNoAllocScratchInts);
  CHECK(check_current_device());
  void* scratch = nullptr;
  CHECK(noalloc_scratch(&scratch));
  hipStream_t st = (hipStream_t)stream;
  if (cfg->dtype != MOE_F32)
    return gemm_fwd_impl<bf16>(cfg, x_perm, expert_offsets, row_gates, w13, w2, hu_save, act, y_perm, x, ws13,
                               ws2, hu_shared_save, act_shared, y_shared, scratch, st);
  return gemm_fwd_impl<float>(cfg, x_perm, expert_offsets, row_gates, w13, w2, hu_save, act, y_perm, x, ws13,
                              ws2, hu_shared_save, act_shared, y_shared, scratch, st);
}

moe_status moe_unpermute_combine(const moe_cfg* cfg, const void* y_perm, const int32_t* row_id_map,
                                 const float* topk_gates, const void* y_shared, void* y, void* stream) {
  CHECK(check_cfg(cfg));
  REQ(y_perm); REQ(row_id_map); REQ(y);
  if (!fold(cfg)) REQ(topk_gates);
  ALIGNED(y_perm); ALIGNED(y_shared); ALIGNED(y);
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  const int T_ = (int)cfg->T, k = (int)cfg->k, d = (int)cfg->d;
  if (fold(cfg)) topk_gates = nullptr;      // the rows carry their gates: an unweighted sum
  if (cfg->dtype != MOE_F32)
    LAUNCH_NAMED("combine", launch_combine<bf16>((const bf16*)y_perm, row_id_map, topk_gates, (const bf16*)y_shared, (bf16*)y,
                                T_, k, d, st));
  else
    LAUNCH_NAMED("combine", launch_combine<float>((const float*)y_perm, row_id_map, topk_gates, (const float*)y_shared,
                                 (float*)y, T_, k, d, st));
  return ok();
}

moe_status moe_unpermute_combine_bwd(const moe_cfg* cfg, const void* dy, const void* y_perm,
                                     const int32_t* row_id_map, const float* topk_gates, void* dy_perm,
                                     float* d_gates, void* stream) {
  CHECK(check_cfg(cfg));
  REQ(dy); REQ(row_id_map); REQ(dy_perm);
  ALIGNED(dy); ALIGNED(dy_perm);
  if (fold(cfg)) {
    // the rows carry their gates: dy_perm[row(t,j)] = dy[t]; d_gates comes from
    // the grouped-GEMM backward
    CHECK(check_current_device());
    hipStream_t st = (hipStream_t)stream;
    LAUNCH_NAMED("scatter_rows", launch_scatter_rows(dy, row_id_map, (int)cfg->T, (int)cfg->k,
                                                     (int)(cfg->d * elt(cfg)), dy_perm, st));
    return ok();
  }
  REQ(y_perm); REQ(topk_gates); REQ(d_gates);
  ALIGNED(y_perm);
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  const int T_ = (int)cfg->T, k = (int)cfg->k, d = (int)cfg->d;
  if (cfg->dtype != MOE_F32)
    LAUNCH_NAMED("combine_bwd", launch_combine_bwd<bf16>((const bf16*)dy, (const bf16*)y_perm, row_id_map, topk_gates,
                                    (bf16*)dy_perm, d_gates, T_, k, d, st));
  else
    LAUNCH_NAMED("combine_bwd", launch_combine_bwd<float>((const float*)dy, (const float*)y_perm, row_id_map, topk_gates,
                                     (float*)dy_perm, d_gates, T_, k, d, st));
  return ok();
}

moe_status moe_grouped_gemm_swiglu_bwd(const moe_cfg* cfg, const void* dy_perm, const void* x_perm,
                                       const int32_t* expert_offsets, const float* row_gates,
                                       const int32_t* row_id_map, const void* hu_save, const void* act,
                                       const void* w13, const void* w2, void* dhu, void* dx_perm, void* dw13,
                                       void* dw2, float* d_gates, const void* dy, const void* x,
                                       const void* hu_shared_save, const void* act_shared, const void* ws13,
                                       const void* ws2, void* dhu_shared, float* dx_partial, void* dws13,
                                       void* dws2, void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_not_mx(cfg));
  CHECK(check_gemm_shapes(cfg));
  REQ(dy_perm); REQ(x_perm); REQ(expert_offsets); REQ(hu_save); REQ(w13); REQ(w2);
  REQ(dhu); REQ(dx_perm); REQ(dw13); REQ(dw2); REQ(dx_partial);
  if (!recompute(cfg)) REQ(act);
  if (fold(cfg)) { REQ(row_gates); REQ(row_id_map); REQ(d_gates); }
  ALIGNED(dy_perm); ALIGNED(x_perm); ALIGNED(hu_save); ALIGNED(act); ALIGNED(w13); ALIGNED(w2);
  ALIGNED(dhu); ALIGNED(dx_perm); ALIGNED(dw13); ALIGNED(dw2); ALIGNED(dx_partial);
  if (cfg->f_shared > 0) {
    REQ(dy); REQ(x); REQ(hu_shared_save); REQ(ws13); REQ(ws2); REQ(dhu_shared);
    REQ(dws13); REQ(dws2);
    if (!recompute(cfg)) REQ(act_shared);
    ALIGNED(dy); ALIGNED(x); ALIGNED(hu_shared_save); ALIGNED(act_shared); ALIGNED(ws13); ALIGNED(ws2);
    ALIGNED(dhu_shared); ALIGNED(dws13); ALIGNED(dws2);
  }
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  if (cfg->dtype != MOE_F32)
    return gemm_bwd_impl<bf16>(cfg, dy_perm, x_perm, expert_offsets, row_gates, row_id_map, hu_save, act, w13, w2,
                               dhu, dx_perm, dw13, dw2, d_gates, dy, x, hu_shared_save, act_shared, ws13, ws2,
                               dhu_shared, dx_partial, dws13, dws2, workspace, st);
  return gemm_bwd_impl<float>(cfg, dy_perm, x_perm, expert_offsets, row_gates, row_id_map, hu_save, act, w13, w2,
                              dhu, dx_perm, dw13, dw2, d_gates, dy, x, hu_shared_save, act_shared, ws13, ws2,
                              dhu_shared, dx_partial, dws13, dws2, workspace, st);
}

moe_status moe_router_topk_bwd(const moe_cfg* cfg, const void* x, const void* w_router, const float* logits,
                               const int32_t* topk_idx, const float* topk_gates, const int32_t* expert_counts,
                               const float* d_gates, float d_aux, float* d_logits, void* dw_router,
                               float* dx_partial, void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_gemm_shapes(cfg));
  REQ(x); REQ(w_router); REQ(logits); REQ(topk_idx); REQ(topk_gates); REQ(d_gates); REQ(d_logits);
  REQ(dw_router); REQ(dx_partial);
  if (cfg->aux_coeff != 0.0f) REQ(expert_counts);
  ALIGNED(x); ALIGNED(w_router); ALIGNED(logits); ALIGNED(d_logits); ALIGNED(dw_router); ALIGNED(dx_partial);
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  if (cfg->dtype != MOE_F32)
    return router_bwd_impl<bf16>(cfg, x, w_router, logits, topk_idx, topk_gates, expert_counts, d_gates, d_aux,
                                 d_logits, dw_router, dx_partial, workspace, st);
  return router_bwd_impl<float>(cfg, x, w_router, logits, topk_idx, topk_gates, expert_counts, d_gates, d_aux,
                                d_logits, dw_router, dx_partial, workspace, st);
}

moe_status moe_permute_bwd(const moe_cfg* cfg, const void* dx_perm, const int32_t* row_id_map,
                           const float* dx_partial, void* dx, void* stream) {
  CHECK(check_cfg(cfg));
  REQ(dx_perm); REQ(row_id_map); REQ(dx);
  ALIGNED(dx_perm); ALIGNED(dx_partial); ALIGNED(dx);
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  const int T_ = (int)cfg->T, k = (int)cfg->k, d = (int)cfg->d;
  if (cfg->dtype != MOE_F32)
    LAUNCH_NAMED("unpermute_sum", launch_unpermute_sum<bf16>((const bf16*)dx_perm, row_id_map, dx_partial, (bf16*)dx, T_, k, d, st));
  else
    LAUNCH_NAMED("unpermute_sum", launch_unpermute_sum<float>((const float*)dx_perm, row_id_map, dx_partial, (float*)dx, T_, k, d, st));
  return ok();
}


static moe_status quantize_mx(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t orientation,
                              uint8_t* codes, uint8_t* scales, bool fp4, void* stream) {
  REQ(src); REQ(codes); REQ(scales);
  ALIGNED(src); ALIGNED(codes);
  if (batch < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "negative size");
  if (batch > 65535) return fail(MOE_ERR_INVALID_ARGUMENT, "batch = %lld above 65535", (long long)batch);
  if (rows * cols >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_ARGUMENT, "rows * cols must stay below 2^31");
  const bool grouped = (orientation & MOE_MX_GROUPED) != 0;
  orientation &= ~MOE_MX_GROUPED;
  if (orientation != MOE_MX_ROWS && orientation != MOE_MX_COLS)
    return fail(MOE_ERR_INVALID_ARGUMENT, "orientation %d unknown", orientation);
  if (grouped && (orientation == MOE_MX_ROWS ? cols : rows) % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "grouped scales need the blocked dimension %% 128 == 0 (%lld x %lld)",
                (long long)rows, (long long)cols);
  if (orientation == MOE_MX_ROWS && cols % 32)
    return fail(MOE_ERR_INVALID_ARGUMENT, "row orientation needs cols %% 32 == 0 (cols = %lld)", (long long)cols);
  if (orientation == MOE_MX_COLS && (rows % 32 || cols % 8))
    return fail(MOE_ERR_INVALID_ARGUMENT, "column orientation needs rows %% 32 == 0 and cols %% 8 == 0 (%lld x %lld)",
                (long long)rows, (long long)cols);
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  if (orientation == MOE_MX_ROWS)
    LAUNCH_NAMED("mx_quant_rows", launch_mx_quant_rows(src, cols, rows * cols, (int)batch, (int)rows, (int)cols,
                                                       codes, scales, fp4, grouped, st));
  else
    LAUNCH_NAMED("mx_quant_cols", launch_mx_quant_cols_batched(src, (int)batch, (int)rows, (int)cols, codes,
                                                               scales, fp4, grouped, st));
  return ok();
}

moe_status moe_quantize_mxfp8(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t orientation,
                              uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_mx(src, batch, rows, cols, orientation, codes, scales, false, stream);
}

static moe_status quantize_mx_both(const void* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_r,
                                   uint8_t* scales_r, uint8_t* codes_c, uint8_t* scales_c, int32_t flags, bool fp4,
                                   void* stream) {
  REQ(src); REQ(codes_r); REQ(scales_r); REQ(codes_c); REQ(scales_c);
  ALIGNED(src); ALIGNED(codes_r); ALIGNED(codes_c);
  if (batch < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "negative size");
  if (batch > 65535) return fail(MOE_ERR_INVALID_ARGUMENT, "batch = %lld above 65535", (long long)batch);
  if (rows * cols >= ((int64_t)1 << 31)) return fail(MOE_ERR_INVALID_ARGUMENT, "rows * cols must stay below 2^31");
  if (flags != 0 && flags != MOE_MX_GROUPED) return fail(MOE_ERR_INVALID_ARGUMENT, "flags %d unknown", flags);
  const bool grouped = flags == MOE_MX_GROUPED;
  if (rows % 32 || cols % 32)
    return fail(MOE_ERR_INVALID_ARGUMENT, "both orientations need rows and cols multiples of 32 (%lld x %lld)",
                (long long)rows, (long long)cols);
  if (grouped && (rows % 128 || cols % 128))
    return fail(MOE_ERR_INVALID_ARGUMENT, "grouped scales need rows and cols multiples of 128 (%lld x %lld)",
                (long long)rows, (long long)cols);
  CHECK(check_current_device());
  hipStream_t st = (hipStream_t)stream;
  LAUNCH_NAMED("mx_quant_both", launch_mx_quant_both(src, (int)batch, (int)rows, (int)cols, codes_r, scales_r,
                                                     codes_c, scales_c, fp4, grouped, st));
  return ok();
}

moe_status moe_quantize_mxfp8_both(const void* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_rows,
                                   uint8_t* scales_rows, uint8_t* codes_cols, uint8_t* scales_cols, int32_t flags,
                                   void* stream) {
  return quantize_mx_both(src, batch, rows, cols, codes_rows, scales_rows, codes_cols, scales_cols, flags, false,
                          stream);
}

moe_status moe_quantize_mxfp4_both(const void* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes_rows,
                                   uint8_t* scales_rows, uint8_t* codes_cols, uint8_t* scales_cols, int32_t flags,
                                   void* stream) {
  return quantize_mx_both(src, batch, rows, cols, codes_rows, scales_rows, codes_cols, scales_cols, flags, true,
                          stream);
}

moe_status moe_quantize_mxfp4(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t orientation,
                              uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_mx(src, batch, rows, cols, orientation, codes, scales, true, stream);
}

static moe_status grouped_swiglu_mx(int32_t want, const moe_cfg* cfg, const void* x_perm,
                                    const int32_t* expert_offsets, const float* row_gates,
                                    const moe_mx_weights* weights, void* hu_save, void* act, void* y_perm,
                                    const void* x, void* hu_shared_save, void* act_shared, void* y_shared,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_mx_shapes(cfg, want));
  REQ(x_perm); REQ(expert_offsets); REQ(weights); REQ(act); REQ(y_perm);
  if (fold(cfg)) REQ(row_gates);
  ALIGNED(x_perm); ALIGNED(hu_save); ALIGNED(act); ALIGNED(y_perm);
  CHECK(check_mx_tensor(weights->w13, "w13"));
  CHECK(check_mx_tensor(weights->w2, "w2"));
  if (cfg->f_shared > 0) {
    REQ(x); REQ(act_shared); REQ(y_shared);
    ALIGNED(x); ALIGNED(hu_shared_save); ALIGNED(act_shared); ALIGNED(y_shared);
    CHECK(check_mx_tensor(weights->ws13, "ws13"));
    CHECK(check_mx_tensor(weights->ws2, "ws2"));
  }
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  return mx_fwd_impl(cfg, x_perm, expert_offsets, row_gates, weights, hu_save, act, y_perm, x, hu_shared_save,
                     act_shared, y_shared, workspace, (hipStream_t)stream);
}

moe_status moe_grouped_gemm_swiglu_mxfp8(const moe_cfg* cfg, const void* x_perm, const int32_t* expert_offsets,
                                         const float* row_gates, const moe_mx_weights* weights, void* hu_save,
                                         void* act, void* y_perm, const void* x, void* hu_shared_save,
                                         void* act_shared, void* y_shared, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return grouped_swiglu_mx(MOE_MXFP8, cfg, x_perm, expert_offsets, row_gates, weights, hu_save, act, y_perm, x,
                           hu_shared_save, act_shared, y_shared, workspace, workspace_bytes, stream);
}

moe_status moe_grouped_gemm_swiglu_mxfp4(const moe_cfg* cfg, const void* x_perm, const int32_t* expert_offsets,
                                         const float* row_gates, const moe_mx_weights* weights, void* hu_save,
                                         void* act, void* y_perm, const void* x, void* hu_shared_save,
                                         void* act_shared, void* y_shared, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return grouped_swiglu_mx(MOE_MXFP4, cfg, x_perm, expert_offsets, row_gates, weights, hu_save, act, y_perm, x,
                           hu_shared_save, act_shared, y_shared, workspace, workspace_bytes, stream);
}

static moe_status grouped_swiglu_bwd_mx(int32_t want, const moe_cfg* cfg, const void* dy_perm,
                                        const void* x_perm, const int32_t* expert_offsets, const float* row_gates,
                                        const int32_t* row_id_map, const void* hu_save, const void* act,
                                        const moe_mx_weights* weights, void* dhu, void* dx_perm, void* dw13,
                                        void* dw2, float* d_gates, const void* dy, const void* x,
                                        const void* hu_shared_save, const void* act_shared, void* dhu_shared,
                                        float* dx_partial, void* dws13, void* dws2, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_mx_shapes(cfg, want));
  REQ(dy_perm); REQ(x_perm); REQ(expert_offsets); REQ(hu_save); REQ(weights);
  REQ(dhu); REQ(dx_perm); REQ(dw13); REQ(dw2); REQ(dx_partial);
  if (!recompute(cfg)) REQ(act);
  if (fold(cfg)) { REQ(row_gates); REQ(row_id_map); REQ(d_gates); }
  ALIGNED(dy_perm); ALIGNED(x_perm); ALIGNED(hu_save); ALIGNED(act); ALIGNED(dhu); ALIGNED(dx_perm);
  ALIGNED(dw13); ALIGNED(dw2); ALIGNED(dx_partial);
  CHECK(check_mx_tensor(weights->w13_t, "w13_t"));
  CHECK(check_mx_tensor(weights->w2_t, "w2_t"));
  if (cfg->f_shared > 0) {
    REQ(dy); REQ(x); REQ(hu_shared_save); REQ(dhu_shared); REQ(dws13); REQ(dws2);
    if (!recompute(cfg)) REQ(act_shared);
    ALIGNED(dy); ALIGNED(x); ALIGNED(hu_shared_save); ALIGNED(act_shared); ALIGNED(dhu_shared);
    ALIGNED(dws13); ALIGNED(dws2);
    CHECK(check_mx_tensor(weights->ws13_t, "ws13_t"));
    CHECK(check_mx_tensor(weights->ws2_t, "ws2_t"));
  }
  CHECK(check_ws(cfg, workspace, workspace_bytes));
  CHECK(check_current_device());
  return mx_bwd_impl(cfg, dy_perm, x_perm, expert_offsets, row_gates, row_id_map, hu_save, act, weights, dhu,
                     dx_perm, dw13, dw2, d_gates, dy, x, hu_shared_save, act_shared, dhu_shared, dx_partial, dws13,
                     dws2, workspace, (hipStream_t)stream);
}

moe_status moe_grouped_gemm_swiglu_bwd_mxfp8(const moe_cfg* cfg, const void* dy_perm, const void* x_perm,
                                             const int32_t* expert_offsets, const float* row_gates,
                                             const int32_t* row_id_map, const void* hu_save, const void* act,
                                             const moe_mx_weights* weights, void* dhu, void* dx_perm, void* dw13,
                                             void* dw2, float* d_gates, const void* dy, const void* x,
                                             const void* hu_shared_save, const void* act_shared, void* dhu_shared,
                                             float* dx_partial, void* dws13, void* dws2, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return grouped_swiglu_bwd_mx(MOE_MXFP8, cfg, dy_perm, x_perm, expert_offsets, row_gates, row_id_map, hu_save, act,
                              weights, dhu, dx_perm, dw13, dw2, d_gates, dy, x, hu_shared_save, act_shared,
                              dhu_shared, dx_partial, dws13, dws2, workspace, workspace_bytes, stream);
}

moe_status moe_grouped_gemm_swiglu_bwd_mxfp4(const moe_cfg* cfg, const void* dy_perm, const void* x_perm,
                                             const int32_t* expert_offsets, const float* row_gates,
                                             const int32_t* row_id_map, const void* hu_save, const void* act,
                                             const moe_mx_weights* weights, void* dhu, void* dx_perm, void* dw13,
                                             void* dw2, float* d_gates, const void* dy, const void* x,
                                             const void* hu_shared_save, const void* act_shared, void* dhu_shared,
                                             float* dx_partial, void* dws13, void* dws2, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return grouped_swiglu_bwd_mx(MOE_MXFP4, cfg, dy_perm, x_perm, expert_offsets, row_gates, row_id_map, hu_save, act,
                              weights, dhu, dx_perm, dw13, dw2, d_gates, dy, x, hu_shared_save, act_shared,
                              dhu_shared, dx_partial, dws13, dws2, workspace, workspace_bytes, stream);
}

}  // extern "C"
