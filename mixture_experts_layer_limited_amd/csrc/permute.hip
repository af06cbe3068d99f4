// Dispatch and combine on one GPU ("System Modules: Dispatcher" and
// "Combiner"; memory-efficient permutation, Figure 7): a stable counting sort
// of (token, choice) pairs by expert, the row scatter into expert-contiguous
// order (each token row read once, written to its k places), and the gate-weighted unpermute-combine with its backward.
//
// Counting sort: tokens are cut into ranges of 64.  perm_hist counts each
// range's assignments per expert, perm_scan turns the [range, expert] table
// into the first row of every (range, expert) pair, and perm_rank walks each
// range in (token, choice) order one wave at a time, ranking equal expert ids
// inside a 64-entry chunk with ballots over the id's bits.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                        int E, int* __restrict__ hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < kMaxExperts; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.x * kPermTokensPerRange * k;
  const int64_t n1 = min((int64_t)(blockIdx.x + 1) * kPermTokensPerRange, (int64_t)T) * k;
  for (int64_t n = n0 + threadIdx.x; n < n1; n += blockDim.x) atomicAdd(&h[idx[n]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

hipError_t launch_perm_hist(const int32_t* idx, int T, int k, int E, int* hist, hipStream_t st) {
  int R = (T + kPermTokensPerRange - 1) / kPermTokensPerRange;
  if (R == 0) return hipSuccess;
  perm_hist_kernel<<<R, 256, 0, st>>>(idx, T, k, E, hist);
  return hipGetLastError();
}

// hist[r][e] (counts) -> base[r][e] = offsets[e] + sum_{r' < r} hist[r'][e]; offsets[E] = rows.
// Thread e walks its column in batches of kScanBatch ranges: the batch's loads
// are all issued before the running sum uses them, so a column of R entries
// costs R / kScanBatch memory round trips instead of R (the loads and stores
// of one batch are independent).
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(256) void perm_scan_kernel(int* __restrict__ hist, int R, int E, int rows,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int tot[kMaxExperts];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int r0 = 0; r0 < R; r0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = r0 + i < R ? hist[(int64_t)(r0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (r0 + i < R) hist[(int64_t)(r0 + i) * E + e] = run;
        run += c[i];
      }
    }
  }
  tot[e] = (e < E) ? run : 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {      // inclusive scan of the totals
    int add = (e >= o) ? tot[e - o] : 0;
    __syncthreads();
    tot[e] += add;
    __syncthreads();
  }
  if (e < E) {
    const int off = tot[e] - run;            // exclusive
    offsets[e] = off;
    for (int r0 = 0; r0 < R; r0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = r0 + i < R ? hist[(int64_t)(r0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (r0 + i < R) hist[(int64_t)(r0 + i) * E + e] = c[i] + off;
    }
  }
  if (e == 0) offsets[E] = rows;
}

hipError_t launch_perm_scan(int* hist, int R, int E, int rows, int32_t* offsets, hipStream_t st) {
  perm_scan_kernel<<<1, 256, 0, st>>>(hist, R, E, rows, offsets);
  return hipGetLastError();
}

// one wave per token range; entries n = t*k + j in increasing order.  With
// gates, each entry's gate also goes to its row (row_gates: the gate of each
// permuted row, for gate folding).
__global__ __launch_bounds__(64) void perm_rank_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                       int E, const int* __restrict__ base,
                                                       int32_t* __restrict__ row_id_map,
                                                       int32_t* __restrict__ src_token,
                                                       const float* __restrict__ gates,
                                                       float* __restrict__ row_gates) {
  __shared__ int run[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.x * kPermTokensPerRange * k;
  const int64_t n1 = min((int64_t)(blockIdx.x + 1) * kPermTokensPerRange, (int64_t)T) * k;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = n0; c0 < n1; c0 += 64) {
    const int64_t n = c0 + lane;
    const bool valid = n < n1;
    const int e = valid ? idx[n] : 0;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {            // E <= 256: 8 id bits
      uint64_t ones = __ballot(valid && ((e >> b) & 1));
      m &= ((e >> b) & 1) ? ones : ~ones;
    }
    int row = 0;
    if (valid) {
      row = run[e] + __popcll(m & below);
      row_id_map[n] = row;
      src_token[row] = (int32_t)(n / k);
      if (row_gates) row_gates[row] = gates[n];
    }
    __syncthreads();
    // the highest lane of each id group advances that expert's running row
    if (valid && (m >> lane) == 1ull) run[e] += __popcll(m);
    __syncthreads();
  }
}

hipError_t launch_perm_rank(const int32_t* idx, int T, int k, int E, int* base, int32_t* row_id_map,
                            int32_t* src_token, const float* gates, float* row_gates, hipStream_t st) {
  int R = (T + kPermTokensPerRange - 1) / kPermTokensPerRange;
  if (R == 0) return hipSuccess;
  perm_rank_kernel<<<R, 64, 0, st>>>(idx, T, k, E, base, row_id_map, src_token, gates, row_gates);
  return hipGetLastError();
}

// Permute as a scatter: x_perm[row_id_map[t, j]] = x[t] for j < k.  One wave
// per token reads the token's row once (16 bytes per lane) and writes its k
// copies, so the row is fetched once instead of once per copy; every
// destination row is written exactly once (row_id_map is a bijection).
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4* __restrict__ x,
                                                           const int32_t* __restrict__ rmap, int T_, int k,
                                                           int vec_per_row, u32x4* __restrict__ out) {
  const int sub = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + sub;
  if (t >= T_) return;
  const u32x4* in = x + (int64_t)t * vec_per_row;
  const int32_t* rm = rmap + (int64_t)t * k;
  // four 16-byte loads per lane in flight before their stores
  constexpr int U = 4;
  for (int c0 = lane; c0 < vec_per_row; c0 += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + 64 * u < vec_per_row) v[u] = in[c0 + 64 * u];
    for (int j = 0; j < k; ++j) {
      u32x4* o = out + (int64_t)rm[j] * vec_per_row;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + 64 * u < vec_per_row) o[c0 + 64 * u] = v[u];
    }
  }
}

hipError_t launch_scatter_rows(const void* x, const int32_t* row_id_map, int T_, int k, int row_bytes,
                               void* out, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  scatter_rows_kernel<<<(T_ + 3) / 4, 256, 0, st>>>((const u32x4*)x, row_id_map, T_, k, row_bytes / 16,
                                                     (u32x4*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j g[t,j] y_perm[row(t,j)] (+ y_shared[t]), fp32, j order;
// gates NULL (folded into the rows already): the unweighted sum.
// One workgroup per token; each thread owns 8 consecutive elements.
// ---------------------------------------------------------------------------
template <class T>
struct Vec8 {
  float v[8];
  __device__ void load(const T* p) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_f32(p[i]);
  }
  __device__ void store(T* p) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = from_f32<T>(v[i]);
  }
};
template <>
__device__ void Vec8<bf16>::load(const bf16* p) {
  u32x4 w = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_bits_lo(w[i]); v[2 * i + 1] = bf16_bits_hi(w[i]); }
}
template <>
__device__ void Vec8<bf16>::store(bf16* p) const {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *(u32x4*)p = w;
}
template <>
__device__ void Vec8<float>::load(const float* p) {
  floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
template <>
__device__ void Vec8<float>::store(float* p) const {
  floatx4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *(floatx4*)p = a;
  *(floatx4*)(p + 4) = b;
}

// Streaming loads of rows read once (the permuted rows of the combine and of
// the permute backward): non-temporal, so they do not displace lines the
// other reads of the kernel reuse.
template <class T>
__device__ __forceinline__ void load_nt(Vec8<T>& v, const T* p) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = __builtin_nontemporal_load((const u32x4*)p);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v.v[2 * i] = bf16_bits_lo(w[i]); v.v[2 * i + 1] = bf16_bits_hi(w[i]); }
  } else {
    v.load(p);
  }
}

// Work split of the row kernels: a block of kRowThreads threads takes
// kRowTokens consecutive tokens, and its threads walk the tokens' 8-element
// chunks as one sequence (chunk q of the block: token q / vec, chunk q % vec),
// so no pass leaves threads idle when a row's chunk count is not a multiple of
// the block size (d = 7168: 896 chunks a row, 1792 for two tokens = 7 passes
// of 256).
constexpr int kRowThreads = 256, kRowTokens = 2;

// KC > 0: k = KC known at compile time, so the k row loads of a chunk are all
// issued before the sum (0: any k, one row at a time).  The fp32 sum keeps the
// j order either way.
// tokens and threads per block of the forward combine (1, 2, 4, 8 tokens of
// 256 threads: DeepSeek-V3 0.108, 0.109, 0.113, 0.123 ms; one token of 128,
// 256, 448, 896 threads: 0.109, 0.109, 0.105, 0.103 ms -- 896 threads give
// each 16-byte chunk of a d = 7168 row its own thread; Qwen3, d = 4096, 0.107,
// 0.102, 0.101, 0.099 ms).  The unpermute-sum of the backward takes the same
// shape (DeepSeek-V3 0.110 -> 0.103 ms, Qwen3 0.122 -> 0.114 ms against two
// tokens of 256 threads).
constexpr int kCombineTokens = 1, kCombineThreads = 896;

template <class T, int KC>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const T* __restrict__ y_perm,
                                                              const int32_t* __restrict__ rmap,
                                                              const float* __restrict__ gates,
                                                              const T* __restrict__ y_shared, T* __restrict__ y,
                                                              int T_, int k_rt, int d) {
  const int k = KC > 0 ? KC : k_rt;
  const int vec = d / 8;
  const int t0 = blockIdx.x * kCombineTokens;
  const int nq = min(kCombineTokens, T_ - t0) * vec;
  for (int q = threadIdx.x; q < nq; q += kCombineThreads) {
    const int t = t0 + q / vec, c = (q % vec) * 8;
    Vec8<T> acc;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.v[i] = 0.0f;
    if constexpr (KC > 0) {
      Vec8<T> r[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) load_nt(r[j], y_perm + (int64_t)rmap[(int64_t)t * KC + j] * d + c);
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float g = gates ? gates[(int64_t)t * KC + j] : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.v[i] += g * r[j].v[i];
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const int64_t row = rmap[(int64_t)t * k + j];
        const float g = gates ? gates[(int64_t)t * k + j] : 1.0f;
        Vec8<T> r;
        load_nt(r, y_perm + row * d + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.v[i] += g * r.v[i];
      }
    }
    if (y_shared) {
      Vec8<T> sh;
      load_nt(sh, y_shared + (int64_t)t * d + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[i] += sh.v[i];
    }
    acc.store(y + (int64_t)t * d + c);
  }
}

// launch `kern<KC>` for the common k (1, 2, 4, 8), else the runtime-k form
#define MOE_DISPATCH_K(k, LAUNCH) \
  do {                               \
    switch (k) {                     \
      case 1: LAUNCH(1); break;      \
      case 2: LAUNCH(2); break;      \
      case 4: LAUNCH(4); break;      \
      case 8: LAUNCH(8); break;      \
      default: LAUNCH(0); break;     \
    }                                \
  } while (0)

template <class T>
hipError_t launch_combine(const T* y_perm, const int32_t* rmap, const float* gates, const T* y_shared,
                          T* y, int T_, int k, int d, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
#define MOE_L(KC)                                                                                   \
  combine_kernel<T, KC><<<(T_ + kCombineTokens - 1) / kCombineTokens, kCombineThreads, 0, st>>>(y_perm, rmap, gates, \
                                                                                      y_shared, y, T_, k, d)
  MOE_DISPATCH_K(k, MOE_L);
#undef MOE_L
  return hipGetLastError();
}

// dy_perm[row(t,j)] = storage(g dy[t]); d_gates[t,j] = <dy[t], y_perm[row(t,j)]>
// KC > 0 (k known at compile time): the block takes kRowTokens tokens with the
// work split of the combine; each chunk of dy is read once for all k rows, the
// k row loads are issued together, and every thread keeps one dot product per
// (token, j) over its chunks, which are reduced over the block in a fixed order
// (the wave sum, then the waves' partials in wave order).  KC = 0: one token
// per block, one j at a time.
template <class T, int KC>
__global__ __launch_bounds__(kRowThreads) void combine_bwd_kernel(const T* __restrict__ dy,
                                                                  const T* __restrict__ y_perm,
                                                                  const int32_t* __restrict__ rmap,
                                                                  const float* __restrict__ gates,
                                                                  T* __restrict__ dy_perm,
                                                                  float* __restrict__ d_gates, int T_, int k_rt,
                                                                  int d) {
  constexpr int NWV = kRowThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (KC > 0) {
    __shared__ float part[NWV][kRowTokens][KC];
    const int vec = d / 8;
    const int t0 = blockIdx.x * kRowTokens;
    const int ntok = min(kRowTokens, T_ - t0);
    float dot[kRowTokens][KC];
#pragma unroll
    for (int tt = 0; tt < kRowTokens; ++tt)
#pragma unroll
      for (int j = 0; j < KC; ++j) dot[tt][j] = 0.0f;
    for (int q = threadIdx.x; q < ntok * vec; q += kRowThreads) {
      const int tt = q / vec, c = (q % vec) * 8, t = t0 + tt;
      int64_t row[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) row[j] = rmap[(int64_t)t * KC + j];
      Vec8<T> a, r[KC];
      load_nt(a, dy + (int64_t)t * d + c);
#pragma unroll
      for (int j = 0; j < KC; ++j) load_nt(r[j], y_perm + row[j] * d + c);
      float dj[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float g = gates[(int64_t)t * KC + j];
        Vec8<T> o;
        dj[j] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dj[j] += a.v[i] * r[j].v[i];
          o.v[i] = g * a.v[i];
        }
        o.store(dy_perm + row[j] * d + c);
      }
      // a chunk belongs to one token: add its terms to that token's sums
#pragma unroll
      for (int u = 0; u < kRowTokens; ++u)
        if (u == tt)
#pragma unroll
          for (int j = 0; j < KC; ++j) dot[u][j] += dj[j];
    }
#pragma unroll
    for (int tt = 0; tt < kRowTokens; ++tt)
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float w = wave_sum(dot[tt][j]);
        if (lane == 0) part[wave][tt][j] = w;
      }
    __syncthreads();
    if (threadIdx.x < ntok * KC) {
      const int tt = threadIdx.x / KC, j = threadIdx.x % KC;
      float sum = part[0][tt][j];
#pragma unroll
      for (int w = 1; w < NWV; ++w) sum += part[w][tt][j];
      d_gates[(int64_t)(t0 + tt) * KC + j] = sum;
    }
  } else {
    __shared__ float part[NWV];
    const int t = blockIdx.x;
    const int k = k_rt;
    for (int j = 0; j < k; ++j) {
      const int64_t row = rmap[(int64_t)t * k + j];
      const float g = gates[(int64_t)t * k + j];
      float dot = 0.0f;
      for (int c = threadIdx.x * 8; c < d; c += kRowThreads * 8) {
        Vec8<T> a, r, o;
        a.load(dy + (int64_t)t * d + c);
        load_nt(r, y_perm + row * d + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot += a.v[i] * r.v[i];
          o.v[i] = g * a.v[i];
        }
        o.store(dy_perm + row * d + c);
      }
      dot = wave_sum(dot);
      if (lane == 0) part[wave] = dot;
      __syncthreads();
      if (threadIdx.x == 0) {
        float sum = part[0];
        for (int w = 1; w < NWV; ++w) sum += part[w];
        d_gates[(int64_t)t * k + j] = sum;
      }
      __syncthreads();
    }
  }
}

template <class T>
hipError_t launch_combine_bwd(const T* dy, const T* y_perm, const int32_t* rmap, const float* gates, T* dy_perm,
                              float* d_gates, int T_, int k, int d, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
#define MOE_L(KC)                                                                                         \
  combine_bwd_kernel<T, KC><<<KC > 0 ? (T_ + kRowTokens - 1) / kRowTokens : T_, kRowThreads, 0, st>>>(         \
      dy, y_perm, rmap, gates, dy_perm, d_gates, T_, k, d)
  MOE_DISPATCH_K(k, MOE_L);
#undef MOE_L
  return hipGetLastError();
}

// dx[t] = storage(partial[t] + sum_j dx_perm[row(t,j)]), j in order; KC and
// the work split as in combine
template <class T, int KC>
__global__ __launch_bounds__(kCombineThreads) void unpermute_sum_kernel(const T* __restrict__ dx_perm,
                                                                    const int32_t* __restrict__ rmap,
                                                                    const float* __restrict__ partial,
                                                                    T* __restrict__ dx, int T_, int k_rt, int d) {
  const int k = KC > 0 ? KC : k_rt;
  const int vec = d / 8;
  const int t0 = blockIdx.x * kCombineTokens;
  const int nq = min(kCombineTokens, T_ - t0) * vec;
  for (int q = threadIdx.x; q < nq; q += kCombineThreads) {
    const int t = t0 + q / vec, c = (q % vec) * 8;
    Vec8<T> acc;
    if (partial) {
      Vec8<float> p;
      p.load(partial + (int64_t)t * d + c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[i] = p.v[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc.v[i] = 0.0f;
    }
    if constexpr (KC > 0) {
      Vec8<T> r[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) load_nt(r[j], dx_perm + (int64_t)rmap[(int64_t)t * KC + j] * d + c);
#pragma unroll
      for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.v[i] += r[j].v[i];
    } else {
      for (int j = 0; j < k; ++j) {
        const int64_t row = rmap[(int64_t)t * k + j];
        Vec8<T> r;
        load_nt(r, dx_perm + row * d + c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc.v[i] += r.v[i];
      }
    }
    acc.store(dx + (int64_t)t * d + c);
  }
}

template <class T>
hipError_t launch_unpermute_sum(const T* dx_perm, const int32_t* rmap, const float* partial, T* dx,
                                int T_, int k, int d, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
#define MOE_L(KC)                                                                                 \
  unpermute_sum_kernel<T, KC><<<(T_ + kCombineTokens - 1) / kCombineTokens, kCombineThreads, 0, st>>>(dx_perm, rmap, \
                                                                                          partial, dx, T_, k, d)
  MOE_DISPATCH_K(k, MOE_L);
#undef MOE_L
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_f32_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

#define MOE_INST(T)                                                                               \
  template hipError_t launch_combine<T>(const T*, const int32_t*, const float*, const T*, T*, int, \
                                        int, int, hipStream_t);                                    \
  template hipError_t launch_combine_bwd<T>(const T*, const T*, const int32_t*, const float*, T*,  \
                                            float*, int, int, int, hipStream_t);                   \
  template hipError_t launch_unpermute_sum<T>(const T*, const int32_t*, const float*, T*, int, int, \
                                              int, hipStream_t);
MOE_INST(float)
MOE_INST(bf16)

}  // namespace moe
