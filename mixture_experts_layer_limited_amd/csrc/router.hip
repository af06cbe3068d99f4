// Router: score function, group-limited top-k, gates, per-expert statistics
// and the router backward ("System Modules: Router"; Figure 2 of the
// figures page: linear projection, score function, top-k, load balancing).
//
// One wave64 handles one token at a time; lane l holds experts l, l+64, ...
// Selection is an iterated wave-wide argmax on the key (ties -> lower id),
// done with cross-lane shuffles, so equal fp32 inputs give the same choice as
// any implementation of the same ordering rule.
#include <limits.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kNI = kMaxExperts / kWave;   // values per lane (E <= 256)
constexpr int kRouterWaves = 4;

// Key order: larger first, equal keys by lower id, and a NaN key below every
// number (-inf included).  Keys are compared as integers that keep the order
// of the floats (negative ones with their magnitude bits flipped, -0 as +0)
// with NaN mapped to INT_MIN.  The search starts from (INT_MIN, INT_MAX),
// which every candidate beats, so a selection always returns a candidate's
// id, whatever values the logits hold.
__device__ __forceinline__ int order_key(float f) {
  if (f != f) return INT_MIN;
  const int b = __float_as_int(f == 0.0f ? 0.0f : f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ bool better(int ka, int ia, int kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}
constexpr int kNoId = 0x7fffffff;

// wave-wide argmax of (key desc, id asc); every lane returns the winner
__device__ __forceinline__ void wave_argmax(int& k, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int ok = __shfl_xor(k, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (better(ok, oi, k, i)) { k = ok; i = oi; }
  }
}

// Centered sums without cancellation.  The router gradients take the form
// w_j (a_j - sum_i w_i a_i) with weights summing to one; when one weight is
// close to 1 the bracket of that term is the difference of two nearly equal
// numbers in fp32.  Written as w_j sum_i w_i (a_j - a_i) (over the k choices,
// pairwise) or, over all E experts, with the largest weight's term split off
// (its 1 - w from the sum of the other weights), every term keeps its
// relative precision.

// k choices, choice j in lane j % 64, slot j / 64: out_j = sum_i w_i (a_j - a_i)
__device__ __forceinline__ void pairwise_centered(const float* w, const float* a, int k, float* out) {
#pragma unroll
  for (int s = 0; s < kNI; ++s) out[s] = 0.0f;
  for (int i = 0; i < k; ++i) {
    const int src = i & 63, slot = i >> 6;
    float wi = 0.0f, ai = 0.0f;
#pragma unroll
    for (int s = 0; s < kNI; ++s)
      if (s == slot) {
        wi = __shfl(w[s], src, kWave);
        ai = __shfl(a[s], src, kWave);
      }
#pragma unroll
    for (int s = 0; s < kNI; ++s) out[s] += wi * (a[s] - ai);
  }
}

// sigmoid evaluated in double and rounded once to fp32
__device__ __forceinline__ float sigmoid_score(float l) {
  return (float)(1.0 / (1.0 + exp(-(double)l)));
}

}  // namespace

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ bias,
                                                          RouterParams p, int32_t* __restrict__ idx_out,
                                                          float* __restrict__ gates_out,
                                                          int* __restrict__ cnt_part,
                                                          float* __restrict__ colsum_part) {
  __shared__ int hist[kMaxExperts];
  __shared__ float csum[kRouterWaves][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < kMaxExperts; e += blockDim.x) hist[e] = 0;
  __syncthreads();

  const int E = p.E, k = p.k;
  const bool softmax = p.score == 0;
  const bool need_p = softmax && (p.aux_coeff != 0.0f || !p.renorm);
  const int per = E / p.n_group;
  float cs[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) cs[i] = 0.0f;

  const int tpw = kRouterTokensPerBlock / kRouterWaves;
  const int t_begin = blockIdx.x * kRouterTokensPerBlock + wave * tpw;
  for (int tt = 0; tt < tpw; ++tt) {
    const int t = t_begin + tt;
    if (t >= p.T) break;                       // wave-uniform
    float v[kNI], key[kNI], pr[kNI];
    bool elig[kNI], taken[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      int e = lane + 64 * i;
      v[i] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
      elig[i] = e < E;
      taken[i] = false;
      pr[i] = 0.0f;
    }
    if (softmax) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kNI; ++i) mx = fmaxf(mx, v[i]);
      mx = wave_max(mx);
      if (need_p) {
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          pr[i] = elig[i] ? expf(v[i] - mx) : 0.0f;
          z += pr[i];
        }
        z = wave_sum(z);
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          pr[i] = pr[i] / z;
          cs[i] += pr[i];
        }
      }
#pragma unroll
      for (int i = 0; i < kNI; ++i) key[i] = v[i];
    } else {
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        int e = lane + 64 * i;
        float s = elig[i] ? sigmoid_score(v[i]) : 0.0f;
        pr[i] = s;                               // the unbiased score
        key[i] = elig[i] ? (bias ? s + bias[e] : s) : -INFINITY;
      }
    }

    // group-limited routing: score groups by the sum of their two best keys
    // (force-balanced routing assigns experts without looking at the keys)
    if (p.n_group > 1 && !p.balanced) {
      int gs[kNI];
#pragma unroll
      for (int i = 0; i < kNI; ++i) gs[i] = INT_MIN;
      for (int g = 0; g < p.n_group; ++g) {
        float t1 = -INFINITY, t2 = -INFINITY;
        bool has_nan = false;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          int e = lane + 64 * i;
          if (elig[i] && e / per == g) {
            float kv = key[i];
            has_nan |= kv != kv;
            if (kv > t1) { t2 = t1; t1 = kv; } else if (kv > t2) { t2 = kv; }
          }
        }
        // a group holding a NaN key scores NaN (it ranks below every group
        // with a numeric score)
        const bool group_nan = __any(has_nan);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          float o1 = __shfl_xor(t1, o, kWave), o2 = __shfl_xor(t2, o, kWave);
          float hi = fmaxf(t1, o1), lo = fminf(t1, o1);
          t2 = fmaxf(lo, fmaxf(t2, o2));
          t1 = hi;
        }
        const float score = group_nan ? __builtin_nanf("") : per >= 2 ? t1 + t2 : t1;
        const int okey = order_key(score);
#pragma unroll
        for (int i = 0; i < kNI; ++i)
          if (lane + 64 * i == g) gs[i] = okey;
      }
      // keep topk_group groups (score desc, group id asc)
      uint64_t gm[kNI] = {0, 0, 0, 0};
      bool gtaken[kNI] = {false, false, false, false};
      for (int r = 0; r < p.topk_group; ++r) {
        int bk = INT_MIN;
        int bi = kNoId;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          int g = lane + 64 * i;
          if (g < p.n_group && !gtaken[i] && better(gs[i], g, bk, bi)) { bk = gs[i]; bi = g; }
        }
        wave_argmax(bk, bi);
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          if (lane + 64 * i == bi) gtaken[i] = true;
          if ((bi >> 6) == i) gm[i] |= 1ull << (bi & 63);
        }
      }
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        int e = lane + 64 * i;
        if (elig[i]) {
          int g = e / per;
          uint64_t w = gm[0];
#pragma unroll
          for (int q = 1; q < kNI; ++q)
            if ((g >> 6) == q) w = gm[q];
          elig[i] = (w >> (g & 63)) & 1ull;
        }
      }
    }

    int okey[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) okey[i] = order_key(key[i]);
    // top-k: k rounds of a wave argmax; lane j%64 keeps choice j.  Force-
    // balanced routing: choice j is expert (t k + j) mod E (uniform over the wave)
    int my_id[kNI];
    float my_val[kNI], my_p[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) { my_id[i] = 0; my_val[i] = 0.0f; my_p[i] = 0.0f; }
    for (int j = 0; j < k; ++j) {
      int bi;
      if (p.balanced) {
        bi = (int)(((int64_t)t * k + j) % E);
      } else {
        int bk = INT_MIN;
        bi = kNoId;
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          int e = lane + 64 * i;
          if (elig[i] && !taken[i] && better(okey[i], e, bk, bi)) { bk = okey[i]; bi = e; }
        }
        wave_argmax(bk, bi);
      }
      // the owner lane publishes the winner's logit (softmax) / score (sigmoid) and p
      float ov = 0.0f, op = 0.0f;
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        if (lane + 64 * i == bi) {
          taken[i] = true;
          ov = softmax ? v[i] : pr[i];
          op = pr[i];
        }
      }
      float wv = __shfl(ov, bi & 63, kWave);
      float wp = __shfl(op, bi & 63, kWave);
#pragma unroll
      for (int i = 0; i < kNI; ++i)
        if (lane + 64 * i == j) { my_id[i] = bi; my_val[i] = wv; my_p[i] = wp; }
    }

    // gates
    float g[kNI];
    if (softmax && p.renorm) {
      float l0 = __shfl(my_val[0], 0, kWave);
      float z = 0.0f;
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        g[i] = (lane + 64 * i < k) ? expf(my_val[i] - l0) : 0.0f;
        z += g[i];
      }
      z = wave_sum(z);
#pragma unroll
      for (int i = 0; i < kNI; ++i) g[i] = g[i] / z * p.scale;
    } else if (softmax) {
#pragma unroll
      for (int i = 0; i < kNI; ++i) g[i] = my_p[i] * p.scale;
    } else {
      float S = 0.0f;
#pragma unroll
      for (int i = 0; i < kNI; ++i) S += (lane + 64 * i < k) ? my_val[i] : 0.0f;
      S = wave_sum(S);
#pragma unroll
      for (int i = 0; i < kNI; ++i) g[i] = p.renorm ? p.scale * my_val[i] / S : p.scale * my_val[i];
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      int j = lane + 64 * i;
      if (j < k) {
        idx_out[(int64_t)t * k + j] = my_id[i];
        gates_out[(int64_t)t * k + j] = g[i];
        atomicAdd(&hist[my_id[i]], 1);          // integer: order-independent
      }
    }
  }

#pragma unroll
  for (int i = 0; i < kNI; ++i) csum[wave][lane + 64 * i] = cs[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    cnt_part[(int64_t)blockIdx.x * E + e] = hist[e];
    if (colsum_part)
      colsum_part[(int64_t)blockIdx.x * E + e] = ((csum[0][e] + csum[1][e]) + csum[2][e]) + csum[3][e];
  }
}

hipError_t launch_router_topk(const float* logits, const float* bias, const RouterParams& p,
                              int32_t* idx, float* gates, int* cnt_part, float* colsum_part,
                              hipStream_t st) {
  int nblk = (p.T + kRouterTokensPerBlock - 1) / kRouterTokensPerBlock;
  if (nblk == 0) return hipSuccess;
  router_topk_kernel<<<nblk, 256, 0, st>>>(logits, bias, p, idx, gates, cnt_part, colsum_part);
  return hipGetLastError();
}

// counts[e] = sum over the router blocks' partial counts; with probability
// sums, colsum_part[e] (the first block's row) becomes their total.  One
// workgroup per expert: thread i sums blocks i, i + 256, ... and a fixed-shape
// tree combines the 256 partial sums, so the result does not depend on
// scheduling.
__global__ __launch_bounds__(256) void router_finalize_kernel(const int* __restrict__ cnt_part,
                                                              float* __restrict__ colsum_part, int nblk,
                                                              int E, int32_t* __restrict__ counts) {
  __shared__ int sc[256];
  __shared__ float sf[256];
  const int e = blockIdx.x, t = threadIdx.x;
  int c = 0;
  float f = 0.0f;
  for (int b = t; b < nblk; b += 256) {
    c += cnt_part[(int64_t)b * E + e];
    if (colsum_part) f += colsum_part[(int64_t)b * E + e];
  }
  sc[t] = c;
  sf[t] = f;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      sc[t] += sc[t + w];
      sf[t] += sf[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    counts[e] = sc[0];
    // only this workgroup reads column e; with no blocks there is no row to hold it
    if (colsum_part && nblk > 0) colsum_part[e] = sf[0];
  }
}

hipError_t launch_router_finalize(const int* cnt_part, float* colsum_part, int nblk, const RouterParams& p,
                                  int32_t* counts, hipStream_t st) {
  if (p.E <= 0) return hipSuccess;
  router_finalize_kernel<<<p.E, 256, 0, st>>>(cnt_part, colsum_part, nblk, p.E, counts);
  return hipGetLastError();
}

// aux = coeff * E * sum_e (c_e / (T k)) (colsum_e / T), summed in expert order
__global__ __launch_bounds__(256) void router_aux_kernel(const int32_t* __restrict__ counts,
                                                         const float* __restrict__ colsum, RouterParams p,
                                                         float* __restrict__ aux) {
  __shared__ double term[kMaxExperts];
  const int e = threadIdx.x;
  if (e < p.E)
    term[e] = (p.T > 0) ? ((double)counts[e] / ((double)p.T * p.k)) * ((double)colsum[e] / p.T) : 0.0;
  __syncthreads();
  if (e == 0) {
    double s = 0.0;
    for (int q = 0; q < p.E; ++q) s += term[q];
    aux[0] = (float)((double)p.aux_coeff * p.E * s);
  }
}

hipError_t launch_router_aux(const int32_t* counts, const float* colsum, const RouterParams& p, float* aux,
                             hipStream_t st) {
  router_aux_kernel<<<1, 256, 0, st>>>(counts, colsum, p, aux);
  return hipGetLastError();
}

// Selection-bias step toward balance: bias[e] += rate * sign(T k - E c_e).
// The sign is integer arithmetic; rate * sign is exact, so the update is one
// fp32 add whatever the compiler contracts.
__global__ __launch_bounds__(256) void router_bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                                 int64_t Tk, float rate, float* __restrict__ bias) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int64_t diff = Tk - (int64_t)E * counts[e];
  const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  bias[e] = bias[e] + rate * sgn;
}

hipError_t launch_router_bias_update(const int32_t* counts, int E, int64_t Tk, float rate, float* bias,
                                     hipStream_t st) {
  router_bias_update_kernel<<<1, 256, 0, st>>>(counts, E, Tk, rate, bias);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router backward: d_logits per token (routing fixed), plus a storage-typed
// copy [T, Ep] (zero padded) feeding the two router GEMMs.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ gates,
                                                         const float* __restrict__ d_gates,
                                                         const int32_t* __restrict__ counts,
                                                         RouterParams p, float d_aux,
                                                         float* __restrict__ d_logits,
                                                         T* __restrict__ dl_store, int Ep) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouterWaves + wave;
  if (t >= p.T) return;
  const int E = p.E, k = p.k;
  const bool softmax = p.score == 0;
  float v[kNI], pr[kNI], dl[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
    dl[i] = 0.0f;
    pr[i] = 0.0f;
  }
  const bool need_p = softmax && (!p.renorm || p.aux_coeff != 0.0f);
  // full softmax p; dom = the lowest expert id of largest logit, rest = 1 - p_dom
  // summed from the other experts' terms
  int dom = 0;
  float rest = 0.0f;
  if (need_p) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kNI; ++i) mx = fmaxf(mx, v[i]);
    mx = wave_max(mx);
    int cand = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kNI; ++i)
      if (lane + 64 * i < E && v[i] == mx && lane + 64 * i < cand) cand = lane + 64 * i;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cand = min(cand, __shfl_xor(cand, o, kWave));
    dom = cand;
    float z = 0.0f, zo = 0.0f;
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      pr[i] = (lane + 64 * i < E) ? expf(v[i] - mx) : 0.0f;
      z += pr[i];
      if (lane + 64 * i != dom) zo += pr[i];
    }
    z = wave_sum(z);
    zo = wave_sum(zo);
#pragma unroll
    for (int i = 0; i < kNI; ++i) pr[i] /= z;
    rest = zo / z;
  }
  // over all E experts: out_e = p_e (a_e - sum_i p_i a_i), the dominant
  // expert's term as p_dom (a_dom rest - sum_{i != dom} p_i a_i)
  auto centered_all = [&](const float* a, float* out) {
    float io = 0.0f, pa_dom = 0.0f;
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      if (lane + 64 * i != dom) io += pr[i] * a[i];
      else pa_dom = pr[i] * a[i];
    }
    io = wave_sum(io);
    const float inner = io + wave_sum(pa_dom);
#pragma unroll
    for (int i = 0; i < kNI; ++i)
      out[i] = lane + 64 * i == dom ? pr[i] * (a[i] * rest - io) : pr[i] * (a[i] - inner);
  };
  // choice j lives in lane j%64, slot j/64
  int sid[kNI];
  float sg[kNI], sdg[kNI], ss[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    int j = lane + 64 * i;
    bool ok = j < k;
    sid[i] = ok ? idx[(int64_t)t * k + j] : 0;
    sg[i] = ok ? gates[(int64_t)t * k + j] : 0.0f;
    sdg[i] = ok ? d_gates[(int64_t)t * k + j] : 0.0f;
    ss[i] = 0.0f;
  }
  float dsel[kNI];
  if (softmax && p.renorm) {
    // g_j = scale q_j, q the softmax over the chosen logits:
    // dl_j = scale q_j sum_i q_i (dg_j - dg_i)
    float q[kNI], cen[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) q[i] = sg[i] / p.scale;
    pairwise_centered(q, sdg, k, cen);
#pragma unroll
    for (int i = 0; i < kNI; ++i) dsel[i] = p.scale * q[i] * cen[i];
  } else if (!softmax) {
    // recompute the selected sigmoid scores from the logits
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      int j = lane + 64 * i;
      ss[i] = 0.0f;
      if (j < k) ss[i] = sigmoid_score(logits[(int64_t)t * E + sid[i]]);
    }
    // renormalised: g_j = scale s_j / S, dL/ds_j = (scale / S) sum_i (s_i / S) (dg_j - dg_i)
    float S = 0.0f;
#pragma unroll
    for (int i = 0; i < kNI; ++i) S += ss[i];
    S = wave_sum(S);
    float w[kNI], cen[kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) w[i] = ss[i] / S;
    if (p.renorm) pairwise_centered(w, sdg, k, cen);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      float ds = p.renorm ? (p.scale / S) * cen[i] : p.scale * sdg[i];
      dsel[i] = ds * ss[i] * (1.0f - ss[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kNI; ++i) dsel[i] = 0.0f;
  }
  // scatter the per-choice values to their experts' lanes
  float dgf[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) dgf[i] = 0.0f;
  for (int j = 0; j < k; ++j) {
    int src_lane = j & 63, slot = j >> 6;
    int e = 0;
    float val = 0.0f, dgv = 0.0f;
#pragma unroll
    for (int i = 0; i < kNI; ++i)
      if (i == slot) {
        e = __shfl(sid[i], src_lane, kWave);
        val = __shfl(dsel[i], src_lane, kWave);
        dgv = __shfl(sdg[i], src_lane, kWave);
      }
#pragma unroll
    for (int i = 0; i < kNI; ++i)
      if (lane + 64 * i == e) { dl[i] += val; dgf[i] += dgv * p.scale; }
  }
  if (softmax && !p.renorm) centered_all(dgf, dl);
  if (softmax && p.aux_coeff != 0.0f) {
    float a[kNI];
    const float norm = p.aux_coeff * (float)E / ((float)p.T * (float)k * (float)p.T);
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      int e = lane + 64 * i;
      a[i] = e < E ? norm * (float)counts[e] : 0.0f;
    }
    float ca[kNI];
    centered_all(a, ca);
#pragma unroll
    for (int i = 0; i < kNI; ++i) dl[i] += d_aux * ca[i];
  }
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    int e = lane + 64 * i;
    if (e < E) d_logits[(int64_t)t * E + e] = dl[i];
    if (dl_store && e < Ep) dl_store[(int64_t)t * Ep + e] = from_f32<T>(e < E ? dl[i] : 0.0f);
  }
}

template <class T>
hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gates,
                             const float* d_gates, const int32_t* counts, const RouterParams& p,
                             float d_aux, float* d_logits, T* dl_store, int Ep, hipStream_t st) {
  int nblk = (p.T + kRouterWaves - 1) / kRouterWaves;
  if (nblk == 0) return hipSuccess;
  router_bwd_kernel<T><<<nblk, 256, 0, st>>>(logits, idx, gates, d_gates, counts, p, d_aux,
                                             d_logits, dl_store, Ep);
  return hipGetLastError();
}

template hipError_t launch_router_bwd<float>(const float*, const int32_t*, const float*, const float*,
                                             const int32_t*, const RouterParams&, float, float*,
                                             float*, int, hipStream_t);
template hipError_t launch_router_bwd<bf16>(const float*, const int32_t*, const float*, const float*,
                                            const int32_t*, const RouterParams&, float, float*,
                                            bf16*, int, hipStream_t);

}  // namespace moe
