// router.hip -- router logits, per-token expert selection and the union
// dispatch tables, for gfx950.
//
// The router is colibrì's DeepSeek-V3-like sigmoid router with the
// aux-loss-free selection bias (noaux_tc) and routed_scaling_factor (colibrì
// README, "Implemented features"), with the adaptive expert top-p knob of the
// README's "Quick start".  The batch-union tables implement the same
// section's batch-union MoE: every unique expert of a batch, with the list of
// (token, slot) pairs routed to it.
//
// Every binary32 step of the selection is the same IEEE operation in the same
// order as the definition (no contraction), so indices and weights are
// reproducible bit for bit; the sigmoid is evaluated in binary64 and rounded
// once.
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace coli {

// ---------------------------------------------------------------------------
// Logits, small batches: one wave per expert row, the row read once and
// applied to every token; binary64 accumulation (each fp32 product is exact
// in binary64), rounded once to binary32.
// ---------------------------------------------------------------------------
template <int MAXT>
__global__ __launch_bounds__(256) void k_logits_gemv(const float *__restrict__ x,
                                                     const float *__restrict__ gw, int T, int E,
                                                     int H, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float4 *wr = reinterpret_cast<const float4 *>(gw + (size_t)e * H);
  double acc[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) acc[t] = 0.0;
  const int n4 = H / 4;
  for (int c = lane; c < n4; c += 64) {
    const float4 wv = wr[c];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < T) {
        const float4 xv = reinterpret_cast<const float4 *>(x + (size_t)t * H)[c];
        acc[t] = fma((double)xv.x, (double)wv.x, acc[t]);
        acc[t] = fma((double)xv.y, (double)wv.y, acc[t]);
        acc[t] = fma((double)xv.z, (double)wv.z, acc[t]);
        acc[t] = fma((double)xv.w, (double)wv.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < T) {
      const double s = wave_sum_f64(acc[t]);
      if (lane == 0) out[(size_t)t * E + e] = (float)s;
    }
  }
}

// ---------------------------------------------------------------------------
// Logits, larger batches: binary64 matrix cores.  A wave owns a 32-token x
// 32-expert tile as 2x2 v_mfma_f64_16x16x4 blocks.  Operand lane layout for
// 16x16x4: lane l supplies row (l % 16) and reduction index (l / 16); the
// reduction order inside a tile does not matter, so for a step of 16 inputs
// lane l loads the float4 at offset 4*(l/16) and feeds component j to the
// j-th MFMA.  Result: lane l holds rows 4*(l/16)+i, column l % 16.
// ---------------------------------------------------------------------------
typedef double d4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_logits_mfma(const float *__restrict__ x,
                                                     const float *__restrict__ gw, int T, int E,
                                                     int H, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 32;
  const int e0 = (blockIdx.x * 4 + wave) * 32;
  if (e0 >= E) return;
  const int r = lane & 15, g = lane >> 4;
  const float *xr[2], *wr[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    xr[a] = x + (size_t)min(t0 + 16 * a + r, T - 1) * H + 4 * g;
    wr[a] = gw + (size_t)min(e0 + 16 * a + r, E - 1) * H + 4 * g;
  }
  d4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = d4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < H; k0 += 16) {
    float4 xv[2], wv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      xv[a] = *reinterpret_cast<const float4 *>(xr[a] + k0);
      wv[a] = *reinterpret_cast<const float4 *>(wr[a] + k0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[a].x, (double)wv[b].x, acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[a].y, (double)wv[b].y, acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[a].z, (double)wv[b].z, acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[a].w, (double)wv[b].w, acc[a][b], 0, 0, 0);
      }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * a + 4 * g + i;
        const int e = e0 + 16 * b + r;
        if (t < T && e < E) out[(size_t)t * E + e] = (float)acc[a][b][i];
      }
}

hipError_t launch_logits(const float *x, const float *gate_w, int T, int E, int H, float *logits,
                         hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (T <= 4) {
    const dim3 grid((E + 3) / 4), block(256);
    hipLaunchKernelGGL(k_logits_gemv<4>, grid, block, 0, st, x, gate_w, T, E, H, logits);
  } else {
    const dim3 grid((E + 127) / 128, (T + 31) / 32), block(256);
    hipLaunchKernelGGL(k_logits_mfma, grid, block, 0, st, x, gate_w, T, E, H, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection: one wave per token.
// ---------------------------------------------------------------------------
struct Cand {
  float v;
  int i;  // index; -1 = no candidate
};

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
  if (a.i < 0) return false;
  if (b.i < 0) return true;
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Cand o;
    o.v = __shfl_xor(c.v, m, 64);
    o.i = __shfl_xor(c.i, m, 64);
    if (better(o, c)) c = o;
  }
  return c;
}

constexpr int kMaxE = 1024, kMaxK = 32;

__global__ __launch_bounds__(64) void k_route(RouterCfg cfg, const float *__restrict__ logits,
                                              const float *__restrict__ bias, int T,
                                              int32_t *__restrict__ idx, float *__restrict__ wout,
                                              int32_t *__restrict__ idx2, float *__restrict__ w2) {
  __shared__ float sig[kMaxE];
  __shared__ float cs[kMaxE];
  __shared__ int rank[kMaxK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int E = cfg.E, k = cfg.k, G = cfg.n_group, per = E / G;
  for (int e = lane; e < E; e += 64) {
    const float l = logits[(size_t)t * E + e];
    const float s = (float)(1.0 / (1.0 + exp(-(double)l)));
    sig[e] = s;
    cs[e] = s + (bias ? bias[e] : 0.f);
  }
  __syncthreads();

  // group scores: sum of the two best biased scores of each group
  Cand gc;
  gc.i = -1;
  gc.v = 0.f;
  if (lane < G) {
    int b1 = -1, b2 = -1;
    for (int e = lane * per; e < (lane + 1) * per; ++e) {
      if (b1 < 0 || cs[e] > cs[b1]) { b2 = b1; b1 = e; }
      else if (b2 < 0 || cs[e] > cs[b2]) { b2 = e; }
    }
    gc.v = per >= 2 ? cs[b1] + cs[b2] : cs[b1];
    gc.i = lane;
  }
  bool gkeep = false;
  for (int n = 0; n < cfg.topk_group; ++n) {
    Cand probe = gc;
    if (gkeep) probe.i = -1;
    const Cand best = wave_best(probe);
    if (lane == best.i) gkeep = true;
  }
  const uint64_t keepmask = __ballot(gkeep);

  // experts: lane owns e = lane + 64*m
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    Cand c;
    c.i = -1;
    c.v = 0.f;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      if (((keepmask >> (e / per)) & 1ull) == 0 || ((taken >> m) & 1u)) continue;
      Cand o{cs[e], e};
      if (better(o, c)) c = o;
    }
    const Cand best = wave_best(c);
    if (best.i >= 0 && (best.i & 63) == lane) taken |= 1u << (best.i >> 6);
    if (lane == 0) rank[j] = best.i;
  }
  __syncthreads();

  if (lane == 0) {
    // a slot with no candidate cannot occur for a validated configuration;
    // it is dropped rather than read out of range
    float S = 0.f;
    for (int j = 0; j < k; ++j)
      if (rank[j] >= 0) S += sig[rank[j]];
    float wv[kMaxK];
    int iv[kMaxK];
    for (int j = 0; j < k; ++j) {
      iv[j] = rank[j];
      if (rank[j] < 0) { wv[j] = 0.f; continue; }
      const float s = sig[rank[j]];
      if (cfg.norm) wv[j] = (S != 0.f) ? (s / S) * cfg.rsf : 0.f;
      else wv[j] = s * cfg.rsf;
    }
    if (cfg.top_p > 0.f && cfg.top_p < 1.f) {
      float pn[kMaxK];
      bool keep[kMaxK], seen[kMaxK];
      for (int j = 0; j < k; ++j) {
        pn[j] = (S != 0.f && iv[j] >= 0) ? sig[iv[j]] / S : 0.f;
        keep[j] = false;
        seen[j] = false;
      }
      float cum = 0.f;
      for (int n = 0; n < k; ++n) {
        int best = -1;
        for (int j = 0; j < k; ++j)
          if (!seen[j] && (best < 0 || pn[j] > pn[best])) best = j;
        seen[best] = true;
        keep[best] = true;
        cum += pn[best];
        if (cum >= cfg.top_p) break;
      }
      float Sk = 0.f;
      for (int j = 0; j < k; ++j)
        if (keep[j] && iv[j] >= 0) Sk += sig[iv[j]];
      for (int j = 0; j < k; ++j) {
        if (!keep[j] || iv[j] < 0) { iv[j] = -1; wv[j] = 0.f; continue; }
        if (cfg.renorm) wv[j] = (Sk != 0.f) ? (sig[iv[j]] / Sk) * cfg.rsf : 0.f;
      }
    }
    for (int j = 0; j < k; ++j) {
      idx[(size_t)t * k + j] = iv[j];
      wout[(size_t)t * k + j] = wv[j];
      if (idx2) idx2[(size_t)t * k + j] = iv[j];
      if (w2) w2[(size_t)t * k + j] = wv[j];
    }
  }
}

hipError_t launch_route(const RouterCfg &cfg, const float *logits, const float *bias, int T,
                        int32_t *idx, float *w, int32_t *idx_copy, float *w_copy, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route, dim3(T), dim3(64), 0, st, cfg, logits, bias, T, idx, w, idx_copy,
                     w_copy);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Union tables: one workgroup.  counts by LDS atomics (order-free), an
// exclusive scan, then a stable placement: entries are taken in chunks of
// 32*W consecutive (token, slot) pairs; each expert gets a W-word bitmask of
// its entries in the chunk, and an entry's position is the expert's running
// base + the popcount of its earlier bits.  Deterministic, and ordered by
// (expert, token, slot) even if a token repeats an expert.
// ---------------------------------------------------------------------------
constexpr int kDispThreads = 1024;
constexpr int kDispWords = 4096;  // E * W <= this

__global__ __launch_bounds__(kDispThreads) void k_dispatch(const int32_t *__restrict__ idx, int T,
                                                           int k, int E, int W,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ uniq,
                                                           int32_t *__restrict__ n_uniq) {
  __shared__ int cnt[kMaxE];
  __shared__ int scan_a[kMaxE];
  __shared__ int scan_b[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ uint32_t mask[kDispWords];
  __shared__ int pref[kDispWords];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)T * k;

  for (int e = tid; e < E; e += kDispThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += kDispThreads) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // inclusive scans (Hillis-Steele) of counts and of nonzero flags
  for (int e = tid; e < E; e += kDispThreads) {
    scan_a[e] = cnt[e];
    scan_b[e] = cnt[e] > 0 ? 1 : 0;
  }
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {
    int va[(kMaxE + kDispThreads - 1) / kDispThreads], vb[(kMaxE + kDispThreads - 1) / kDispThreads];
    int q = 0;
    for (int e = tid; e < E; e += kDispThreads, ++q) {
      va[q] = scan_a[e] + (e >= d ? scan_a[e - d] : 0);
      vb[q] = scan_b[e] + (e >= d ? scan_b[e - d] : 0);
    }
    __syncthreads();
    q = 0;
    for (int e = tid; e < E; e += kDispThreads, ++q) {
      scan_a[e] = va[q];
      scan_b[e] = vb[q];
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += kDispThreads) {
    const int excl = scan_a[e] - cnt[e];
    counts[e] = cnt[e];
    offs[e] = excl;
    base[e] = excl;
    if (cnt[e] > 0) uniq[scan_b[e] - 1] = e;
  }
  if (tid == 0) {
    offs[E] = scan_a[E - 1];
    n_uniq[0] = scan_b[E - 1];
  }
  __syncthreads();

  const int chunk = 32 * W;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    for (int m = tid; m < E * W; m += kDispThreads) mask[m] = 0u;
    __syncthreads();
    for (int i = tid; i < chunk && c0 + i < n; i += kDispThreads) {
      const int e = idx[c0 + i];
      if (e >= 0 && e < E) atomicOr(&mask[e * W + (i >> 5)], 1u << (i & 31));
    }
    __syncthreads();
    for (int e = tid; e < E; e += kDispThreads) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        pref[e * W + w] = run;
        run += __popc(mask[e * W + w]);
      }
    }
    __syncthreads();
    for (int i = tid; i < chunk && c0 + i < n; i += kDispThreads) {
      const int e = idx[c0 + i];
      if (e >= 0 && e < E) {
        const int w = i >> 5;
        const uint32_t below = mask[e * W + w] & ((1u << (i & 31)) - 1u);
        perm[base[e] + pref[e * W + w] + __popc(below)] = (int32_t)(c0 + i);
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kDispThreads)
      base[e] += pref[e * W + W - 1] + __popc(mask[e * W + W - 1]);
    __syncthreads();
  }
}

hipError_t launch_dispatch(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offs,
                           int32_t *perm, int32_t *uniq, int32_t *n_uniq, hipStream_t st) {
  int W = kDispWords / E;
  if (W > 32) W = 32;
  if (W < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kDispThreads), 0, st, idx, T, k, E, W, counts, offs,
                     perm, uniq, n_uniq);
  return hipGetLastError();
}

}  // namespace coli
