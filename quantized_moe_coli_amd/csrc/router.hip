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
#include "actq.hpp"
#include "kernels.hpp"
#include "select.hpp"

#pragma clang fp contract(off)

namespace coli {

// ---------------------------------------------------------------------------
// Front of the layer for small batches (T <= 4), one launch:
//   blocks [0, nlog): router logits of expert row b.  The 4 waves split the
//     row in quarters; binary64 accumulation (each fp32 product is exact in
//     binary64), partials added in a fixed order, rounded once to binary32.
//   blocks [nlog, nlog + naq): Q8_0 quantisation of the activations, one
//     thread per block of 32 (codes in the ordering of container BITS).
// ---------------------------------------------------------------------------
template <int BITS, int MAXT>
__global__ __launch_bounds__(256) void k_front_small(const float *__restrict__ x,
                                                     const float *__restrict__ gw,
                                                     const float *__restrict__ loff, int T, int E,
                                                     int H, float *__restrict__ out, int nlog,
                                                     int8_t *__restrict__ xq,
                                                     float *__restrict__ xd,
                                                     double *__restrict__ xd64) {
  __shared__ double red[4][MAXT];
  const int b = blockIdx.x;
  if (b >= nlog) {
    const int64_t nb = H / 32;
    const int64_t i = (int64_t)(b - nlog) * 256 + threadIdx.x;
    if (i >= (int64_t)T * nb) return;
    const int64_t t = i / nb, blk = i % nb;
    act_quant_block<BITS>(x + t * H + blk * 32, xq + t * H + blk * 32, xd + i);
    if (xd64) xd64[t * xd64_ld(H) + blk] = (double)xd[i];
    return;
  }
  const int e = b;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = H / 16;  // float4 per quarter row (<= 128 for H <= 8192)
  constexpr int kPer = 2;  // float4 per lane per step
  const float4 *wr = reinterpret_cast<const float4 *>(gw + (size_t)e * H) + wave * q4;
  double acc[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) acc[t] = 0.0;
  for (int c0 = 0; c0 < q4; c0 += 64 * kPer) {
    float4 wv[kPer];
    bool ok[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = c0 + lane + 64 * i;
      ok[i] = c < q4;
      wv[i] = wr[min(c, q4 - 1)];
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < T) {
        const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * H) + wave * q4;
        float4 xv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) xv[i] = xr[min(c0 + lane + 64 * i, q4 - 1)];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          if (!ok[i]) continue;
          acc[t] = fma((double)xv[i].x, (double)wv[i].x, acc[t]);
          acc[t] = fma((double)xv[i].y, (double)wv[i].y, acc[t]);
          acc[t] = fma((double)xv[i].z, (double)wv[i].z, acc[t]);
          acc[t] = fma((double)xv[i].w, (double)wv[i].w, acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const double s = wave_sum_f64(acc[t]);
    if (lane == 0) red[wave][t] = s;
  }
  __syncthreads();
  if (threadIdx.x < MAXT && (int)threadIdx.x < T) {
    const int t = threadIdx.x;
    const double s = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    float l = (float)s;
    if (loff) l += loff[e];
    out[(size_t)t * E + e] = l;
  }
}

// ---------------------------------------------------------------------------
// Logits, larger batches: binary64 matrix cores.  A workgroup owns a
// 16-token x 16-expert tile; its 8 waves take the reduction steps of 16
// inputs round-robin, each into its own v_mfma_f64_16x16x4 accumulator, and
// the 8 partial tiles are added in wave order through LDS and rounded once.
// Operand lane layout for 16x16x4: lane l supplies row (l % 16) and
// reduction index (l / 16); for a step of 16 inputs lane l loads the float4
// at offset 4*(l/16) and feeds component j to the j-th MFMA.  Result
// (binary64 layout): register i of lane l holds row (l / 16) + 4*i, column
// l % 16.  Small tiles keep every batch size spread over many workgroups
// (16 experts x 16 tokens each).
// ---------------------------------------------------------------------------
typedef double d4 __attribute__((ext_vector_type(4)));
constexpr int kLogWaves = 8;

__global__ __launch_bounds__(64 * kLogWaves) void k_logits_mfma(const float *__restrict__ x,
                                                                const float *__restrict__ gw,
                                                                const float *__restrict__ loff,
                                                                int T, int E, int H,
                                                                float *__restrict__ out) {
  __shared__ double part[kLogWaves][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 16;
  const int e0 = blockIdx.x * 16;
  const int r = lane & 15, g = lane >> 4;
  const float *xr = x + (size_t)min(t0 + r, T - 1) * H + 4 * g;
  const float *wr = gw + (size_t)min(e0 + r, E - 1) * H + 4 * g;
  d4 acc = {0.0, 0.0, 0.0, 0.0};
  constexpr int kBatch = 4;  // steps whose loads are issued together
  for (int k0 = 16 * wave; k0 < H; k0 += 16 * kLogWaves * kBatch) {
    float4 xv[kBatch], wv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int k = min(k0 + 16 * kLogWaves * j, H - 16);  // clamped: valid, unused
      xv[j] = *reinterpret_cast<const float4 *>(xr + k);
      wv[j] = *reinterpret_cast<const float4 *>(wr + k);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + 16 * kLogWaves * j < H) {
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[j].x, (double)wv[j].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[j].y, (double)wv[j].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[j].z, (double)wv[j].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[j].w, (double)wv[j].w, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][i][lane] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int i = threadIdx.x >> 6;
    double sum = part[0][i][lane];
#pragma unroll
    for (int w = 1; w < kLogWaves; ++w) sum += part[w][i][lane];
    const int t = t0 + g + 4 * i, e = e0 + r;
    if (t < T && e < E) {
      float l = (float)sum;
      if (loff) l += loff[e];
      out[(size_t)t * E + e] = l;
    }
  }
}

template <int BITS>
static void front_small(const float *x, const float *gate_w, const float *loff, int T, int E,
                        int H, float *logits, int8_t *xq, float *xd, double *xd64, hipStream_t st,
                        KEvents ev) {
  const int nlog = gate_w ? E : 0;
  const int naq = xq ? (int)(((int64_t)T * (H / 32) + 255) / 256) : 0;
  COLI_LAUNCH(ev, (k_front_small<BITS, 4>), dim3(nlog + naq), dim3(256), 0, st, x, gate_w, loff, T,
              E, H, logits, nlog, xq, xd, xd64);
}

hipError_t launch_front(int bits, const float *x, const float *gate_w, const float *loff, int T,
                        int E, int H, float *logits, int8_t *xq, float *xd, hipStream_t st,
                        KEvents ev, double *xd64) {
  if (T == 0 || (!gate_w && !xq)) return hipSuccess;
  if (T <= 4) {
    switch (bits) {
      case 8: front_small<8>(x, gate_w, loff, T, E, H, logits, xq, xd, xd64, st, ev); break;
      case 4: front_small<4>(x, gate_w, loff, T, E, H, logits, xq, xd, xd64, st, ev); break;
      case 2: front_small<2>(x, gate_w, loff, T, E, H, logits, xq, xd, xd64, st, ev); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // the kernel events time the logits kernel, or the activation
  // quantisation when the logits are supplied
  if (gate_w) {
    const dim3 grid((E + 15) / 16, (T + 15) / 16), block(64 * kLogWaves);
    COLI_LAUNCH(ev, k_logits_mfma, grid, block, 0, st, x, gate_w, loff, T, E, H, logits);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (xq) return launch_act_quant(bits, x, T, H, xq, xd, st, gate_w ? KEvents{} : ev, xd64);
  return hipSuccess;
}

hipError_t launch_logits(const float *x, const float *gate_w, int T, int E, int H, float *logits,
                         hipStream_t st) {
  return launch_front(8, x, gate_w, nullptr, T, E, H, logits, nullptr, nullptr, st);
}

// ---------------------------------------------------------------------------
// Selection: one wave per token (select.hpp), four tokens per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_route(RouterCfg cfg, const float *__restrict__ logits,
                                               const float *__restrict__ bias, int T,
                                               int32_t *__restrict__ idx, float *__restrict__ wout,
                                               int32_t *__restrict__ idx2, float *__restrict__ w2) {
  __shared__ SelScratch sc[4];
  __shared__ int32_t li[4][kSelMaxK];
  __shared__ float lw[4][kSelMaxK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int k = cfg.k;
  select_token(cfg, logits + (size_t)t * cfg.E, bias, sc[wave], li[wave], lw[wave]);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (lane < k) {
    idx[(size_t)t * k + lane] = li[wave][lane];
    wout[(size_t)t * k + lane] = lw[wave][lane];
    if (idx2) idx2[(size_t)t * k + lane] = li[wave][lane];
    if (w2) w2[(size_t)t * k + lane] = lw[wave][lane];
  }
}

hipError_t launch_route(const RouterCfg &cfg, const float *logits, const float *bias, int T,
                        int32_t *idx, float *w, int32_t *idx_copy, float *w_copy, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(256), 0, st, cfg, logits, bias, T, idx, w,
                     idx_copy, w_copy);
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
  __shared__ int cnt[kSelMaxE];
  __shared__ int scan_a[kSelMaxE];
  __shared__ int scan_b[kSelMaxE];
  __shared__ int base[kSelMaxE];
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
    int va[(kSelMaxE + kDispThreads - 1) / kDispThreads], vb[(kSelMaxE + kDispThreads - 1) / kDispThreads];
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
