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
#include <algorithm>

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

// One workgroup per token: the scores in LDS (one expert per thread), then
// the workgroup-parallel selection (select_fast: the same order and binary32
// operations as select_token, so the same experts and weights), for layers
// whose expert count and groups it covers.  Shorter per token than one wave
// running the k rounds of arg-max.
constexpr int kRouteWgThreads = 256;
__global__ __launch_bounds__(kRouteWgThreads) void k_route_wg(RouterCfg cfg,
                                                              const float *__restrict__ logits,
                                                              const float *__restrict__ bias,
                                                              int32_t *__restrict__ idx,
                                                              float *__restrict__ wout,
                                                              int32_t *__restrict__ idx2,
                                                              float *__restrict__ w2) {
  __shared__ SelInput in;
  __shared__ SelFastScratch sc;
  __shared__ int32_t sidx[kSelMaxK];
  __shared__ float sw[kSelMaxK];
  const int t = blockIdx.x, e = threadIdx.x, k = cfg.k;
  if (e < cfg.E) {
    const float l = logits[(size_t)t * cfg.E + e];
    const float bv = bias ? bias[e] : 0.f;
    const float sg = sigmoid_f64(l);
    in.sg[e] = sg;
    in.c[e] = sg + bv;
  }
  __syncthreads();
  select_fast<kRouteWgThreads>(cfg, in, sc, sidx, sw);
  if (e < k) {
    const int32_t i = (unsigned)sidx[e] < (unsigned)cfg.E ? sidx[e] : -1;
    idx[(size_t)t * k + e] = i;
    wout[(size_t)t * k + e] = sw[e];
    if (idx2) idx2[(size_t)t * k + e] = i;
    if (w2) w2[(size_t)t * k + e] = sw[e];
  }
}

hipError_t launch_route(const RouterCfg &cfg, const float *logits, const float *bias, int T,
                        int32_t *idx, float *w, int32_t *idx_copy, float *w_copy, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (select_fast_ok(cfg.E, cfg.n_group, cfg.topk_group, cfg.k, kRouteWgThreads))
    hipLaunchKernelGGL(k_route_wg, dim3(T), dim3(kRouteWgThreads), 0, st, cfg, logits, bias, idx, w,
                       idx_copy, w_copy);
  else
    hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(256), 0, st, cfg, logits, bias, T, idx, w,
                       idx_copy, w_copy);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Union tables: one workgroup of 1024 threads.  Counts by LDS atomics
// (order-free); one scan of (count, nonzero) pairs gives offs, uniq and
// n_uniq.  Placement is a stable counting sort in rounds of up to 64 * C
// pairs: wave w takes chunks w, w + 16, ... of 64 consecutive pairs; in each
// chunk a pair's rank among the chunk's pairs of its expert comes from the
// lanes holding the same expert id (one ballot per bit of the id), and the
// expert's first lane writes the chunk's count of it into an LDS matrix
// [C][E].  A scan of each expert's column over the chunks then gives every
// chunk's first position for the expert, so pair i of expert e goes to
// base[e] + column prefix + rank.  Ordered by (expert, token, slot) even if
// a token repeats an expert; deterministic.
//
// With mgofs, the matrix-core item tables too, one per token-group size:
// mgofs[u] = first 64-token group of union slot u (slots 0 .. n_uniq-1 are
// the unique routed experts, slot n_uniq the shared expert), mgofs[n_uniq +
// 1] the total; the same for 32-token groups from mgofs + E + 2.  Then, from
// mgofs + 2 (E + 2), the slot of each 64-token group, and mfma_gmax entries
// on, of each 32-token group.  Both group counts are scanned at once as the
// halves of one 64-bit word.
// ---------------------------------------------------------------------------
constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / 64;
constexpr int kDispCells = 16384;    // chunk x expert count matrix in LDS (64 KB)
constexpr int kDispMaxChunks = 256;  // chunks per round (16 per wave)

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, d, 64);
  const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

// C chunks per round (a multiple of 16 and of P), P threads per expert
// column in the column scan (a power of two dividing 64).
__global__ __launch_bounds__(kDispThreads) void k_dispatch(const int32_t *__restrict__ idx, int T,
                                                           int k, int E, int C, int P,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ uniq,
                                                           int32_t *__restrict__ n_uniq,
                                                           int32_t *__restrict__ mgofs,
                                                           int mfma_min, int mfma_min_shared) {
  __shared__ int cm[kDispCells];
  __shared__ int cnt[kSelMaxE];
  __shared__ int base[kSelMaxE];
  __shared__ int ucnt[kSelMaxE];  // count of the u-th unique expert
  __shared__ int uexp[kSelMaxE];  // its expert id
  __shared__ int uoff[kSelMaxE];  // its first pair
  __shared__ uint64_t wtot[kDispWaves];
  __shared__ int s_nu;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = (int64_t)T * k;

  constexpr int kJ = kDispMaxChunks / kDispWaves;
  // this thread's pairs of the round starting at r0 (chunk wave + 16 j,
  // lane): the expert ids, E for none; every load issued before any use
  int ky[kJ];
  auto load_keys = [&](int64_t r0) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = wave + kDispWaves * j;
      const int64_t i = r0 + 64 * c + lane;
      const int e = (c < C && i < n) ? idx[i] : -1;
      ky[j] = (e >= 0 && e < E) ? e : E;
    }
  };
  // a single round: the keys are loaded once and counted from registers
  const bool one_round = n <= (int64_t)64 * C;
  if (one_round) load_keys(0);
  for (int e = tid; e < E; e += kDispThreads) cnt[e] = 0;
  __syncthreads();
  if (one_round) {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (ky[j] < E) atomicAdd(&cnt[ky[j]], 1);
  } else {
    for (int64_t i0 = tid; i0 < n; i0 += 4 * kDispThreads) {
      int ev[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + (int64_t)u * kDispThreads;
        ev[u] = i < n ? idx[i] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ev[u] >= 0 && ev[u] < E) atomicAdd(&cnt[ev[u]], 1);
    }
  }
  __syncthreads();

  // inclusive scan over the experts (thread e holds expert e) of the count
  // and the nonzero flag, as the halves of one 64-bit word
  const int c0 = tid < E ? cnt[tid] : 0;
  const uint64_t v = (uint64_t)(uint32_t)c0 | ((uint64_t)(c0 > 0 ? 1 : 0) << 32);
  uint64_t inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up_u64(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wtot[w];
  const uint64_t exc = inc - v;
  if (tid < E) {
    counts[tid] = c0;
    offs[tid] = (int32_t)(uint32_t)exc;
    base[tid] = (int)(uint32_t)exc;
    if (c0 > 0) {
      uniq[(int)(exc >> 32)] = tid;
      ucnt[(int)(exc >> 32)] = c0;
      uexp[(int)(exc >> 32)] = tid;
      uoff[(int)(exc >> 32)] = (int)(uint32_t)exc;
    }
  }
  if (tid == kDispThreads - 1) {
    offs[E] = (int32_t)(uint32_t)inc;
    n_uniq[0] = (int32_t)(inc >> 32);
    s_nu = (int)(inc >> 32);
  }
  __syncthreads();

  if (mgofs) {
    // thread i: union slots 2i, 2i + 1 (at most 1025 slots)
    const int nu = s_nu, slots = nu + 1;
    auto groups = [&](int u) -> uint64_t {
      const int nt = u < nu ? ucnt[u] : T;
      const int mn = u < nu ? mfma_min : mfma_min_shared;
      return (uint64_t)mfma_groups(nt, mn, kMfmaGroup) |
             ((uint64_t)mfma_groups(nt, mn, kMfmaGroup / 2) << 32);
    };
    const uint64_t g0 = 2 * tid < slots ? groups(2 * tid) : 0;
    const uint64_t g1 = 2 * tid + 1 < slots ? groups(2 * tid + 1) : 0;
    uint64_t gi = g0 + g1;
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t o = shfl_up_u64(gi, d);
      if (lane >= d) gi += o;
    }
    if (lane == 63) wtot[wave] = gi;
    __syncthreads();
    for (int w = 0; w < wave; ++w) gi += wtot[w];
    const uint64_t ge = gi - (g0 + g1);
    int32_t *m32 = mgofs + E + 2;
    if (2 * tid < slots) {
      mgofs[2 * tid] = (int32_t)(uint32_t)ge;
      m32[2 * tid] = (int32_t)(ge >> 32);
    }
    if (2 * tid + 1 < slots) {
      mgofs[2 * tid + 1] = (int32_t)(uint32_t)(ge + g0);
      m32[2 * tid + 1] = (int32_t)((ge + g0) >> 32);
    }
    if (tid == kDispThreads - 1) {  // totals
      mgofs[slots] = (int32_t)(uint32_t)gi;
      m32[slots] = (int32_t)(gi >> 32);
    }
    // group -> slot
    int32_t *s64 = mgofs + 2 * (E + 2), *s32 = s64 + mfma_gmax(T, k, E);
    const uint32_t e64 = (uint32_t)ge, e32 = (uint32_t)(ge >> 32);
    const uint32_t a64 = (uint32_t)g0, a32 = (uint32_t)(g0 >> 32);
    const uint32_t b64 = (uint32_t)g1, b32 = (uint32_t)(g1 >> 32);
    for (uint32_t j = 0; j < a64; ++j) s64[e64 + j] = 2 * tid;
    for (uint32_t j = 0; j < b64; ++j) s64[e64 + a64 + j] = 2 * tid + 1;
    for (uint32_t j = 0; j < a32; ++j) s32[e32 + j] = 2 * tid;
    for (uint32_t j = 0; j < b32; ++j) s32[e32 + a32 + j] = 2 * tid + 1;
    // group counts and descriptors: {expert, first pair, first token, tokens}
    int4 *hdr = reinterpret_cast<int4 *>(mgofs + mfma_desc_off(T, k, E));
    int4 *d64 = hdr + 1, *d32 = d64 + mfma_gmax(T, k, E);
    if (tid == kDispThreads - 1) hdr[0] = make_int4((int)(uint32_t)gi, (int)(gi >> 32), nu, 0);
    auto descs = [&](int u, uint32_t first, uint32_t ng, int tok, int4 *d) {
      const bool sh = u == nu;
      const int e = sh ? -1 : uexp[u], p0 = sh ? -1 : uoff[u], nt = sh ? T : ucnt[u];
      for (uint32_t j = 0; j < ng; ++j)
        d[first + j] = make_int4(e, p0, (int)j * tok, min(tok, nt - (int)j * tok));
    };
    if (2 * tid < slots) {
      descs(2 * tid, e64, a64, kMfmaGroup, d64);
      descs(2 * tid, e32, a32, kMfmaGroup / 2, d32);
    }
    if (2 * tid + 1 < slots) {
      descs(2 * tid + 1, e64 + a64, b64, kMfmaGroup, d64);
      descs(2 * tid + 1, e32 + a32, b32, kMfmaGroup / 2, d32);
    }
  }

  const int nb = 32 - __clz(E);  // bits of the ids 0 .. E (E: no expert)
  const int rows = C / P;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t r0 = 0; r0 < n; r0 += (int64_t)64 * C) {
    if (!one_round) load_keys(r0);
    for (int m = tid; m < C * E; m += kDispThreads) cm[m] = 0;
    __syncthreads();
    int rk[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = wave + kDispWaves * j;
      rk[j] = 0;
      if (c < C) {  // uniform: every lane of the wave
        const int key = ky[j];
        uint64_t same = ~0ull;
        for (int b = 0; b < nb; ++b) {
          const bool bit = (key >> b) & 1;
          const uint64_t bal = __ballot(bit);
          same &= bit ? bal : ~bal;
        }
        const int rank = __popcll(same & below);
        if (key < E && rank == 0) cm[c * E + key] = __popcll(same);
        rk[j] = rank;
      }
    }
    __syncthreads();
    // each expert's column: P consecutive lanes of one wave, rows apiece,
    // turned into first positions: base + exclusive prefix over the chunks
    if (tid < E * P) {
      const int e = tid / P, p = tid % P;
      int s = 0;
      for (int c = p * rows; c < (p + 1) * rows; ++c) {
        const int x = cm[c * E + e];
        cm[c * E + e] = s;
        s += x;
      }
      int ip = s;
      for (int d = 1; d < P; d <<= 1) {
        const int o = __shfl_up(ip, d, 64);
        if (p >= d) ip += o;
      }
      const int add = base[e] + ip - s;
      for (int c = p * rows; c < (p + 1) * rows; ++c) cm[c * E + e] += add;
      // the column's lanes are one wave's, whose reads of base[e] above
      // precede this write
      if (p == P - 1) base[e] += ip;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = wave + kDispWaves * j;
      if (c < C && ky[j] < E) {
        const int64_t i = r0 + 64 * c + lane;
        perm[cm[c * E + ky[j]] + rk[j]] = (int32_t)i;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_dispatch(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offs,
                           int32_t *perm, int32_t *uniq, int32_t *n_uniq, hipStream_t st,
                           int32_t *mgofs, int mfma_min, int mfma_min_shared) {
  if (E < 1 || E > kSelMaxE) return hipErrorInvalidValue;
  int P = 1;
  while (P * 2 <= 64 && P * 2 * E <= kDispThreads) P *= 2;
  int C = std::min(kDispMaxChunks, kDispCells / E / 16 * 16);
  if (C < 16 || C % P) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dispatch, dim3(1), dim3(kDispThreads), 0, st, idx, T, k, E, C, P, counts,
                     offs, perm, uniq, n_uniq, mgofs, mfma_min, mfma_min_shared);
  return hipGetLastError();
}

}  // namespace coli
