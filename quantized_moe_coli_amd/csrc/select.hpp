// select.hpp -- one wavefront selects the routed experts of one token.
//
// colibrì README, "Implemented features": DeepSeek-V3-like sigmoid router
// with the aux-loss-free selection bias (noaux_tc) and routed_scaling_factor;
// README "Quick start": adaptive expert top-p.  Steps (all binary32 unless
// stated, in the order of the definition, no contraction):
//   sigma_e = fl32(1/(1+exp(-l_e))) evaluated in binary64;
//   c_e = sigma_e + bias_e (selection only);
//   group score = sum of the two largest c of the group (contiguous groups);
//   keep topk_group groups, then top_k experts of the kept groups by c
//   (ties to the lower index; rank order = output slot order);
//   w_j = (sigma_j / S) * rsf, S the sum of the chosen sigma in rank order;
//   expert top-p drops the slots outside the smallest weight-descending
//   prefix whose normalised sum reaches p.
// Lane l holds experts l, l+64, ... (up to 16 each, E <= 1024).  Arg-max
// steps are a DPP max of the value, then a DPP min of the indices holding it.
#pragma once

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace coli {

constexpr int kSelMaxE = 1024, kSelMaxK = 32, kSelEPL = kSelMaxE / 64;

// sigma(l) evaluated in binary64, rounded once to binary32.
__device__ __forceinline__ float sigmoid_f64(float l) {
  return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// A value every lane of the wave holds, as a wave-uniform (scalar) value.
__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int L>
__device__ __forceinline__ int group_min_i32(int v) {
  if constexpr (L >= 2) v = min(v, dpp_i32<0xB1>(v));
  if constexpr (L >= 4) v = min(v, dpp_i32<0x4E>(v));
  if constexpr (L >= 8) v = min(v, dpp_i32<0x141>(v));
  if constexpr (L >= 16) v = min(v, dpp_i32<0x140>(v));
  if constexpr (L >= 32) v = min(v, dpp_i32<0x142, 0xA>(v));
  if constexpr (L >= 64) v = min(v, dpp_i32<0x143, 0xC>(v));
  return v;
}

// Index of the best (value desc, index asc) valid candidate over the wave;
// uniform result, -1 if no lane has a valid candidate.
__device__ __forceinline__ int wave_argmax(float v, int i, bool valid) {
  const float vm = valid ? v : -INFINITY;
  const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(group_max<64>(vm)), 63));
  const int key = (valid && v == mx) ? i : 0x7fffffff;
  const int mn = __builtin_amdgcn_readlane(group_min_i32<64>(key), 63);
  return mn == 0x7fffffff ? -1 : mn;
}

// Max over aligned segments of L lanes, broadcast to every lane of the segment.
template <int L>
__device__ __forceinline__ float seg_max_all(float v) {
  v = group_max<L>(v);
  if constexpr (L == 32) v = __shfl(v, (threadIdx.x & 32) | 31, 64);
  if constexpr (L == 64) v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return v;
}

// Sum of the two largest values in each aligned segment of L lanes (the
// second largest counts a repeated maximum), broadcast to the segment.
template <int L>
__device__ __forceinline__ float seg_top2_sum(float v) {
  const float t1 = seg_max_all<L>(v);
  const uint64_t eq = __ballot(v == t1);
  const int lane = threadIdx.x & 63;
  const uint64_t segmask = (L == 64) ? ~0ull : (((1ull << L) - 1ull) << (lane & ~(L - 1)));
  const float rest = seg_max_all<L>(v == t1 ? -INFINITY : v);  // all lanes take part
  const float t2 = (__popcll(eq & segmask) >= 2) ? t1 : rest;
  return t1 + t2;
}

struct SelScratch {  // LDS scratch of one wave
  float sig[kSelMaxE];
  float cst[kSelMaxE];  // biased scores, for group sizes that do not tile a wave
  float gs[64];
  int rank[kSelMaxK];
  float pn[kSelMaxK];
  int keep[kSelMaxK];
  float sum;
};

template <int EPL = kSelEPL>
__device__ __forceinline__ void select_core(const RouterCfg &cfg, const float *c,
                                            const float *__restrict__ sig, SelScratch &sc,
                                            int32_t *idx_out, float *w_out);

// Selects a token's experts.  Lane j < k writes slot j of `idx_out`/`w_out`
// (any address space).  EPL >= (E + 63) / 64 candidates per lane.
template <int EPL>
__device__ __forceinline__ void select_token_t(const RouterCfg &cfg, const float *__restrict__ lrow,
                                               const float *__restrict__ bias, SelScratch &sc,
                                               int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  const int E = cfg.E;
  const int epl = (E + 63) / 64;  // candidates per lane (uniform)
  float c[EPL], lv[EPL], bv[EPL];
  // all loads first (clamped addresses), so they are in flight together
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    if (m < epl) {
      const int ec = min(lane + 64 * m, E - 1);
      lv[m] = lrow[ec];
      bv[m] = bias ? bias[ec] : 0.f;
    }
  }
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    const int e = lane + 64 * m;
    c[m] = 0.f;
    if (m < epl) {
      const float s = sigmoid_f64(lv[m]);
      if (e < E) sc.sig[e] = s;
      c[m] = s + bv[m];
    }
  }

  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  select_core<EPL>(cfg, c, sc.sig, sc, idx_out, w_out);
}

// The instance with as few candidates per lane as the expert count allows
// (the same selection: lanes' candidates past E are never eligible).
__device__ __forceinline__ void select_token(const RouterCfg &cfg, const float *__restrict__ lrow,
                                             const float *__restrict__ bias, SelScratch &sc,
                                             int32_t *idx_out, float *w_out) {
  if (cfg.E <= 64) select_token_t<1>(cfg, lrow, bias, sc, idx_out, w_out);
  else if (cfg.E <= 256) select_token_t<4>(cfg, lrow, bias, sc, idx_out, w_out);
  else select_token_t<kSelEPL>(cfg, lrow, bias, sc, idx_out, w_out);
}

// The selection itself from the biased scores c[m] of experts lane + 64 m
// (every lane, c[m] = 0 past E; EPL >= E / 64 of them) and the sigmoid
// scores sig[e] (any address space, visible to the whole wave): groups,
// experts in rank order, weights and expert top-p, by one wave.
template <int EPL>
__device__ __forceinline__ void select_core(const RouterCfg &cfg, const float *c,
                                            const float *__restrict__ sig, SelScratch &sc,
                                            int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  const int E = cfg.E, k = cfg.k, G = cfg.n_group, per = E / G;
  // groups
  uint32_t allowed = 0;  // bit m: candidate lane + 64 m is in a kept group
  if (cfg.topk_group >= G) {
#pragma unroll
    for (int m = 0; m < EPL; ++m)
      if (lane + 64 * m < E) allowed |= 1u << m;
  } else {
    const bool aligned = per <= 64 && (64 % per) == 0;
    if (aligned) {
#pragma unroll
      for (int m = 0; m < EPL; ++m) {
        if (64 * m >= E) break;
        float gsum;
        switch (per) {
          case 1: gsum = c[m]; break;
          case 2: gsum = seg_top2_sum<2>(c[m]); break;
          case 4: gsum = seg_top2_sum<4>(c[m]); break;
          case 8: gsum = seg_top2_sum<8>(c[m]); break;
          case 16: gsum = seg_top2_sum<16>(c[m]); break;
          case 32: gsum = seg_top2_sum<32>(c[m]); break;
          default: gsum = seg_top2_sum<64>(c[m]); break;
        }
        const int e = lane + 64 * m;
        if (e < E && (e % per) == 0) sc.gs[e / per] = gsum;
      }
    } else {
      // general group size: one lane per group scans it (binary32 adds of
      // the same two values, so the score is identical)
      float *cstage = sc.cst;
#pragma unroll
      for (int m = 0; m < EPL; ++m)
        if (lane + 64 * m < E) cstage[lane + 64 * m] = c[m];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      if (lane < G) {
        int b1 = -1, b2 = -1;
        for (int e = lane * per; e < (lane + 1) * per; ++e) {
          if (b1 < 0 || cstage[e] > cstage[b1]) { b2 = b1; b1 = e; }
          else if (b2 < 0 || cstage[e] > cstage[b2]) { b2 = e; }
        }
        sc.gs[lane] = per >= 2 ? cstage[b1] + cstage[b2] : cstage[b1];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const float gv = lane < G ? sc.gs[lane] : 0.f;
    uint64_t keep = 0;
    for (int n = 0; n < cfg.topk_group; ++n) {
      const int gb = wave_argmax(gv, lane, lane < G && !((keep >> lane) & 1ull));
      if (gb >= 0) keep |= 1ull << gb;
    }
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = lane + 64 * m;
      if (e < E && ((keep >> (e / per)) & 1ull)) allowed |= 1u << m;
    }
  }

  // experts, in rank order
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = 0x7fffffff;
    bool have = false;
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      if ((allowed >> m) & 1u) {
        if (!have || c[m] > bv) { bv = c[m]; bi = lane + 64 * m; have = true; }
      }
    }
    const int win = wave_argmax(bv, bi, have);
    if (win >= 0 && (win & 63) == lane) allowed &= ~(1u << (win >> 6));
    if (lane == 0) sc.rank[j] = win;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // weights: lane j owns slot j; the sums run serially in rank order (lane 0)
  if (lane == 0) {
    float S = 0.f;
    for (int j = 0; j < k; ++j)
      if (sc.rank[j] >= 0) S += sig[sc.rank[j]];
    sc.sum = S;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const float S = sc.sum;
  int my_i = -1;
  float my_w = 0.f, my_s = 0.f;
  if (lane < k) {
    my_i = sc.rank[lane];
    if (my_i >= 0) {
      my_s = sig[my_i];
      if (cfg.norm) my_w = (S != 0.f) ? (my_s / S) * cfg.rsf : 0.f;
      else my_w = my_s * cfg.rsf;
    }
  }
  if (cfg.top_p > 0.f && cfg.top_p < 1.f) {
    if (lane < k) {
      sc.pn[lane] = (S != 0.f && my_i >= 0) ? my_s / S : 0.f;
      sc.keep[lane] = 0;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane == 0) {
      // visit slots by normalised weight (desc, rank order on ties) until the
      // running binary32 sum reaches p
      uint32_t seen = 0;
      float cum = 0.f;
      for (int n = 0; n < k; ++n) {
        int best = -1;
        for (int j = 0; j < k; ++j)
          if (!((seen >> j) & 1u) && (best < 0 || sc.pn[j] > sc.pn[best])) best = j;
        seen |= 1u << best;
        sc.keep[best] = 1;
        cum += sc.pn[best];
        if (cum >= cfg.top_p) break;
      }
      float Sk = 0.f;
      for (int j = 0; j < k; ++j)
        if (sc.keep[j] && sc.rank[j] >= 0) Sk += sig[sc.rank[j]];
      sc.sum = Sk;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane < k) {
      const float Sk = sc.sum;
      if (!sc.keep[lane] || my_i < 0) {
        my_i = -1;
        my_w = 0.f;
      } else if (cfg.renorm) {
        my_w = (Sk != 0.f) ? (my_s / Sk) * cfg.rsf : 0.f;
      }
    }
  }
  if (lane < k) {
    idx_out[lane] = my_i;
    w_out[lane] = my_w;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

}  // namespace coli

namespace coli {

// ---------------------------------------------------------------------------
// The same selection computed by a whole workgroup of NT threads, for the
// latency-critical single-token path.  Instead of k rounds of wave arg-max it
// counts, for every candidate of the kept groups, how many candidates beat it
// (value desc, index asc): that count is the candidate's rank, a total order
// identical to repeated arg-max, so the chosen experts, their slot order and
// the weights are bit-identical to select_token.
// ---------------------------------------------------------------------------
// A token's router scores: sigma = fl32(sigmoid(logit)) and the biased
// score c = sigma + bias, per expert.
struct SelInput {
  float c[kSelMaxE];
  float sg[kSelMaxE];
};

struct SelWgScratch {
  float candv[kSelMaxE];  // biased scores of the kept groups' experts
  int cande[kSelMaxE];    // their expert ids
  float gtop[64][2];      // two largest biased scores of each group
  float gs[64];
  int gkeep[64];          // kept group ids, in rank order
  int slot[kSelMaxK];     // expert of each rank
  float ssig[kSelMaxK];   // its sigmoid score
  float pn[kSelMaxK];
  int keep[kSelMaxK];
  float sum;
};

// (v2, e2) beats (v, e): larger value, or equal value and lower index.
__device__ __forceinline__ int beats(float v2, int e2, float v, int e) {
  return (v2 > v || (v2 == v && e2 < e)) ? 1 : 0;
}

// The last step of a selection: ranks M candidates (biased scores candv,
// expert ids cande; sig_of(m, e) gives candidate m's sigmoid score) by
// (value desc, index asc), keeps the k best in rank order and writes their
// weights -- normalised by the binary32 sum of the kept sigmoids in rank
// order, times rsf -- with expert top-p applied if configured.  P threads
// share a candidate, so the ranking is spread over the whole workgroup.
// slot[0..k) must hold -1 on entry (visible to every thread).
template <int NT, typename SigOf>
__device__ __forceinline__ void rank_and_weigh(const RouterCfg &cfg, int M, const float *candv,
                                               const int *cande, SigOf sig_of, int *slot,
                                               float *ssig, float *pn, int *keep, float &sum,
                                               int32_t *idx_out, float *w_out) {
  const int tid = threadIdx.x, k = cfg.k;
  // rank of each candidate = number of candidates that beat it; P lanes of a
  // wave share a candidate (P a power of two, P * candidates <= NT)
  int P = 1;
  while (P < 64 && 2 * P * M <= NT) P *= 2;
  const int per_pass = NT / P;
  for (int m0 = 0; m0 < M; m0 += per_pass) {
    const int m = m0 + tid / P, part = tid % P;
    const bool valid = m < M;
    const float v = valid ? candv[m] : 0.f;
    const int e = valid ? cande[m] : 0;
    int r = 0;
    if (valid)
      for (int q = part; q < M; q += P) r += beats(candv[q], cande[q], v, e);
    for (int o = 1; o < P; o *= 2) r += __shfl_xor(r, o, 64);
    if (valid && part == 0 && r < k) {
      slot[r] = e;
      ssig[r] = sig_of(m, e);
    }
  }
  __syncthreads();

  // weights: the sums run in rank order (one thread), slot j by thread j
  if (tid == 0) {
    float S = 0.f;
    for (int j = 0; j < k; ++j)
      if (slot[j] >= 0) S += ssig[j];
    sum = S;
  }
  __syncthreads();
  const float S = sum;
  int my_i = -1;
  float my_w = 0.f, my_s = 0.f;
  if (tid < k) {
    my_i = slot[tid];
    if (my_i >= 0) {
      my_s = ssig[tid];
      if (cfg.norm) my_w = (S != 0.f) ? (my_s / S) * cfg.rsf : 0.f;
      else my_w = my_s * cfg.rsf;
    }
  }
  if (cfg.top_p > 0.f && cfg.top_p < 1.f) {
    if (tid < k) {
      pn[tid] = (S != 0.f && my_i >= 0) ? my_s / S : 0.f;
      keep[tid] = 0;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t seen = 0;
      float cum = 0.f;
      for (int n = 0; n < k; ++n) {
        int best = -1;
        for (int j = 0; j < k; ++j)
          if (!((seen >> j) & 1u) && (best < 0 || pn[j] > pn[best])) best = j;
        seen |= 1u << best;
        keep[best] = 1;
        cum += pn[best];
        if (cum >= cfg.top_p) break;
      }
      float Sk = 0.f;
      for (int j = 0; j < k; ++j)
        if (keep[j] && slot[j] >= 0) Sk += ssig[j];
      sum = Sk;
    }
    __syncthreads();
    if (tid < k) {
      const float Sk = sum;
      if (!keep[tid] || my_i < 0) {
        my_i = -1;
        my_w = 0.f;
      } else if (cfg.renorm) {
        my_w = (Sk != 0.f) ? (my_s / Sk) * cfg.rsf : 0.f;
      }
    }
  }
  if (tid < k) {
    idx_out[tid] = my_i;
    w_out[tid] = my_w;
  }
  __syncthreads();
}

// `in`: the token's scores (typically in LDS).
template <int NT>
__device__ __forceinline__ void select_wg(const RouterCfg &cfg, const SelInput &in,
                                          SelWgScratch &sc, int32_t *idx_out, float *w_out) {
  const int tid = threadIdx.x;
  const int E = cfg.E, G = cfg.n_group, per = E / G;
  const float *cval = in.c, *sig = in.sg;
  if (tid < kSelMaxK) sc.slot[tid] = -1;
  if (tid < 64) sc.gkeep[tid] = tid < G ? tid : 0;  // valid ids even if NaN scores tie every rank
  __syncthreads();

  // groups: score = sum of the two largest biased scores (rank 0 and 1 of
  // the group); keep the topk_group best groups
  const bool all_groups = cfg.topk_group >= G;
  if (!all_groups) {
    for (int e = tid; e < E; e += NT) {
      const int g = e / per, base = g * per;
      const float v = cval[e];
      int r = 0;
      for (int q = base; q < base + per; ++q) r += beats(cval[q], q, v, e);
      if (r < 2) sc.gtop[g][r] = v;
    }
    __syncthreads();
    for (int g = tid; g < G; g += NT) sc.gs[g] = per >= 2 ? sc.gtop[g][0] + sc.gtop[g][1] : sc.gtop[g][0];
    __syncthreads();
    for (int g = tid; g < G; g += NT) {
      const float v = sc.gs[g];
      int r = 0;
      for (int g2 = 0; g2 < G; ++g2) r += beats(sc.gs[g2], g2, v, g);
      if (r < cfg.topk_group) sc.gkeep[r] = g;
    }
    __syncthreads();
  }
  const int ng = all_groups ? G : cfg.topk_group;

  // the kept groups' experts, compacted
  const int M = ng * per;
  for (int m = tid; m < M; m += NT) {
    const int gi = m / per;
    const int e = (all_groups ? gi : sc.gkeep[gi]) * per + (m - gi * per);
    sc.candv[m] = cval[e];
    sc.cande[m] = e;
  }
  __syncthreads();

  rank_and_weigh<NT>(cfg, M, sc.candv, sc.cande, [&](int, int e) { return sig[e]; }, sc.slot, sc.ssig,
                     sc.pn, sc.keep, sc.sum, idx_out, w_out);
}


// ---------------------------------------------------------------------------
// Fast form of the workgroup selection, for E <= NT experts in groups of
// `per` that tile a wavefront (per divides 64) with at most 64 experts left
// after the group step -- the GLM-5.2 router.  Only an expert ranked below
// k inside its own group can be among the token's k (the top k of a union
// of groups lie in the groups' own top k).  Thread e owns expert e: it
// counts the members of its group that beat it (reading the group's scores
// from LDS as broadcasts), every wave ranks the groups itself from their
// DPP-reduced scores, the kept groups' top min(k, per) experts are ranked
// by wave 0 the same way, and wave 0 computes the weights.  Same total order
// (value desc, index asc) and the same binary32 operations in the same
// order as select_token: bit-identical.
// ---------------------------------------------------------------------------
struct SelFastScratch {
  __align__(16) float candv[64];  // biased scores of the candidates
  __align__(16) int cande[64];    // their expert ids
  float cands[64];                // their sigmoid scores
  __align__(16) float gs[64];
  __align__(16) int slot[kSelMaxK];
  __align__(16) float ssig[kSelMaxK];
  float pn[kSelMaxK];
  int keep[kSelMaxK];
  float sum;
};

__host__ __device__ __forceinline__ bool select_fast_ok(int E, int G, int topk_group, int k,
                                                        int nt) {
  const int per = E / G;
  const int ng = topk_group < G ? topk_group : G;
  return E <= nt && per <= 64 && 64 % per == 0 && ng * (k < per ? k : per) <= 64;
}

__device__ __forceinline__ float rdlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Number of entries of v[0, N) (16-byte aligned, LDS) that beat (x, xi),
// entry j carrying index base + j.  All loads are issued before the first
// comparison.
template <int N>
__device__ __forceinline__ int count_beating(const float *v, int base, float x, int xi) {
  int r = 0;
  if constexpr (N >= 4) {
    float4 q[N / 4];
    const float4 *v4 = reinterpret_cast<const float4 *>(v);
#pragma unroll
    for (int j = 0; j < N / 4; ++j) q[j] = v4[j];
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      const int b = base + 4 * j;
      r += (q[j].x > x || (q[j].x == x && b < xi)) ? 1 : 0;
      r += (q[j].y > x || (q[j].y == x && b + 1 < xi)) ? 1 : 0;
      r += (q[j].z > x || (q[j].z == x && b + 2 < xi)) ? 1 : 0;
      r += (q[j].w > x || (q[j].w == x && b + 3 < xi)) ? 1 : 0;
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) r += (v[j] > x || (v[j] == x && base + j < xi)) ? 1 : 0;
  }
  return r;
}

template <int NT, int PER>
__device__ __forceinline__ void select_fast_t(const RouterCfg &cfg, const SelInput &in,
                                              SelFastScratch &sc, int32_t *idx_out, float *w_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int E = cfg.E, k = cfg.k, G = cfg.n_group;
  const int kk = k < PER ? k : PER;  // candidates per kept group
  const bool valid = tid < E;
  const int g = tid / PER;
  const float c = valid ? in.c[tid] : -INFINITY;

  // rank inside the group, and the group scores
  const int rin = valid ? count_beating<PER>(in.c + g * PER, g * PER, c, tid) : 0;
  unsigned long long gmask = G >= 64 ? ~0ull : ((1ull << G) - 1ull);
  if (cfg.topk_group < G) {
    float gsum;
    if constexpr (PER == 1) gsum = c;
    else gsum = seg_top2_sum<PER>(c);
    if (valid && tid % PER == 0) sc.gs[g] = gsum;
    __syncthreads();
    // every wave ranks the groups (lane g2 < G holds group g2)
    const float gv = lane < G ? sc.gs[lane] : 0.f;
    int r = 0;
#pragma unroll 8
    for (int g2 = 0; g2 < G; ++g2) {
      const float v2 = sc.gs[g2];  // broadcast read
      r += (v2 > gv || (v2 == gv && g2 < lane)) ? 1 : 0;
    }
    gmask = __ballot(lane < G && r < cfg.topk_group);
    // finite scores rank the groups as a permutation, so exactly topk_group
    // bits are set; NaN scores (a wait that gave up) can tie ranks, and the
    // highest extra bits are dropped so the candidate slots stay in range
    while (__popcll(gmask) > cfg.topk_group) gmask &= ~(1ull << (63 - __clzll(gmask)));
  }

  // the kept groups' top kk experts, by group id then rank inside the group
  if (valid && rin < kk && ((gmask >> g) & 1ull)) {
    const int pos = __popcll(gmask & ((1ull << g) - 1ull)) * kk + rin;
    sc.candv[pos] = c;
    sc.cande[pos] = tid;
    sc.cands[pos] = in.sg[tid];
  }
  __syncthreads();

  // rank of each candidate among the M <= 64: P = NT/64 consecutive lanes
  // share candidate m, each comparing it with every P-th candidate; the
  // partial counts are summed with DPP (exact: counts are small integers)
  constexpr int P = NT / 64;
  static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "P lanes per candidate");
  const int M = __popcll(gmask) * kk;
  {
    const int m = tid / P, part = tid % P;
    const bool valid = m < M;
    const float v = valid ? sc.candv[m] : 0.f;
    const int e = valid ? sc.cande[m] : 0;
    float r = 0.f;
    if (valid)
      for (int q2 = part; q2 < M; q2 += P) r += (float)beats(sc.candv[q2], sc.cande[q2], v, e);
    r = group_sum<P>(r);
    if (valid && part == 0 && (int)r < k) {
      sc.slot[(int)r] = e;
      sc.ssig[(int)r] = sc.cands[m];
    }
  }
  __syncthreads();
  if (tid < 64) {
    // wave 0, lane j < k: slot j.  S = the kept sigmoids summed in slot
    // order, read across lanes (no memory round trips)
    const int my_i = lane < k ? sc.slot[lane] : -1;
    const bool win = my_i >= 0;
    const float sgv = win ? sc.ssig[lane] : 0.f;
    float S = 0.f;
    for (int j = 0; j < k; ++j)
      if (__builtin_amdgcn_readlane(my_i, j) >= 0) S += rdlane(sgv, j);
    float my_w;
    if (cfg.norm) my_w = (S != 0.f) ? (sgv / S) * cfg.rsf : 0.f;
    else my_w = sgv * cfg.rsf;
    bool kept = win;
    if (cfg.top_p > 0.f && cfg.top_p < 1.f) {
      // slots by normalised weight (desc, slot order on ties) while the
      // running binary32 sum is below p
      const float pn = (S != 0.f && win) ? sgv / S : 0.f;
      int rk = 0;
      for (int j = 0; j < k; ++j) {
        const bool wj = __builtin_amdgcn_readlane(my_i, j) >= 0;
        const float pj = rdlane(pn, j);
        rk += (wj && (pj > pn || (pj == pn && j < lane))) ? 1 : 0;
      }
      float cum = 0.f;
      kept = false;
      for (int q2 = 0; q2 < k; ++q2) {
        if (cum >= cfg.top_p) break;
        const unsigned long long who = __ballot(win && rk == q2);
        if (!who) break;
        const int src = __ffsll((long long)who) - 1;
        if (lane == src) kept = true;
        cum += rdlane(pn, src);
      }
      float Sk = 0.f;
      for (int j = 0; j < k; ++j) {
        const int kj = __builtin_amdgcn_readlane((int)(win && kept), j);
        if (kj) Sk += rdlane(sgv, j);
      }
      if (kept && cfg.renorm) my_w = (Sk != 0.f) ? (sgv / Sk) * cfg.rsf : 0.f;
    }
    if (lane < k) {
      idx_out[lane] = kept ? my_i : -1;
      w_out[lane] = kept ? my_w : 0.f;
    }
  }
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ void select_fast(const RouterCfg &cfg, const SelInput &in,
                                            SelFastScratch &sc, int32_t *idx_out, float *w_out) {
  // slots no candidate reaches (only with NaN scores) stay empty
  if ((int)threadIdx.x < kSelMaxK) sc.slot[threadIdx.x] = -1;
  switch (cfg.E / cfg.n_group) {
    case 1: select_fast_t<NT, 1>(cfg, in, sc, idx_out, w_out); break;
    case 2: select_fast_t<NT, 2>(cfg, in, sc, idx_out, w_out); break;
    case 4: select_fast_t<NT, 4>(cfg, in, sc, idx_out, w_out); break;
    case 8: select_fast_t<NT, 8>(cfg, in, sc, idx_out, w_out); break;
    case 16: select_fast_t<NT, 16>(cfg, in, sc, idx_out, w_out); break;
    case 32: select_fast_t<NT, 32>(cfg, in, sc, idx_out, w_out); break;
    default: select_fast_t<NT, 64>(cfg, in, sc, idx_out, w_out); break;
  }
}

}  // namespace coli
