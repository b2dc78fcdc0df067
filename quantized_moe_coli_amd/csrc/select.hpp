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

// Selects a token's experts.  Lane j < k writes slot j of `idx_out`/`w_out`
// (any address space).
__device__ __forceinline__ void select_token(const RouterCfg &cfg, const float *__restrict__ lrow,
                                             const float *__restrict__ bias, SelScratch &sc,
                                             int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  const int E = cfg.E, k = cfg.k, G = cfg.n_group, per = E / G;
  const int epl = (E + 63) / 64;  // candidates per lane (uniform)
  float c[kSelEPL], lv[kSelEPL], bv[kSelEPL];
  // all loads first (clamped addresses), so they are in flight together
#pragma unroll
  for (int m = 0; m < kSelEPL; ++m) {
    if (m < epl) {
      const int ec = min(lane + 64 * m, E - 1);
      lv[m] = lrow[ec];
      bv[m] = bias ? bias[ec] : 0.f;
    }
  }
#pragma unroll
  for (int m = 0; m < kSelEPL; ++m) {
    const int e = lane + 64 * m;
    c[m] = 0.f;
    if (m < epl) {
      const float s = (float)(1.0 / (1.0 + exp(-(double)lv[m])));
      if (e < E) sc.sig[e] = s;
      c[m] = s + bv[m];
    }
  }

  // groups
  uint32_t allowed = 0;  // bit m: candidate lane + 64 m is in a kept group
  if (cfg.topk_group >= G) {
#pragma unroll
    for (int m = 0; m < kSelEPL; ++m)
      if (lane + 64 * m < E) allowed |= 1u << m;
  } else {
    const bool aligned = per <= 64 && (64 % per) == 0;
    if (aligned) {
#pragma unroll
      for (int m = 0; m < kSelEPL; ++m) {
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
      for (int m = 0; m < kSelEPL; ++m)
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
    for (int m = 0; m < kSelEPL; ++m) {
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
    for (int m = 0; m < kSelEPL; ++m) {
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
      if (sc.rank[j] >= 0) S += sc.sig[sc.rank[j]];
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
      my_s = sc.sig[my_i];
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
        if (sc.keep[j] && sc.rank[j] >= 0) Sk += sc.sig[sc.rank[j]];
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
