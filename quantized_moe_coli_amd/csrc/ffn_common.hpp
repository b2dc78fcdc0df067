// ffn_common.hpp -- device pieces shared by the expert-FFN kernels (ffn.hip)
// and the fused decode kernel (decode.hip): activation chunks, the integer
// chunk products with their block scales, expert pointers, token lists of a
// work item and the gate/up + SwiGLU + Q8_0(h) body.
#pragma once

#include "kernels.hpp"

namespace coli {

template <int BITS>
struct Act {
  static constexpr int kInts = Q<BITS>::kElems / 4;
  static constexpr int kD = Q<BITS>::kBlocks;
  int a[kInts];
  float d[kD];
};

// Activation codes/scales for chunk c of a row (codes in BITS ordering).
template <int BITS>
__device__ __forceinline__ void load_act(Act<BITS> &ac, const int8_t *q, const float *d, int c) {
  const uint4 *p = reinterpret_cast<const uint4 *>(q + (size_t)c * Q<BITS>::kElems);
#pragma unroll
  for (int m = 0; m < Act<BITS>::kInts / 4; ++m) {
    const uint4 v = p[m];
    ac.a[4 * m] = (int)v.x;
    ac.a[4 * m + 1] = (int)v.y;
    ac.a[4 * m + 2] = (int)v.z;
    ac.a[4 * m + 3] = (int)v.w;
  }
  if constexpr (BITS == 8) ac.d[0] = d[c >> 1];
  else if constexpr (BITS == 4) ac.d[0] = d[c];
  else { ac.d[0] = d[2 * c]; ac.d[1] = d[2 * c + 1]; }
}

template <int BITS>
__device__ __forceinline__ void zero_act(Act<BITS> &ac) {
#pragma unroll
  for (int m = 0; m < Act<BITS>::kInts; ++m) ac.a[m] = 0;
#pragma unroll
  for (int m = 0; m < Act<BITS>::kD; ++m) ac.d[m] = 0.f;
}

template <int BITS>
__device__ __forceinline__ float chunk_part(const uint4 w, const Act<BITS> &ac) {
  if constexpr (BITS == 8) return ac.d[0] * (float)chunk_dot_q8(w, ac.a);
  else if constexpr (BITS == 4) return ac.d[0] * (float)chunk_dot_q4(w, ac.a);
  else {
    int b0, b1;
    chunk_dot_q2(w, ac.a, b0, b1);
    return ac.d[0] * (float)b0 + ac.d[1] * (float)b1;
  }
}

// The chunk's block sums times their activation scales, in binary64: every
// product of a binary32 scale and an exact int32 block sum is exact there,
// so only the additions of a row's partial sums round (at the 2^-53 level).
template <int BITS>
__device__ __forceinline__ double chunk_part_f64(const uint4 w, const Act<BITS> &ac) {
  if constexpr (BITS == 8) return (double)ac.d[0] * (double)chunk_dot_q8(w, ac.a);
  else if constexpr (BITS == 4) return (double)ac.d[0] * (double)chunk_dot_q4(w, ac.a);
  else {
    int b0, b1;
    chunk_dot_q2(w, ac.a, b0, b1);
    return fma((double)ac.d[0], (double)b0, (double)ac.d[1] * (double)b1);
  }
}

// h = fl32(silu(g) * u) from the binary32 g and u, with silu(z) =
// z / (1 + exp(-z)) and the product evaluated in binary64 and rounded once
// (the expert definition: g and u are the rescaled integer products
// rounded to binary32, the SwiGLU step is exact up to that one rounding).
__device__ __forceinline__ float swiglu_h(float g, float u) {
  const double z = (double)g;
  return (float)((z / (1.0 + exp(-z))) * (double)u);
}

// A row's rescaled product: fl32(s * sum), the sum of its block partials
// taken in binary64.
__device__ __forceinline__ float row_out(double sum, float s) { return (float)(sum * (double)s); }

__device__ __forceinline__ float bcast(float v, int lane_idx) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane_idx));
}

// Row scale of row (p * RPP + rsub) of a wave whose lane i holds the scale of
// its i-th row (p is a compile-time pass index after unrolling).
template <int RPP>
__device__ __forceinline__ float row_scale(float sv, int p, int rsub) {
  if constexpr (RPP == 1) return bcast(sv, p);
  else return rsub ? bcast(sv, RPP * p + 1) : bcast(sv, RPP * p);
}

// Pointers of one expert (e = -1: the shared expert).
struct ExpertPtrs {
  const uint8_t *wg, *wu, *wd;
  const float *sg, *su, *sd;
};

// Where expert e's weights are stored: its own index, or through the expert
// cache its slot (an out-of-range slot reads slot 0).
__device__ __forceinline__ int expert_store(const LayerPtrs &L, int e) {
  if (e < 0 || !L.slot_of) return e;
  const int s = L.slot_of[e];
  return (unsigned)s < (unsigned)L.n_slots ? s : 0;
}

// Pointers of the expert stored at index e (-1: the shared expert).
__device__ __forceinline__ ExpertPtrs expert_ptrs_at(const LayerPtrs &L, int e) {
  ExpertPtrs p;
  if (e < 0) {
    p.wg = L.sh_gate; p.wu = L.sh_up; p.wd = L.sh_down;
    p.sg = L.sh_s_gate; p.su = L.sh_s_up; p.sd = L.sh_s_down;
  } else {
    const size_t gu_stride = (size_t)L.I * (L.H * L.bits / 8);
    const size_t d_stride = (size_t)L.H * (L.I * L.bits / 8);
    p.wg = L.w_gate + (size_t)e * gu_stride;
    p.wu = L.w_up + (size_t)e * gu_stride;
    p.wd = L.w_down + (size_t)e * d_stride;
    p.sg = L.s_gate + (size_t)e * L.I;
    p.su = L.s_up + (size_t)e * L.I;
    p.sd = L.s_down + (size_t)e * L.H;
  }
  return p;
}

__device__ __forceinline__ ExpertPtrs expert_ptrs(const LayerPtrs &L, int e) {
  return expert_ptrs_at(L, expert_store(L, e));
}

// The tokens of one work item: decode -> token 0 at h row `slot`; union ->
// the expert's perm range (routed) or every token (shared); a small fused
// batch (slot kTokPacked) -> up to four tokens named in `tok` (8 bits each)
// at h rows p0, p0 + 1, ....
constexpr int kTokPacked = -2;
struct TokList {
  int n_tok;
  int p0;      // union routed: first perm position; packed: first h row; -1 otherwise
  int slot;    // decode: slot index; kTokPacked: packed list
  bool shared;
  int tok;     // packed list: token n in bits 8n .. 8n + 7
};

__device__ __forceinline__ void tok_at(const FfnArgs &a, bool union_mode, const TokList &s, int n,
                                       int &t, int &hrow, int &j) {
  if (s.slot == kTokPacked) {
    t = (s.tok >> (8 * n)) & 0xFF;
    hrow = s.p0 + n;
    j = 0;
  } else if (!union_mode) {
    t = 0;
    hrow = s.slot;
    j = s.slot;
  } else if (s.shared) {
    t = n;
    hrow = a.disp.offs[a.E] + n;
    j = a.k;
  } else {
    const int p = a.disp.perm[s.p0 + n];
    t = p / a.k;
    j = p % a.k;
    hrow = s.p0 + n;
  }
}

// Union item u -> expert and token list; false past the last unique expert
// and for slots the matrix-core kernels take.
__device__ __forceinline__ bool union_item(const FfnArgs &a, int u, int &e, TokList &s) {
  const int nu = *a.disp.n_uniq;
  if (u > nu) return false;
  s.slot = -1;
  s.shared = (u == nu);
  if (s.shared) {
    e = -1;
    s.n_tok = a.T;
    s.p0 = -1;
  } else {
    e = a.disp.uniq[u];
    s.p0 = a.disp.offs[e];
    s.n_tok = a.disp.offs[e + 1] - s.p0;
  }
  return s.n_tok < (e < 0 ? a.mfma_min_shared : a.mfma_min);
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + Q8_0(h) for BLK blocks of 32 rows (from row block rb)
// of one expert over its tokens, by a workgroup of WAVES waves
// (32*BLK/WAVES rows each); the loads of the next row pass are in flight
// while the current one is reduced.  Each 32-row block is one Q8_0 block of
// h, quantised here.
// ---------------------------------------------------------------------------
// Relaxed device-scope 32-bit store/load: coherent across XCDs per access,
// with no cache-wide write-back or invalidation.
__device__ __forceinline__ void st_dev(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// xq_all/xd_all: the tokens' Q8_0 codes [T][H] and scales [T][H/32] (global
// memory or LDS).  COHERENT_OUT: h codes and scales are written with
// device-scope stores (read by other workgroups of the same kernel).
// PIPE = 2: the loads of the next row pass are issued before the current
// pass's products (two passes of weights in registers); PIPE = 1: after them,
// reusing their registers (the reduction of the current pass overlaps the
// loads), for kernels held to few registers.  hs receives g, and u goes to
// LDS of its own; SwiGLU is evaluated in the Q8_0 step, one lane per row.
template <int BITS, int LPR, int CPL, int NT, int WAVES = 4, bool COHERENT_OUT = false,
          int BLK = 1, int PIPE = 2>
__device__ __forceinline__ void gateup_body(const FfnArgs &a, bool union_mode, const ExpertPtrs &ep,
                                            const TokList &s, int rb, float (*hs)[32 * BLK],
                                            const int8_t *xq_all, const float *xd_all) {
  static_assert(PIPE == 1 || PIPE == 2, "row passes in flight");
  __shared__ __align__(16) int8_t hcode[NT][32 * BLK];
  __shared__ float hu[NT][32 * BLK];
  constexpr int RPP = 64 / LPR;  // rows per pass of a wave
  constexpr int ROWS_PER_WAVE = 32 * BLK / WAVES;
  constexpr int PASSES = ROWS_PER_WAVE / RPP;
  const int H = a.L.H, I = a.L.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % LPR;           // lane in its row group
  const int rsub = lane / LPR;         // row within the pass
  const int nchunks = H * BITS / 128;  // 16-byte chunks per row
  const size_t row_bytes = (size_t)H * BITS / 8;
  const int xblocks = H / 32;

  // lane i < ROWS_PER_WAVE holds the gate/up scales of the wave's i-th row
  const int srow = rb * 32 + wave * ROWS_PER_WAVE + min(lane, ROWS_PER_WAVE - 1);
  const float sgv = ep.sg[srow], suv = ep.su[srow];
  for (int t0 = 0; t0 < s.n_tok; t0 += NT) {
    Act<BITS> act[CPL][NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      int t = 0, hrow = 0, j = 0;
      const bool tv = t0 + tt < s.n_tok;
      if (tv) tok_at(a, union_mode, s, t0 + tt, t, hrow, j);
      const int8_t *xq = xq_all + (size_t)t * H;
      const float *xd = xd_all + (size_t)t * xblocks;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = gl + LPR * i;
        if (tv && c < nchunks) load_act<BITS>(act[i][tt], xq, xd, c);
        else zero_act<BITS>(act[i][tt]);
      }
    }
    uint4 wg[PIPE][CPL], wu[PIPE][CPL];
    // chunks past the row end reload the last chunk; their activations are
    // zero, so they add exactly 0 -- no branch around the loads
    auto load_rows = [&](int p, int buf) {
      const int row = rb * 32 + wave * ROWS_PER_WAVE + p * RPP + rsub;
      const uint4 *gp = reinterpret_cast<const uint4 *>(ep.wg + (size_t)row * row_bytes);
      const uint4 *up = reinterpret_cast<const uint4 *>(ep.wu + (size_t)row * row_bytes);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = min(gl + LPR * i, nchunks - 1);
        wg[buf][i] = ld_nt(gp + c);
        wu[buf][i] = ld_nt(up + c);
      }
    };
    load_rows(0, 0);
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      if (PIPE == 2 && p + 1 < PASSES) load_rows(p + 1, (p + 1) & 1);
      const int buf = PIPE == 2 ? (p & 1) : 0;
      const int rl = wave * ROWS_PER_WAVE + p * RPP + rsub;  // row within the item
      // g and u of the row: block partials in binary64, summed across the
      // row's lanes in binary64, times the row scale, rounded once
      double pg[NT], pu[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        pg[tt] = 0.0;
        pu[tt] = 0.0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          pg[tt] += chunk_part_f64<BITS>(wg[buf][i], act[i][tt]);
          pu[tt] += chunk_part_f64<BITS>(wu[buf][i], act[i][tt]);
        }
      }
      if (PIPE == 1 && p + 1 < PASSES) load_rows(p + 1, 0);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        pg[tt] = group_sum_f64<LPR>(pg[tt]);
        pu[tt] = group_sum_f64<LPR>(pu[tt]);
      }
      const float sg = row_scale<RPP>(sgv, p, rsub), su = row_scale<RPP>(suv, p, rsub);
      if (lane == group_sum_lane<LPR>(lane)) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          hs[tt][rl] = row_out(pg[tt], sg);
          hu[tt][rl] = row_out(pu[tt], su);
        }
      }
    }
    __syncthreads();
    // SwiGLU and Q8_0 of each token's h blocks: thread -> (token tt, block b,
    // element i)
    const int tt = threadIdx.x / (32 * BLK), b = (threadIdx.x >> 5) % BLK, i = threadIdx.x & 31;
    if (tt < NT) {
      const float h = swiglu_h(hs[tt][b * 32 + i], hu[tt][b * 32 + i]);
      float amax = group_max<32>(fabsf(h));
      amax = __shfl(amax, (lane & 32) | 31, 64);
      if (t0 + tt < s.n_tok) {
        int t, hrow, j;
        tok_at(a, union_mode, s, t0 + tt, t, hrow, j);
        const float db = amax / 127.f;
        float c = 0.f;
        if (db != 0.f) c = fminf(fmaxf(rintf(h / db), -127.f), 127.f);
        if constexpr (COHERENT_OUT) {
          hcode[tt][b * 32 + perm_dst<BITS>(i)] = (int8_t)c;
          if (i == 0)
            st_dev(reinterpret_cast<uint32_t *>(a.hd) + (size_t)hrow * (I / 32) + rb + b,
                   __float_as_uint(db));
        } else {
          a.hq[(size_t)hrow * I + (rb + b) * 32 + perm_dst<BITS>(i)] = (int8_t)c;
          if (i == 0) a.hd[(size_t)hrow * (I / 32) + rb + b] = db;
        }
      }
    }
    __syncthreads();
    if constexpr (COHERENT_OUT) {
      // each block's 32 codes as 8 device-scope word stores
      if (tt < NT && i < 8 && t0 + tt < s.n_tok) {
        int t, hrow, j;
        tok_at(a, union_mode, s, t0 + tt, t, hrow, j);
        st_dev(reinterpret_cast<uint32_t *>(a.hq + (size_t)hrow * I + (rb + b) * 32) + i,
               reinterpret_cast<const uint32_t *>(hcode[tt] + b * 32)[i]);
      }
      __syncthreads();
    }
  }
}

}  // namespace coli
