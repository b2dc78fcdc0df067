// decode.hip -- the routed-MoE layer for one token (batch-1 decode) as ONE
// gfx950 kernel.
//
// colibrì README, "Implemented features": a DeepSeek-V3-like sigmoid router
// (noaux_tc, routed_scaling_factor) picks 8 of 256 experts; the shared expert
// always runs; every expert is a SwiGLU FFN over int8 / packed int4 / packed
// int2 weights with per-row scales, dequantised on use against Q8_0-style
// int8 activations.  At batch 1 the layer streams ~176 MB of weights per
// token, so it is bound by HBM; separate kernels for the front, gate/up and
// down phases each pay a launch, ramp-up and drain that one streaming kernel
// pays once.
//
// Work items, in ticket order:
//   L   router logits, four expert rows per item (two waves per row, each
//       summing half of the row in binary64; skipped if logits are given)
//   GS  shared-expert gate/up + SwiGLU + Q8_0(h), kGuRows rows per item
//   GR  routed-expert gate/up, one (slot, kGuRows-row block) per item
//   D   down projection + combine for a block of output rows, all slots in
//       the combine order (shared, then routed 0 .. k-1).
// Item i sits in work queue i % 8; workgroup b serves queue b % 8, taking
// its first item statically (its own index) and later ones from the
// queue's counter, so within a queue items start in ticket order.  GR and D
// items wait for the router scores, D items for the gate/up items of every
// slot.  These waits assume that the grid, sized to what the GPU holds at
// once, becomes resident together, which holds when the kernel has the GPU
// to itself.  If other work holds part of the GPU, a waiting workgroup can
// occupy a slot that the producer of its data needs; then the wait gives up
// after a bounded number of polling rounds (~0.1 s for the scores, ~0.8 s
// for the slots), the call's outputs are undefined, and the give-up is
// recorded in a sticky status word of the workspace header that the caller
// reads (coli_moe_workspace_status).  No wait can hang the GPU.
// GR and D items select the token's experts themselves with their whole
// workgroup (select.hpp): a few microseconds of arithmetic, but no further
// round trip through memory before the expert weights stream.  Every gate/up
// item quantises x into its own LDS (x is an input, so no item has to
// publish it).  Data passed between workgroups (scores, h codes and scales)
// is written and read with relaxed device-scope atomics, coherent across
// XCDs per access; a producer waits for its stores to complete, then bumps
// a counter (relaxed atomic add).  No cache-wide write-back or invalidation
// is needed -- such fences, issued by every workgroup, cost far more than
// the whole layer.  The last workgroup to finish resets the counters, so
// they are zero for the next call; the counters live in the first bytes of
// the workspace, which must be zero before its first use.
#include <algorithm>

#include "actq.hpp"
#include "ffn_common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace coli {

// Workspace header (uint32 words, zero between calls except the status):
//   counters, each on its own 256-byte line so polls and atomic adds on one
//   do not contend with the others: one ticket per work queue, the finished
//   workgroups, and per slot (routed 0 .. k-1, shared k) the finished
//   gate/up items;
//   the status word (sticky: give-ups of bounded waits, never cleared by the
//   kernel) and the polling bound override (test hook: if nonzero at the
//   start of a call, the bound on every wait's polling rounds; cleared by
//   the call);
//   then one 64-bit word per expert from the router: the complemented bits of
//   the biased score c = sigma + bias (low half) and sigma (high half).  Zero
//   means "not written yet", so consumers poll the scores themselves.
constexpr int kCtrStride = 64;  // uint32 words
constexpr int kQueues = 8;      // one work queue per XCD (workgroup b serves queue b % 8)
enum : int {
  kCtrTicket = 0,
  kCtrExit = kQueues * kCtrStride,
  kCtrSlot0 = kCtrExit + kCtrStride,
  kCtrStatus = kCtrSlot0 + (kSelMaxK + 1) * kCtrStride,
  kCtrSpin = kCtrStatus + kCtrStride,
  kScoreWords = 3072
};
static_assert(kCtrSpin + kCtrStride <= kScoreWords, "counters overlap scores");
static_assert((kScoreWords + 2 * kSelMaxE) * 4 <= kDecodeCounterBytes,
              "decode state exceeds the workspace header");
static_assert(kCtrStatus * 4 == COLI_WORKSPACE_STATUS_OFFSET, "status word offset");
static_assert(kCtrSpin * 4 == COLI_WORKSPACE_SPIN_LIMIT_OFFSET, "polling bound offset");
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr uint32_t kSpinLimit = 1u << 19;  // ~100 ms of polling
constexpr int kLogRows = 4;                // logit rows per L item (two waves each)
constexpr int kGuRows = 32;                // gate/up rows per GS/GR item
// cache-policy bits of global_load_lds giving sc1, the policy of the relaxed
// device-scope loads, so staged data is as coherent across XCDs as theirs
constexpr int kLoadSc1 = 16;

struct DecodeArgs {
  FfnArgs f;
  const float *x;        // [H]
  const float *gate_w;   // [E][H], null when logits are supplied
  const float *logits_in;  // [E] supplied logits, or null
  float *logits_out;       // [E] copy of the computed logits for the caller, or null
  uint32_t *ctr;         // workspace header
  int n_log, n_gsh, n_gr, n_down, total;
  int down_rows;         // output rows per D item
  int slot_group;        // slots staged in LDS at a time by a D item
  int lds_main;          // byte offset of the per-role region in dynamic LDS
};

__device__ __forceinline__ uint32_t ld_ctr(const uint32_t *c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave waits until its device-scope stores have completed, then one
// thread adds to the counter.
__device__ __forceinline__ void publish(uint32_t *c, uint32_t v) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polling rounds of a wait: the header's override when it is nonzero (at
// most the default), else `dflt`.
__device__ __forceinline__ uint32_t spin_bound(const DecodeArgs &d, uint32_t dflt) {
  const uint32_t v = ld_ctr(d.ctr + kCtrSpin);
  return v ? min(v, dflt) : dflt;
}

// A bounded wait that ran out of polling rounds: record it (the call's
// outputs are undefined).
__device__ __forceinline__ void gave_up(const DecodeArgs &d, uint32_t what) {
  __hip_atomic_fetch_or(d.ctr + kCtrStatus, what, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// L item: logits of experts e0 .. e0 + kLogRows - 1.  The kWpr waves of a
// row each sum one 1/kWpr part of it in binary64; the parts are added in
// order and the result rounded once to binary32.
__device__ __forceinline__ void logits_rows(const DecodeArgs &d, int e0, double *part) {
  constexpr int kWpr = kDecWaves / kLogRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = wave / kWpr, seg = wave % kWpr;
  const int e = min(e0 + r, d.f.E - 1);  // a row past E recomputes the last row, unused
  const int H = d.f.L.H;
  const int q4 = H / (4 * kWpr);  // float4 per part (H % 32 == 0)
  const float4 *wr = reinterpret_cast<const float4 *>(d.gate_w + (size_t)e * H) + seg * q4;
  const float4 *xr = reinterpret_cast<const float4 *>(d.x) + seg * q4;
  constexpr int kPer = 6;
  double acc = 0.0;
  for (int c0 = 0; c0 < q4; c0 += 64 * kPer) {
    float4 wv[kPer], xv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = min(c0 + lane + 64 * i, q4 - 1);
      wv[i] = wr[c];
      xv[i] = xr[c];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (c0 + lane + 64 * i < q4) {
        acc = fma((double)xv[i].x, (double)wv[i].x, acc);
        acc = fma((double)xv[i].y, (double)wv[i].y, acc);
        acc = fma((double)xv[i].z, (double)wv[i].z, acc);
        acc = fma((double)xv[i].w, (double)wv[i].w, acc);
      }
    }
  }
  const double s = wave_sum_f64(acc);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if ((int)threadIdx.x < kLogRows && e0 + (int)threadIdx.x < d.f.E) {
    const int e = e0 + threadIdx.x;
    const double *p = part + kWpr * threadIdx.x;
    double sum = p[0];
#pragma unroll
    for (int i = 1; i < kWpr; ++i) sum += p[i];
    float l = (float)sum;
    if (d.f.loff) l += d.f.loff[e];
    const float sg = sigmoid_f64(l);
    const float c = sg + (d.f.bias ? d.f.bias[e] : 0.f);
    const uint64_t w = ((uint64_t)__float_as_uint(sg) << 32) | (uint64_t)(~__float_as_uint(c));
    __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + e, w, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (d.logits_out) d.logits_out[e] = l;
  }
}

// The token's experts and weights into LDS (sidx, sw), from the router's
// scores: polled in the header until every expert's word has been written
// (bounded: a lost word leaves garbage, never a hang), or computed here from
// supplied logits.  `scratch` holds a SelInput followed by the selection's
// own scratch.
__device__ __forceinline__ void select_local(const DecodeArgs &d, unsigned char *scratch,
                                             int32_t *sidx, float *sw) {
  const RouterCfg &cfg = d.f.cfg;
  SelInput &in = *reinterpret_cast<SelInput *>(scratch);
  unsigned char *sel = scratch + sizeof(SelInput);
  for (int e = threadIdx.x; e < cfg.E; e += kDecThreads) {
    if (d.logits_in) {
      const float sg = sigmoid_f64(d.logits_in[e]);
      in.sg[e] = sg;
      in.c[e] = sg + (d.f.bias ? d.f.bias[e] : 0.f);
    } else {
      const uint64_t *w = reinterpret_cast<const uint64_t *>(d.ctr + kScoreWords) + e;
      uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t spin = spin_bound(d, kSpinLimit);
      uint32_t it = 0;
      while ((uint32_t)v == 0u && it < spin) {
        __builtin_amdgcn_s_sleep(2);
        v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ++it;
      }
      if ((uint32_t)v == 0u) gave_up(d, COLI_WAIT_SCORES);
      in.c[e] = __uint_as_float(~(uint32_t)v);
      in.sg[e] = __uint_as_float((uint32_t)(v >> 32));
    }
  }
  __syncthreads();
  if (select_fast_ok(cfg.E, cfg.n_group, cfg.topk_group, cfg.k, kDecThreads))
    select_fast<kDecThreads>(cfg, in, *reinterpret_cast<SelFastScratch *>(sel), sidx, sw);
  else
    select_wg<kDecThreads>(cfg, in, *reinterpret_cast<SelWgScratch *>(sel), sidx, sw);
  for (int j = threadIdx.x; j < d.f.k; j += kDecThreads)
    if ((unsigned)sidx[j] >= (unsigned)d.f.E) sidx[j] = -1;  // never index outside the experts
  __syncthreads();
}

// D item: output rows [r0, r0 + down_rows).  Wave w owns rows
// r0 + w*PR .. r0 + w*PR + PR-1 (PR = NPASS * RPP) for every slot, so it
// combines y = o_shared + sum_j w_j * o_j itself: each lane accumulates its
// chunks' share of every slot (shared first, then slots 0 .. k-1), and the
// lanes of a row are summed once at the end -- a fixed order, so the result
// is reproducible.
template <int BITS, int LPR, int CPL, int NPASS, int SG>
__device__ __forceinline__ void down_rows(const DecodeArgs &d, int r0, int8_t *lds_q, float *lds_d,
                                          const int32_t *sidx, const float *sw) {
  constexpr int RPP = 64 / LPR;
  const FfnArgs &a = d.f;
  const int I = a.L.I, k = a.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % LPR, rsub = lane / LPR;
  const int nchunks = I * BITS / 128;
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int nslots = k + 1;
  const int wrow0 = r0 + wave * NPASS * RPP;
  float y[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) y[p] = 0.f;

  // slot order: shared (k), then routed 0 .. k-1
  for (int g0 = 0; g0 < nslots; g0 += d.slot_group) {
    const int gn = min(d.slot_group, nslots - g0);
    uint4 wv[SG][NPASS][CPL];
    float sdv[SG][NPASS];
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const int sl = g0 + q == 0 ? k : g0 + q - 1;
      const int e = (q >= gn || sl == k) ? -1 : uniform_i32(sidx[sl]);
      if (q < gn && (sl == k || e >= 0)) {
        const ExpertPtrs ep = expert_ptrs(a.L, e);
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          const int row = wrow0 + p * RPP + rsub;
          const uint4 *wp = reinterpret_cast<const uint4 *>(ep.wd + (size_t)row * row_bytes);
#pragma unroll
          for (int i = 0; i < CPL; ++i) wv[q][p][i] = ld_nt(wp + min(gl + LPR * i, nchunks - 1));
          sdv[q][p] = ep.sd[row];
        }
      }
    }
    // once every gate/up item of the group's slots is done, stage their h
    // codes and scales in LDS (device-scope loads, all in flight together)
    if ((int)threadIdx.x < gn) {
      const int q = threadIdx.x;
      const int sl = g0 + q == 0 ? k : g0 + q - 1;
      const uint32_t *c = d.ctr + kCtrSlot0 + sl * kCtrStride;
      const uint32_t spin = spin_bound(d, 8u * kSpinLimit);
      uint32_t it = 0, v;
      while ((v = ld_ctr(c)) < (uint32_t)(I / kGuRows) && it < spin) {
        __builtin_amdgcn_s_sleep(8);
        ++it;
      }
      if (v < (uint32_t)(I / kGuRows)) gave_up(d, COLI_WAIT_SLOTS);
    }
    __syncthreads();
    if (I % 128 == 0) {
      // straight into LDS: 16-byte loads with the cache policy of the
      // device-scope loads (sc1), all in flight at once and no registers.
      // One wave instruction fills 64 consecutive 16-byte LDS chunks.
      const int cq = I / 16, cd = I / 128;  // chunks of codes / of scales per slot
      const int nA = gn * cq, nB = gn * cd;
      const int nwA = (nA + 63) / 64, nwB = (nB + 63) / 64;
      for (int ii = wave; ii < nwA + nwB; ii += kDecWaves) {
        const bool codes = ii < nwA;
        const int base = (codes ? ii : ii - nwA) * 64;
        const int c = base + lane, per = codes ? cq : cd;
        unsigned char *dst = (codes ? reinterpret_cast<unsigned char *>(lds_q)
                                    : reinterpret_cast<unsigned char *>(lds_d)) + (size_t)base * 16;
        if (c < (codes ? nA : nB)) {
          const int q = c / per, r = c - q * per;
          const int sl = g0 + q == 0 ? k : g0 + q - 1;
          const unsigned char *src =
              codes ? reinterpret_cast<const unsigned char *>(a.hq) + (size_t)sl * I + r * 16
                    : reinterpret_cast<const unsigned char *>(a.hd) + (size_t)sl * (I / 8) + r * 16;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0,
                                           kLoadSc1);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      // 64-bit device-scope loads, kStage per thread issued before any is
      // written to LDS
      constexpr int kStage = 2;
      const int wq = I / 8, wd = I / 64;  // 8-byte words of codes and scales per slot
      const int n = gn * (wq + wd);
      for (int i0 = 0; i0 < n; i0 += kStage * kDecThreads) {
        uint64_t v[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
          const int i = i0 + j * kDecThreads + threadIdx.x;
          v[j] = 0;
          if (i < n) {
            const int q = i / (wq + wd), r = i - q * (wq + wd);
            const int sl = g0 + q == 0 ? k : g0 + q - 1;
            const uint64_t *src = r < wq ? reinterpret_cast<const uint64_t *>(a.hq + (size_t)sl * I) + r
                                         : reinterpret_cast<const uint64_t *>(a.hd + (size_t)sl * (I / 32)) + (r - wq);
            v[j] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
          const int i = i0 + j * kDecThreads + threadIdx.x;
          if (i < n) {
            const int q = i / (wq + wd), r = i - q * (wq + wd);
            uint64_t *dst = r < wq ? reinterpret_cast<uint64_t *>(lds_q + (size_t)q * I) + r
                                   : reinterpret_cast<uint64_t *>(lds_d + q * (I / 32)) + (r - wq);
            *dst = v[j];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      const int sl = g0 + q == 0 ? k : g0 + q - 1;
      const bool shared = sl == k;
      if (q < gn && (shared || uniform_i32(sidx[sl]) >= 0)) {
        const float wgt = shared ? 1.f : sw[sl];
        Act<BITS> act[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = gl + LPR * i;
          if (c < nchunks) load_act<BITS>(act[i], lds_q + (size_t)q * I, lds_d + q * (I / 32), c);
          else zero_act<BITS>(act[i]);
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) acc += chunk_part<BITS>(wv[q][p][i], act[i]);
          // each lane's share of w_j * s_j * o_j; the lanes of a row are
          // summed once, after the last slot
          y[p] += (shared ? sdv[q][p] : wgt * sdv[q][p]) * acc;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const float yr = group_sum<LPR>(y[p]);
    if (lane == group_sum_lane<LPR>(lane)) a.y[wrow0 + p * RPP + rsub] = yr;
  }
}

// Persistent: the grid is at most the workgroups the GPU holds at once;
// each workgroup takes tickets until none are left.  x's Q8_0 codes and the
// selection are computed once per workgroup and reused by its later items
// (tickets only increase, so a workgroup never returns to gate/up work
// after a D item, whose staging overwrites x's codes).
template <int BITS, int GLPR, int GCPL, int DLPR, int DCPL>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(BITS == 4 ? 4 : 1))) void k_decode_fused(DecodeArgs d) {
  constexpr int DNPASS = DCPL == 1 ? 2 : 1;
  constexpr int DSG = DCPL == 1 ? 9 : 3;
  constexpr int BLK = kGuRows / 32;
  __shared__ int32_t sidx[kSelMaxK];
  __shared__ float sw[kSelMaxK];
  __shared__ float hs[1][kGuRows];
  __shared__ double lpart[kDecWaves];
  __shared__ int s_ticket;
  // dynamic LDS: [selection scratch | x's Q8_0 codes and scales]; a D item's
  // staged h overlays both once the selection is done
  extern __shared__ __align__(16) unsigned char dyn[];
  unsigned char *lds_x = dyn + d.lds_main;
  const FfnArgs &a = d.f;
  const int k = a.k, I = a.L.I, H = a.L.H;
  const int n_rb = I / kGuRows;
  const int b_gsh = d.n_log, b_gr = b_gsh + d.n_gsh, b_down = b_gr + d.n_gr;
  int8_t *xq_lds = reinterpret_cast<int8_t *>(lds_x);
  float *xd_lds = reinterpret_cast<float *>(lds_x + H);

  // Tickets only increase, so the items of each kind form one loop of their
  // own (this keeps each kind's registers apart).
  // Work queue q = b % 8 holds items q, q + 8, ...; consecutive workgroups
  // go to consecutive XCDs, so each XCD streams an equal share of every
  // kind of item.  Within a queue the items keep their global order.
  // A workgroup's first item is its own index (queue q's nq workgroups take
  // its first nq items in order), which saves the first atomic round trip;
  // later tickets come from the queue's counter, offset by nq.
  const int q = blockIdx.x % kQueues;
  const int nq = ((int)gridDim.x - q + kQueues - 1) / kQueues;
  auto next_ticket = [&]() -> int {
    if (threadIdx.x == 0)
      s_ticket = (int)__hip_atomic_fetch_add(d.ctr + kCtrTicket + q * kCtrStride, 1u,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = q + kQueues * (nq + uniform_i32(s_ticket));
    __syncthreads();
    return t;
  };
  int t = (int)blockIdx.x;

  // L: four logit rows per item
  for (; t < b_gsh; t = next_ticket()) {
    logits_rows(d, t * kLogRows, lpart);
    __syncthreads();
  }
  if (t < b_down) {
    // gate/up items: x's Q8_0 codes, once
    for (int i = threadIdx.x; i < H / 32; i += kDecThreads)
      act_quant_block<BITS>(d.x + i * 32, xq_lds + i * 32, xd_lds + i);
    __syncthreads();
  }
  // GS: shared expert, rows [kGuRows (t - b_gsh), +kGuRows)
  for (; t < b_gr; t = next_ticket()) {
    TokList s{1, -1, k, true};
    gateup_body<BITS, GLPR, GCPL, 1, kDecWaves, true, BLK>(a, false, expert_ptrs(a.L, -1), s,
                                                          BLK * (t - b_gsh), hs, xq_lds, xd_lds);
    publish(d.ctr + kCtrSlot0 + k * kCtrStride, 1u);
  }
  // routed gate/up and down items: the token's experts, once
  if (t < d.total) select_local(d, dyn, sidx, sw);
  // GR: routed slot u, rows [kGuRows rb, +kGuRows)
  for (; t < b_down; t = next_ticket()) {
    const int u = (t - b_gr) / n_rb, rb = (t - b_gr) % n_rb;
    if (u == 0 && rb == 0) {
      for (int j = threadIdx.x; j < k; j += kDecThreads) {
        if (a.idx_user) a.idx_user[j] = sidx[j];
        if (a.w_user) a.w_user[j] = sw[j];
      }
    }
    const int e = uniform_i32(sidx[u]);
    if (e >= 0) {
      TokList s{1, -1, u, false};
      gateup_body<BITS, GLPR, GCPL, 1, kDecWaves, true, BLK>(a, false, expert_ptrs(a.L, e), s,
                                                            BLK * rb, hs, xq_lds, xd_lds);
    }
    publish(d.ctr + kCtrSlot0 + u * kCtrStride, 1u);
  }
  // D: output rows; the staged h overwrites x's codes
  for (; t < d.total; t = next_ticket()) {
    int8_t *lds_q = reinterpret_cast<int8_t *>(dyn);
    float *lds_d = reinterpret_cast<float *>(dyn + (size_t)d.slot_group * I);
    down_rows<BITS, DLPR, DCPL, DNPASS, DSG>(d, (t - b_down) * d.down_rows, lds_q, lds_d, sidx, sw);
  }

  // the last workgroup out clears the header for the next call
  __syncthreads();
  if (threadIdx.x == 0)
    s_ticket = (int)__hip_atomic_fetch_add(d.ctr + kCtrExit, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (uniform_i32(s_ticket) == (int)gridDim.x - 1) {
    const int nc = kCtrSlot0 / kCtrStride + k + 1;
    for (int i = threadIdx.x; i < nc; i += kDecThreads)
      __hip_atomic_store(d.ctr + i * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0)
      __hip_atomic_store(d.ctr + kCtrSpin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d.n_log > 0)
      for (int e = threadIdx.x; e < a.E; e += kDecThreads)
        __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + e, (uint64_t)0,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static int dec_lpr(int nchunks) { return (nchunks % 64 != 0 && nchunks % 32 == 0) ? 32 : 64; }

static int dec_cpl(int nchunks, int lpr) {
  const int c = (nchunks + lpr - 1) / lpr;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 3 ? 3 : c <= 4 ? 4 : c <= 6 ? 6 : c <= 8 ? 8 : -1;
}

template <int BITS, int GLPR, int GCPL, int DLPR, int DCPL>
static hipError_t launch_fused_t(DecodeArgs d, hipStream_t st, KEvents ev) {
  constexpr int DNPASS = DCPL == 1 ? 2 : 1;
  constexpr int DSG = DCPL == 1 ? 9 : 3;
  const int I = d.f.L.I;
  d.down_rows = kDecWaves * DNPASS * (64 / DLPR);
  if (d.f.L.H % d.down_rows) return hipErrorNotSupported;
  d.n_down = d.f.L.H / d.down_rows;
  // dynamic LDS: the selection scratch, then the larger of x's Q8_0 codes
  // and scales and the D items' staged h (I code bytes + I/32 scales a slot)
  const int per_slot = I + (I / 32) * 4;
  d.slot_group = DSG;
  while (d.slot_group > 1 && d.slot_group * per_slot > 24 * 1024) --d.slot_group;
  d.total = d.n_log + d.n_gsh + d.n_gr + d.n_down;
  d.lds_main =
      (int)((sizeof(SelInput) + std::max(sizeof(SelWgScratch), sizeof(SelFastScratch)) + 15) / 16 * 16);
  const size_t shmem = std::max((size_t)d.slot_group * per_slot,
                                (size_t)d.lds_main + (size_t)d.f.L.H + (size_t)(d.f.L.H / 32) * 4);
  // as many workgroups as the GPU holds at once (never more than the items)
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(&k_decode_fused<BITS, GLPR, GCPL, DLPR, DCPL>),
          kDecThreads, shmem) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  // every queue that holds an item has a workgroup (grid >= min(total, 8))
  const int grid = std::min(d.total, std::max(per_cu * n_cu, kQueues));
  COLI_LAUNCH(ev, (k_decode_fused<BITS, GLPR, GCPL, DLPR, DCPL>), dim3(grid), dim3(kDecThreads),
              shmem, st, d);
  return hipGetLastError();
}

// The single-kernel decode is built for the row shapes below (gate/up lanes
// per row x chunks per lane, down likewise): the GLM-5.2 layer (H 6144,
// I 2048) in each container, and one-chunk rows (H, I <= 1024 at int8).
// Other shapes return hipErrorNotSupported and take the multi-kernel decode.
template <int BITS>
static hipError_t launch_fused_bits(DecodeArgs d, hipStream_t st, KEvents ev) {
  const int gn = d.f.L.H * BITS / 128, dn = d.f.L.I * BITS / 128;
  const int gl = dec_lpr(gn), gc = dec_cpl(gn, gl), dl = dec_lpr(dn), dc = dec_cpl(dn, dl);
#define COLI_DEC_CASE(GL, GC, DL, DC) \
  if (gl == GL && gc == GC && dl == DL && dc == DC) return launch_fused_t<BITS, GL, GC, DL, DC>(d, st, ev);
  COLI_DEC_CASE(64, 1, 64, 1)
  if constexpr (BITS == 8) { COLI_DEC_CASE(64, 6, 64, 2) }
  if constexpr (BITS == 4) { COLI_DEC_CASE(64, 3, 64, 1) }
  if constexpr (BITS == 2) { COLI_DEC_CASE(32, 3, 32, 1) }
#undef COLI_DEC_CASE
  return hipErrorNotSupported;
}

// The header's status word into *out, cleared afterwards when `clear`.
__global__ void k_workspace_status(uint32_t *ctr, int32_t *out, int clear) {
  if (threadIdx.x == 0) {
    const uint32_t v = clear ? __hip_atomic_exchange(ctr + kCtrStatus, 0u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                             : ld_ctr(ctr + kCtrStatus);
    *out = (int32_t)v;
  }
}

hipError_t launch_workspace_status(uint32_t *ctr, int32_t *out, int clear, hipStream_t st) {
  hipLaunchKernelGGL(k_workspace_status, dim3(1), dim3(64), 0, st, ctr, out, clear);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const FfnArgs &f, const float *x, const float *gate_w,
                               const float *logits_in, float *logits_out, uint32_t *ctr,
                               hipStream_t st, KEvents ev) {
  DecodeArgs d{};
  d.f = f;
  d.x = x;
  d.gate_w = gate_w;
  d.logits_in = gate_w ? nullptr : logits_in;
  d.logits_out = gate_w ? logits_out : nullptr;
  d.ctr = ctr;
  d.n_log = gate_w ? (f.E + kLogRows - 1) / kLogRows : 0;
  d.n_gsh = f.L.I / kGuRows;
  d.n_gr = f.k * (f.L.I / kGuRows);
  if (f.L.I % kGuRows) return hipErrorNotSupported;
  switch (f.L.bits) {
    case 8: return launch_fused_bits<8>(d, st, ev);
    case 4: return launch_fused_bits<4>(d, st, ev);
    case 2: return launch_fused_bits<2>(d, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace coli
