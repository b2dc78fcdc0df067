// cache.hip -- tiered expert residency: per-layer HBM slots over a host tier
// in pinned host memory.  The pages keep a per-layer LRU cache of routed
// experts with an optional pinned store of the hot ones in front of the slow
// tier they stream experts from (colibrì README, "Idea"; CSDN feature,
// "把内存、显存和磁盘当成同一块蛋糕"), and pick the pinned set from the usage
// they record (labhub post, "让它变得可以忍受的那些装置").
//
// Three kernels, all enqueued after routing with no host round trip:
//   k_cache_init  -- empties a cache's state;
//   k_cache_plan  -- one workgroup: marks hits, ranks the misses, picks the
//                    LRU victims among unpinned slots, updates the state in
//                    LDS and writes it back with the list of copies (for one
//                    token, k_cache_route_plan also selects the experts from
//                    the logits in the same launch);
//   k_cache_fill  -- one workgroup per CU: copies the listed experts' bytes
//                    from the host tier into their slots in 64 KiB chunks
//                    (the host link bounds it; sixteen 16-byte loads of host
//                    memory per lane are in flight at once).
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "select.hpp"

namespace coli {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kMaxCacheE = 1024;
constexpr int kFillThreads = 256;
constexpr int kFillPerLane = 16;  // uint4 per lane per chunk
constexpr size_t kFillChunk = (size_t)kFillThreads * kFillPerLane * 16;  // 64 KiB

__global__ __launch_bounds__(256) void k_cache_init(CacheState c) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kCacheCtlWords) c.ctl[i] = 0u;
  if (i < c.E) {
    c.slot_of[i] = -1;
    c.use_count[i] = 0u;
  }
  if (i < c.S) {
    c.expert_of[i] = -1;
    c.last_use[i] = 0u;
    c.pinned[i] = 0u;
    c.copy_list[2 * i] = -1;
    c.copy_list[2 * i + 1] = -1;
  }
}

// Exclusive prefix sum of v over the workgroup (kPlanThreads lanes); *total
// receives the sum.  Shuffle scan inside each wave, then the wave totals.
__device__ int wg_exclusive_scan(int v, int *wave_tot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const int t = wave_tot[w];
    base += w < wave ? t : 0;
    all += t;
  }
  *total = all;
  return base + incl - v;
}

// LDS image of a cache's state plus the set one call needs.
struct PlanLds {
  int slot_of[kMaxCacheE], expert_of[kMaxCacheE], need[kMaxCacheE];
  int mrank[kMaxCacheE], victim[kMaxCacheE];
  uint32_t last[kMaxCacheE], pin[kMaxCacheE], use[kMaxCacheE];
  int wave_tot[kPlanThreads / 64];
  int hits, nelig;
};

// Loads the state into LDS (words outside their ranges -- a state never
// initialised -- read as absent / empty, so every LDS index stays in bounds)
// and clears the need set.  Ends with a barrier.
__device__ void plan_load(const CacheState &c, PlanLds &p, bool repin) {
  const int t = threadIdx.x, E = c.E, S = c.S;
  for (int i = t; i < E; i += kPlanThreads) {
    const int sl = c.slot_of[i];
    p.slot_of[i] = (sl >= 0 && sl < S) ? sl : -1;
    p.need[i] = 0;
    p.use[i] = c.use_count[i];
  }
  for (int i = t; i < S; i += kPlanThreads) {
    const int ex = c.expert_of[i];
    p.expert_of[i] = (ex >= 0 && ex < E) ? ex : -1;
    p.last[i] = c.last_use[i];
    p.pin[i] = repin ? 0u : c.pinned[i];
  }
  if (t == 0) {
    p.hits = 0;
    p.nelig = 0;
  }
  __syncthreads();
}

// The replacement once p.need holds the call's set (pair counts, or 1 for
// a repin's chosen experts): hits touch their slots, misses take the LRU
// unpinned slots this call does not use, the state and the copy list are
// written back.  Called by the whole workgroup after a barrier.
__device__ void plan_core(const CacheState &c, PlanLds &p, bool repin) {
  const int t = threadIdx.x, E = c.E, S = c.S;
  const uint32_t clock = c.ctl[0] + 1u;

  // hits: touch their slots; usage learned from the routed pairs
  int hits = 0;
  for (int e = t; e < E; e += kPlanThreads) {
    const int n = p.need[e];
    if (!n) continue;
    if (!repin) c.use_count[e] = p.use[e] + (uint32_t)n;
    const int sl = p.slot_of[e];
    if (sl >= 0) {
      p.last[sl] = clock;
      ++hits;
    }
  }
  if (hits) atomicAdd(&p.hits, hits);
  __syncthreads();

  // misses ranked in increasing expert order (each lane scans a contiguous run)
  const int per = (E + kPlanThreads - 1) / kPlanThreads;
  const int e0 = t * per, e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (p.need[e] && p.slot_of[e] < 0);
  int n_miss = 0;
  int r = wg_exclusive_scan(local, p.wave_tot, &n_miss);
  for (int e = e0; e < e1; ++e) p.mrank[e] = (p.need[e] && p.slot_of[e] < 0) ? r++ : -1;

  // victims: unpinned slots not used by this call, in (last_use, slot) order
  if (n_miss > 0) {
    for (int s = t; s < S; s += kPlanThreads) {
      const bool el = !p.pin[s] && p.last[s] < clock;
      if (!el) continue;
      atomicAdd(&p.nelig, 1);
      const uint32_t ls = p.last[s];
      int rank = 0;
      for (int s2 = 0; s2 < S; ++s2) {
        const uint32_t l2 = p.last[s2];
        rank += (!p.pin[s2] && l2 < clock) && (l2 < ls || (l2 == ls && s2 < s));
      }
      if (rank < n_miss) p.victim[rank] = s;
    }
  }
  __syncthreads();
  const int n_copy = min(n_miss, p.nelig);

  // move the misses in; evicted experts become absent
  for (int e = t; e < E; e += kPlanThreads) {
    const int m = p.mrank[e];
    if (m < 0 || m >= n_copy) continue;
    const int s = p.victim[m];
    const int old = p.expert_of[s];
    if (old >= 0) p.slot_of[old] = -1;
    p.slot_of[e] = s;
    p.expert_of[s] = e;
    p.last[s] = clock;
    c.copy_list[2 * m] = e;
    c.copy_list[2 * m + 1] = s;
  }
  __syncthreads();
  if (repin) {
    for (int e = t; e < E; e += kPlanThreads)
      if (p.need[e] && p.slot_of[e] >= 0) p.pin[p.slot_of[e]] = 1u;
    __syncthreads();
  }

  for (int i = t; i < E; i += kPlanThreads) c.slot_of[i] = p.slot_of[i];
  for (int i = t; i < S; i += kPlanThreads) {
    c.expert_of[i] = p.expert_of[i];
    c.last_use[i] = p.last[i];
    c.pinned[i] = p.pin[i];
  }
  if (t == 0) {
    c.ctl[0] = clock;
    c.ctl[1] = (uint32_t)n_copy;
    if (n_miss > n_copy) c.ctl[2] |= 1u;
    if (!repin) {
      unsigned long long *st = reinterpret_cast<unsigned long long *>(c.ctl + 4);
      st[0] += (unsigned long long)p.hits;
      st[1] += (unsigned long long)n_miss;
    }
  }
}

// repin < 0: a forward call's update from idx[0..n_pairs-1];
// repin >= 0: pin the `repin` most-used experts, ranked by (use_count
// desc, expert asc).
__global__ __launch_bounds__(kPlanThreads) void k_cache_plan(CacheState c, const int32_t *idx,
                                                             int n_pairs, int repin) {
  __shared__ PlanLds p;
  const int t = threadIdx.x, E = c.E;
  plan_load(c, p, repin >= 0);
  if (repin < 0) {
    for (int i = t; i < n_pairs; i += kPlanThreads) {
      const int e = idx[i];
      if (e >= 0 && e < E) atomicAdd(&p.need[e], 1);
    }
  } else {
    for (int e = t; e < E; e += kPlanThreads) {
      const uint32_t u = p.use[e];
      int r = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const uint32_t u2 = p.use[e2];
        r += (u2 > u) || (u2 == u && e2 < e);
      }
      p.need[e] = r < repin ? 1 : 0;
    }
  }
  __syncthreads();
  plan_core(c, p, repin >= 0);
}

// One token: its routing from the logits (the same selection, bit for bit,
// as every other path of the library) and the cache update in one launch.
__global__ __launch_bounds__(kPlanThreads) void k_cache_route_plan(RouterCfg cfg,
                                                                   const float *__restrict__ logits,
                                                                   const float *__restrict__ bias,
                                                                   CacheState c) {
  __shared__ PlanLds p;
  __shared__ SelInput in;
  __shared__ union {
    SelFastScratch fast;
    SelWgScratch wg;
  } sel;
  __shared__ int32_t sidx[kSelMaxK];
  __shared__ float sw[kSelMaxK];
  const int t = threadIdx.x, E = cfg.E;
  for (int e = t; e < E; e += kPlanThreads) {
    const float sg = sigmoid_f64(logits[e]);
    in.sg[e] = sg;
    in.c[e] = sg + (bias ? bias[e] : 0.f);
  }
  plan_load(c, p, false);  // ends with a barrier
  if (select_fast_ok(E, cfg.n_group, cfg.topk_group, cfg.k, kPlanThreads))
    select_fast<kPlanThreads>(cfg, in, sel.fast, sidx, sw);
  else
    select_wg<kPlanThreads>(cfg, in, sel.wg, sidx, sw);
  if (t < cfg.k) {
    const int e = sidx[t];
    if (e >= 0 && e < E) atomicAdd(&p.need[e], 1);
  }
  __syncthreads();
  plan_core(c, p, false);
}

// One expert's six tensors, in the order the chunks walk them.
struct Seg {
  const uint8_t *src;
  uint8_t *dst;
  size_t bytes;
};

__device__ __forceinline__ Seg fill_seg(const CacheTier &t, int e, int s, int which) {
  switch (which) {
    case 0: return {t.hw_gate + (size_t)e * t.gu_bytes, t.dw_gate + (size_t)s * t.gu_bytes, t.gu_bytes};
    case 1: return {t.hw_up + (size_t)e * t.gu_bytes, t.dw_up + (size_t)s * t.gu_bytes, t.gu_bytes};
    case 2: return {t.hw_down + (size_t)e * t.d_bytes, t.dw_down + (size_t)s * t.d_bytes, t.d_bytes};
    case 3:
      return {reinterpret_cast<const uint8_t *>(t.hs_gate + (size_t)e * t.I),
              reinterpret_cast<uint8_t *>(t.ds_gate + (size_t)s * t.I), (size_t)t.I * 4};
    case 4:
      return {reinterpret_cast<const uint8_t *>(t.hs_up + (size_t)e * t.I),
              reinterpret_cast<uint8_t *>(t.ds_up + (size_t)s * t.I), (size_t)t.I * 4};
    default:
      return {reinterpret_cast<const uint8_t *>(t.hs_down + (size_t)e * t.H),
              reinterpret_cast<uint8_t *>(t.ds_down + (size_t)s * t.H), (size_t)t.H * 4};
  }
}

__global__ __launch_bounds__(kFillThreads) void k_cache_fill(CacheState c, CacheTier t) {
  const int n = min((int)c.ctl[1], c.S);
  if (n <= 0) return;
  // chunks per segment and per expert
  size_t nch[6];
  size_t per = 0;
#pragma unroll
  for (int w = 0; w < 6; ++w) {
    const size_t b = w < 2 ? t.gu_bytes : w == 2 ? t.d_bytes : w < 5 ? (size_t)t.I * 4 : (size_t)t.H * 4;
    nch[w] = (b + kFillChunk - 1) / kFillChunk;
    per += nch[w];
  }
  const size_t total = (size_t)n * per;
  for (size_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int ci = (int)(u / per);
    size_t r = u - (size_t)ci * per;
    const int e = c.copy_list[2 * ci], s = c.copy_list[2 * ci + 1];
    if (e < 0 || e >= c.E || s < 0 || s >= c.S) continue;
    int w = 0;
    while (w < 5 && r >= nch[w]) r -= nch[w++];
    const Seg g = fill_seg(t, e, s, w);
    const size_t base = r * kFillChunk;
    uint4 v[kFillPerLane];
#pragma unroll
    for (int j = 0; j < kFillPerLane; ++j) {
      const size_t o = base + ((size_t)j * kFillThreads + threadIdx.x) * 16;
      if (o < g.bytes) v[j] = *reinterpret_cast<const uint4 *>(g.src + o);
    }
#pragma unroll
    for (int j = 0; j < kFillPerLane; ++j) {
      const size_t o = base + ((size_t)j * kFillThreads + threadIdx.x) * 16;
      if (o < g.bytes) {
        const u32x4 q = {v[j].x, v[j].y, v[j].z, v[j].w};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(g.dst + o));
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_init(const CacheState &c, hipStream_t st) {
  const int n = max(max(c.E, c.S), kCacheCtlWords);
  hipLaunchKernelGGL(k_cache_init, dim3((n + 255) / 256), dim3(256), 0, st, c);
  return hipGetLastError();
}

hipError_t launch_cache_plan(const CacheState &c, const int32_t *idx, int n_pairs, int repin,
                             hipStream_t st) {
  if (c.E < 1 || c.E > kMaxCacheE || c.S < 1 || c.S > c.E) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_plan, dim3(1), dim3(kPlanThreads), 0, st, c, idx, n_pairs, repin);
  return hipGetLastError();
}

hipError_t launch_cache_route_plan(const RouterCfg &cfg, const float *logits, const float *bias,
                                   const CacheState &c, hipStream_t st) {
  if (c.E < 1 || c.E > kMaxCacheE || c.S < 1 || c.S > c.E || cfg.E != c.E || cfg.k > kSelMaxK)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_route_plan, dim3(1), dim3(kPlanThreads), 0, st, cfg, logits, bias, c);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheState &c, const CacheTier &t, hipStream_t st) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  hipLaunchKernelGGL(k_cache_fill, dim3(n_cu), dim3(kFillThreads), 0, st, c, t);
  return hipGetLastError();
}

}  // namespace coli
