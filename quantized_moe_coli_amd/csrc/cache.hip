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
//                    LDS and writes it back with the list of copies;
//   k_cache_fill  -- every workgroup: copies the listed experts' bytes from
//                    the host tier into their slots in 32 KiB chunks (the
//                    host link bounds it; loads of host memory issued eight
//                    per lane so that many requests are in flight).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace coli {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kMaxCacheE = 1024;
constexpr int kFillThreads = 256;
constexpr int kFillPerLane = 8;  // uint4 per lane per chunk
constexpr size_t kFillChunk = (size_t)kFillThreads * kFillPerLane * 16;  // 32 KiB

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
// receives the sum.  Hillis-Steele over LDS.
__device__ int wg_exclusive_scan(int v, int *buf, int *total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {
    const int add = t >= d ? buf[t - d] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const int incl = buf[t];
  *total = buf[kPlanThreads - 1];
  __syncthreads();
  return incl - v;
}

// repin < 0: a forward call's update from idx[0..n_pairs-1];
// repin >= 0: pin the `repin` most-used experts.
__global__ __launch_bounds__(kPlanThreads) void k_cache_plan(CacheState c, const int32_t *idx,
                                                             int n_pairs, int repin) {
  __shared__ int s_slot_of[kMaxCacheE], s_expert_of[kMaxCacheE], s_need[kMaxCacheE];
  __shared__ int s_mrank[kMaxCacheE], s_victim[kMaxCacheE];
  __shared__ uint32_t s_last[kMaxCacheE], s_pin[kMaxCacheE], s_use[kMaxCacheE];
  __shared__ int s_scan[kPlanThreads];
  __shared__ int s_hits, s_nelig;
  const int t = threadIdx.x, E = c.E, S = c.S;
  const uint32_t clock = c.ctl[0] + 1u;
  // state words outside their ranges (a state never initialised) read as
  // absent / empty, so every LDS index below stays in bounds
  for (int i = t; i < E; i += kPlanThreads) {
    const int sl = c.slot_of[i];
    s_slot_of[i] = (sl >= 0 && sl < S) ? sl : -1;
    s_need[i] = 0;
    s_use[i] = c.use_count[i];
  }
  for (int i = t; i < S; i += kPlanThreads) {
    const int ex = c.expert_of[i];
    s_expert_of[i] = (ex >= 0 && ex < E) ? ex : -1;
    s_last[i] = c.last_use[i];
    s_pin[i] = repin >= 0 ? 0u : c.pinned[i];
  }
  if (t == 0) {
    s_hits = 0;
    s_nelig = 0;
  }
  __syncthreads();

  // the set this call needs: selected experts (with their pair counts), or
  // the `repin` most-used ones, ranked by (use_count desc, expert asc)
  if (repin < 0) {
    for (int i = t; i < n_pairs; i += kPlanThreads) {
      const int e = idx[i];
      if (e >= 0 && e < E) atomicAdd(&s_need[e], 1);
    }
  } else {
    for (int e = t; e < E; e += kPlanThreads) {
      const uint32_t u = s_use[e];
      int r = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const uint32_t u2 = s_use[e2];
        r += (u2 > u) || (u2 == u && e2 < e);
      }
      s_need[e] = r < repin ? 1 : 0;
    }
  }
  __syncthreads();

  // hits: touch their slots; usage learned from the routed pairs
  int hits = 0;
  for (int e = t; e < E; e += kPlanThreads) {
    const int n = s_need[e];
    if (!n) continue;
    if (repin < 0) c.use_count[e] = s_use[e] + (uint32_t)n;
    const int sl = s_slot_of[e];
    if (sl >= 0) {
      s_last[sl] = clock;
      ++hits;
    }
  }
  if (hits) atomicAdd(&s_hits, hits);
  __syncthreads();

  // misses ranked in increasing expert order (each lane scans a contiguous run)
  const int per = (E + kPlanThreads - 1) / kPlanThreads;
  const int e0 = t * per, e1 = min(E, e0 + per);
  int local = 0;
  for (int e = e0; e < e1; ++e) local += (s_need[e] && s_slot_of[e] < 0);
  int n_miss = 0;
  int r = wg_exclusive_scan(local, s_scan, &n_miss);
  for (int e = e0; e < e1; ++e) s_mrank[e] = (s_need[e] && s_slot_of[e] < 0) ? r++ : -1;

  // victims: unpinned slots not used by this call, in (last_use, slot) order
  for (int s = t; s < S; s += kPlanThreads) {
    const bool el = !s_pin[s] && s_last[s] < clock;
    if (!el) continue;
    atomicAdd(&s_nelig, 1);
    const uint32_t ls = s_last[s];
    int rank = 0;
    for (int s2 = 0; s2 < S; ++s2) {
      const uint32_t l2 = s_last[s2];
      rank += (!s_pin[s2] && l2 < clock) && (l2 < ls || (l2 == ls && s2 < s));
    }
    if (rank < n_miss) s_victim[rank] = s;
  }
  __syncthreads();
  const int n_copy = min(n_miss, s_nelig);

  // move the misses in; evicted experts become absent
  for (int e = t; e < E; e += kPlanThreads) {
    const int m = s_mrank[e];
    if (m < 0 || m >= n_copy) continue;
    const int s = s_victim[m];
    const int old = s_expert_of[s];
    if (old >= 0) s_slot_of[old] = -1;
    s_slot_of[e] = s;
    s_expert_of[s] = e;
    s_last[s] = clock;
    c.copy_list[2 * m] = e;
    c.copy_list[2 * m + 1] = s;
  }
  __syncthreads();
  if (repin >= 0) {
    for (int e = t; e < E; e += kPlanThreads)
      if (s_need[e] && s_slot_of[e] >= 0) s_pin[s_slot_of[e]] = 1u;
    __syncthreads();
  }

  for (int i = t; i < E; i += kPlanThreads) c.slot_of[i] = s_slot_of[i];
  for (int i = t; i < S; i += kPlanThreads) {
    c.expert_of[i] = s_expert_of[i];
    c.last_use[i] = s_last[i];
    c.pinned[i] = s_pin[i];
  }
  if (t == 0) {
    c.ctl[0] = clock;
    c.ctl[1] = (uint32_t)n_copy;
    if (n_miss > n_copy) c.ctl[2] |= 1u;
    if (repin < 0) {
      unsigned long long *st = reinterpret_cast<unsigned long long *>(c.ctl + 4);
      st[0] += (unsigned long long)s_hits;
      st[1] += (unsigned long long)n_miss;
    }
  }
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

hipError_t launch_cache_fill(const CacheState &c, const CacheTier &t, hipStream_t st) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  hipLaunchKernelGGL(k_cache_fill, dim3(n_cu * 4), dim3(kFillThreads), 0, st, c, t);
  return hipGetLastError();
}

}  // namespace coli
