// api.hip -- the C ABI declared in include/coli_moe.h: argument validation,
// workspace layout and the kernel sequence of each call.  Nothing here
// allocates device memory or synchronises the stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>

#include "coli_moe.h"
#include "kernels.hpp"

namespace {


constexpr int kMaxDim = 8192;
constexpr int kMaxTokens = 1 << 20;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device check, cached per device: 0 unknown, 1 usable gfx950, 2 not usable.
std::atomic<int> g_dev_state[64];

coli_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return COLI_ERR_DEVICE;
  }
  if (dev >= 64) return COLI_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    st = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      st = 1;
    (void)hipGetLastError();
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? COLI_OK : COLI_ERR_DEVICE;
}

coli_status from_hip(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_ERR_DEVICE; }

bool qtype_ok(int q) { return q == COLI_Q8 || q == COLI_Q4 || q == COLI_Q2; }

bool router_ok(const coli_router_cfg *c) {
  if (!c) return false;
  const int E = c->n_experts, G = c->n_group;
  if (E < 1 || E > 1024 || G < 1 || G > 64 || E % G) return false;
  if (c->topk_group < 1 || c->topk_group > G) return false;
  if (c->top_k < 1 || c->top_k > 32 || c->top_k > c->topk_group * (E / G)) return false;
  return true;
}

bool layer_ok(const coli_moe_layer *L) {
  if (!L || !qtype_ok(L->qtype) || !router_ok(&L->router)) return false;
  const int H = L->hidden, I = L->inter;
  if (H < 64 || I < 64 || H > kMaxDim || I > kMaxDim || H % 64 || I % 64) return false;
  const void *w[] = {L->w_gate, L->w_up, L->w_down, L->sh_gate, L->sh_up, L->sh_down};
  for (const void *p : w)
    if (!p || !aligned(p, 16)) return false;
  const void *s[] = {L->s_gate, L->s_up, L->s_down, L->sh_s_gate, L->sh_s_up, L->sh_s_down};
  for (const void *p : s)
    if (!p || !aligned(p, 4)) return false;
  if (L->gate_w && !aligned(L->gate_w, 16)) return false;
  if (L->gate_bias && !aligned(L->gate_bias, 4)) return false;
  if (L->gate_offset && !aligned(L->gate_offset, 4)) return false;
  if (L->mfma_min_tokens < 0) return false;
  return true;
}

coli::RouterCfg to_cfg(const coli_router_cfg &c) {
  return coli::RouterCfg{c.n_experts, c.top_k, c.n_group, c.topk_group, c.norm_topk_prob,
                         c.routed_scaling_factor, c.expert_top_p, c.top_p_renorm};
}

struct WsLayout {
  size_t ctr, xq, xd, xd64, logits, idx, w, counts, offs, perm, uniq, nuniq, mgofs, hq, hd, hsh, obuf,
      total;
};

WsLayout ws_layout(const coli_moe_layer *L, int Tmax) {
  const size_t H = L->hidden, I = L->inter, E = L->router.n_experts, k = L->router.top_k;
  const size_t T = Tmax < 1 ? 1 : Tmax;
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + (bytes ? bytes : 1), 256);
    return o;
  };
  w.ctr = take(COLI_WORKSPACE_COUNTER_BYTES);  // decode counters: zero before first use, left zero
  w.xq = take(T * H);
  w.xd = take(T * (H / 32) * 4);
  w.xd64 = take(Tmax >= 2 ? T * coli::xd64_ld(H) * 8 : 0);  // union batches only
  w.logits = take(T * E * 4);
  w.idx = take(T * k * 4);
  w.w = take(T * k * 4);
  w.counts = take(E * 4);
  w.offs = take((E + 1) * 4);
  w.perm = take(T * k * 4);
  w.uniq = take(E * 4);
  w.nuniq = take(4);
  // matrix-core item tables of 64- and 32-token groups
  w.mgofs = take(coli::mfma_table_words((int)T, (int)k, (int)E) * 4);
  w.hq = take((T * k + T) * I);
  w.hd = take((T * k + T) * (I / 32) * 4);
  w.hsh = take(4 * I * 4);  // decode and batches up to 4: the shared expert's h in binary32
  w.obuf = take(Tmax >= 2 ? T * (k + 1) * H * 4 : 0);
  w.total = off;
  return w;
}

// Scratch of coli_moe_forward_noalloc: the forward's workspace as a
// file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  Host code never names it except to look up each
// device's address (the name is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[COLI_NOALLOC_SCRATCH_BYTES];

// Per device: its copy's address, found once with that device current.
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

__global__ void k_zero_words(uint32_t *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address (nullptr on failure).  The first call
// on a device also clears the decode header at the start of the scratch with
// a kernel on `st` (a fill kernel, not a memset node, so it may be captured).
void *scratch_ptr(int dev, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    hipLaunchKernelGGL(k_zero_words, dim3(COLI_WORKSPACE_COUNTER_BYTES / 4 / 256), dim3(256), 0, st,
                       static_cast<uint32_t *>(p), COLI_WORKSPACE_COUNTER_BYTES / 4);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Pinned host allocations made by coli_host_alloc: base -> bytes.  A cache's
// host tier must lie inside one of them, so the copy kernel only reads host
// memory that is mapped for the GPU.
std::mutex g_host_mu;
std::map<uintptr_t, size_t> g_host_allocs;

bool in_host_alloc(const void *p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  std::lock_guard<std::mutex> lock(g_host_mu);
  auto it = g_host_allocs.upper_bound(a);
  if (it == g_host_allocs.begin()) return false;
  --it;
  return a >= it->first && bytes <= it->second && a - it->first <= it->second - bytes;
}

bool cache_layout(int E, int S, coli_expert_cache_layout *o) {
  if (E < 1 || E > 1024 || S < 1 || S > E) return false;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  o->ctl = take(coli::kCacheCtlWords * 4);
  o->slot_of = take((size_t)E * 4);
  o->expert_of = take((size_t)S * 4);
  o->last_use = take((size_t)S * 4);
  o->pinned = take((size_t)S * 4);
  o->use_count = take((size_t)E * 4);
  o->copy_list = take((size_t)S * 8);
  o->total = off;
  return true;
}

bool cache_state(const coli_expert_cache *C, coli::CacheState *st) {
  coli_expert_cache_layout lo;
  if (!C || !cache_layout(C->n_experts, C->n_slots, &lo) || !C->state || !aligned(C->state, 256))
    return false;
  if (C->n_pinned < 0 || C->n_pinned >= C->n_slots) return false;
  char *b = static_cast<char *>(C->state);
  st->ctl = reinterpret_cast<uint32_t *>(b + lo.ctl);
  st->slot_of = reinterpret_cast<int32_t *>(b + lo.slot_of);
  st->expert_of = reinterpret_cast<int32_t *>(b + lo.expert_of);
  st->last_use = reinterpret_cast<uint32_t *>(b + lo.last_use);
  st->pinned = reinterpret_cast<uint32_t *>(b + lo.pinned);
  st->use_count = reinterpret_cast<uint32_t *>(b + lo.use_count);
  st->copy_list = reinterpret_cast<int32_t *>(b + lo.copy_list);
  st->E = C->n_experts;
  st->S = C->n_slots;
  return true;
}

// The copy description of a cache over layer L: the host tier (checked to
// lie inside coli_host_alloc allocations) and L's routed arrays as slots.
bool cache_tier(const coli_moe_layer *L, const coli_expert_cache *C, coli::CacheTier *t) {
  if (!L || !C || C->n_experts != L->router.n_experts) return false;
  const size_t E = C->n_experts, H = L->hidden, I = L->inter, b = L->qtype;
  const size_t gu = I * (H * b / 8), d = H * (I * b / 8);
  const void *hw[] = {C->host_w_gate, C->host_w_up, C->host_w_down};
  const size_t hwb[] = {E * gu, E * gu, E * d};
  const void *hs[] = {C->host_s_gate, C->host_s_up, C->host_s_down};
  const size_t hsb[] = {E * I * 4, E * I * 4, E * H * 4};
  for (int i = 0; i < 3; ++i) {
    if (!hw[i] || !aligned(hw[i], 16) || !in_host_alloc(hw[i], hwb[i])) return false;
    if (!hs[i] || !aligned(hs[i], 16) || !in_host_alloc(hs[i], hsb[i])) return false;
  }
  // the copies move 16-byte words: the slot arrays' scales must be 16-byte aligned too
  if (!aligned(L->s_gate, 16) || !aligned(L->s_up, 16) || !aligned(L->s_down, 16)) return false;
  t->hw_gate = C->host_w_gate;
  t->hw_up = C->host_w_up;
  t->hw_down = C->host_w_down;
  t->hs_gate = C->host_s_gate;
  t->hs_up = C->host_s_up;
  t->hs_down = C->host_s_down;
  t->dw_gate = const_cast<uint8_t *>(L->w_gate);
  t->dw_up = const_cast<uint8_t *>(L->w_up);
  t->dw_down = const_cast<uint8_t *>(L->w_down);
  t->ds_gate = const_cast<float *>(L->s_gate);
  t->ds_up = const_cast<float *>(L->s_up);
  t->ds_down = const_cast<float *>(L->s_down);
  t->gu_bytes = gu;
  t->d_bytes = d;
  t->I = (int)I;
  t->H = (int)H;
  return true;
}

struct CacheRun {
  coli::CacheState st;
  coli::CacheTier tier;
};

coli_status forward_impl(const coli_moe_layer *L, const CacheRun *cache, const float *x,
                         int32_t T, const float *logits_in, float *y, int32_t *idx_out,
                         float *w_out, float *logits_out, void *workspace, size_t workspace_bytes,
                         void *stream, void *const *stage_events, int32_t n_stage_events);

template <typename F>
coli_status guarded(F &&f) {
  try {
    return f();
  } catch (...) {
    return COLI_ERR_DEVICE;
  }
}

}  // namespace

extern "C" {

int coli_abi_version(void) { return COLI_ABI_VERSION; }

const char *coli_status_str(int32_t s) {
  switch (s) {
    case COLI_OK: return "ok";
    case COLI_ERR_INVALID_ARG: return "invalid argument";
    case COLI_ERR_UNSUPPORTED: return "unsupported configuration";
    case COLI_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case COLI_ERR_DEVICE: return "no usable gfx950 device, or a launch failed";
  }
  return "unknown status";
}

coli_status coli_quant_pack(int32_t qtype, const float *w, int64_t rows, int64_t cols,
                            uint8_t *q_out, float *scale_out, void *stream) {
  return guarded([&] {
    if (!qtype_ok(qtype) || rows < 0 || cols <= 0 || cols % 32 || !w || !q_out || !scale_out)
      return COLI_ERR_INVALID_ARG;
    if (!aligned(w, 4) || !aligned(q_out, 4) || !aligned(scale_out, 4)) return COLI_ERR_INVALID_ARG;
    if (rows > (int64_t)1 << 34) return COLI_ERR_UNSUPPORTED;
    const coli_status d = check_device();
    if (d != COLI_OK) return d;
    return from_hip(coli::launch_quant_pack(qtype, w, rows, cols, q_out, scale_out,
                                            static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_quant_pack_fp8(int32_t qtype, const uint8_t *w8, const float *block_scale,
                                int64_t rows, int64_t cols, uint8_t *q_out, float *scale_out,
                                void *stream) {
  return guarded([&] {
    if (!qtype_ok(qtype) || rows < 0 || cols <= 0 || cols % 32 || !w8 || !block_scale || !q_out ||
        !scale_out)
      return COLI_ERR_INVALID_ARG;
    if (!aligned(w8, 16) || !aligned(q_out, 16) || !aligned(block_scale, 4) ||
        !aligned(scale_out, 4))
      return COLI_ERR_INVALID_ARG;
    if (rows > (int64_t)1 << 34 || cols > (int64_t)1 << 30) return COLI_ERR_UNSUPPORTED;
    const coli_status d = check_device();
    if (d != COLI_OK) return d;
    return from_hip(coli::launch_quant_pack_fp8(qtype, w8, block_scale, rows, cols, q_out,
                                                scale_out, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_gemv_f32act(int32_t qtype, const uint8_t *w, const float *scale, int64_t rows,
                             int64_t cols, const float *x, float *y, void *stream) {
  return guarded([&] {
    if (!qtype_ok(qtype) || rows < 0 || cols <= 0 || (cols * qtype) % 128 || !w || !scale || !x ||
        !y)
      return COLI_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(scale, 4) || !aligned(y, 4))
      return COLI_ERR_INVALID_ARG;
    if (rows > (int64_t)1 << 34 || (cols * qtype / 128 + 63) / 64 > 8 || cols > 16384)
      return COLI_ERR_UNSUPPORTED;
    const coli_status d = check_device();
    if (d != COLI_OK) return d;
    return from_hip(coli::launch_gemv_f32act(qtype, w, scale, rows, cols, x, y,
                                             static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_quant_act_q8_0(const float *x, int32_t T, int32_t n, int8_t *q, float *d,
                                void *stream) {
  return guarded([&] {
    if (T < 0 || n <= 0 || n % 32 || !x || !q || !d) return COLI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4)) return COLI_ERR_INVALID_ARG;
    // one thread per 32-value block; the launch's thread count is 32-bit
    if ((int64_t)T * (n / 32) > (int64_t)UINT32_MAX - 255) return COLI_ERR_UNSUPPORTED;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_act_quant(8, x, T, n, q, d, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_moe_logits(const float *x, const float *gate_w, int32_t T, int32_t E, int32_t H,
                            float *logits, void *stream) {
  return guarded([&] {
    if (T < 0 || E < 1 || H < 32 || H % 32 || !x || !gate_w || !logits) return COLI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(gate_w, 16) || !aligned(logits, 4)) return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_logits(x, gate_w, T, E, H, logits, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_moe_route(const coli_router_cfg *cfg, const float *logits, const float *bias,
                           int32_t T, int32_t *topk_idx, float *topk_w, void *stream) {
  return guarded([&] {
    if (!router_ok(cfg) || T < 0 || T > kMaxTokens || !logits || !topk_idx || !topk_w)
      return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_route(to_cfg(*cfg), logits, bias, T, topk_idx, topk_w, nullptr,
                                       nullptr, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_moe_dispatch(const int32_t *topk_idx, int32_t T, int32_t k, int32_t E,
                              int32_t *counts, int32_t *offs, int32_t *perm, int32_t *uniq,
                              int32_t *n_uniq, void *stream) {
  return guarded([&] {
    if (T < 0 || T > kMaxTokens || k < 1 || k > 32 || E < 1 || E > 1024 || !topk_idx || !counts ||
        !offs || !perm || !uniq || !n_uniq)
      return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_dispatch(topk_idx, T, k, E, counts, offs, perm, uniq, n_uniq,
                                          static_cast<hipStream_t>(stream)));
  });
}

size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int32_t max_tokens) {
  if (!layer_ok(L) || max_tokens < 0 || max_tokens > kMaxTokens) return 0;
  return ws_layout(L, max_tokens).total;
}

coli_status coli_moe_forward(const coli_moe_layer *L, const float *x, int32_t T,
                             const float *logits_in, float *y, int32_t *idx_out, float *w_out,
                             float *logits_out, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return coli_moe_forward_profiled(L, x, T, logits_in, y, idx_out, w_out, logits_out, workspace,
                                   workspace_bytes, stream, nullptr, 0);
}

coli_status coli_moe_forward_profiled(const coli_moe_layer *L, const float *x, int32_t T,
                                      const float *logits_in, float *y, int32_t *idx_out,
                                      float *w_out, float *logits_out, void *workspace,
                                      size_t workspace_bytes, void *stream,
                                      void *const *stage_events, int32_t n_stage_events) {
  return forward_impl(L, nullptr, x, T, logits_in, y, idx_out, w_out, logits_out, workspace,
                      workspace_bytes, stream, stage_events, n_stage_events);
}

}  // extern "C"

namespace {

// The layer on T tokens; with `cache`, routing runs first, then the cache
// update and copies, and routed experts are read from their slots.
coli_status forward_impl(const coli_moe_layer *L, const CacheRun *cache, const float *x,
                         int32_t T, const float *logits_in, float *y, int32_t *idx_out,
                         float *w_out, float *logits_out, void *workspace, size_t workspace_bytes,
                         void *stream, void *const *stage_events, int32_t n_stage_events) {
  return guarded([&] {
    if (n_stage_events < 0 || (n_stage_events > 0 && !stage_events)) return COLI_ERR_INVALID_ARG;
    if (!layer_ok(L) || T < 0 || T > kMaxTokens) return COLI_ERR_INVALID_ARG;
    if (T == 0) return COLI_OK;
    if (!x || !y) return COLI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return COLI_ERR_INVALID_ARG;
    if (!logits_in && !L->gate_w) return COLI_ERR_INVALID_ARG;
    if (logits_in && !aligned(logits_in, 4)) return COLI_ERR_INVALID_ARG;
    if ((idx_out && !aligned(idx_out, 4)) || (w_out && !aligned(w_out, 4)) ||
        (logits_out && !aligned(logits_out, 4)))
      return COLI_ERR_INVALID_ARG;
    const WsLayout ws = ws_layout(L, T);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < ws.total)
      return COLI_ERR_WORKSPACE;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(workspace);
    const int H = L->hidden, I = L->inter, E = L->router.n_experts, k = L->router.top_k;
    int8_t *xq = reinterpret_cast<int8_t *>(base + ws.xq);
    float *xd = reinterpret_cast<float *>(base + ws.xd);
    int32_t *idx = reinterpret_cast<int32_t *>(base + ws.idx);
    float *wts = reinterpret_cast<float *>(base + ws.w);

    // kernel i in (front, gate/up, down) gets events [2i] and [2i+1]
    auto kev = [&](int i) {
      coli::KEvents ev;
      if (2 * i < n_stage_events) ev.start = static_cast<hipEvent_t>(stage_events[2 * i]);
      if (2 * i + 1 < n_stage_events) ev.stop = static_cast<hipEvent_t>(stage_events[2 * i + 1]);
      return ev;
    };
    hipError_t e = hipSuccess;
    float *lp_dst = logits_out ? logits_out : reinterpret_cast<float *>(base + ws.logits);
    if (logits_in && logits_out) {
      e = hipMemcpyAsync(logits_out, logits_in, (size_t)T * E * sizeof(float),
                         hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return COLI_ERR_DEVICE;
    }
    const float *lp = logits_in ? logits_in : lp_dst;

    coli::FfnArgs fa{};
    fa.L = coli::LayerPtrs{H, I, L->qtype, L->w_gate, L->w_up, L->w_down, L->s_gate, L->s_up,
                           L->s_down, L->sh_gate, L->sh_up, L->sh_down, L->sh_s_gate,
                           L->sh_s_up, L->sh_s_down};
    if (cache) {
      fa.L.slot_of = cache->st.slot_of;
      fa.L.n_slots = cache->st.S;
    }
    fa.T = T;
    fa.k = k;
    fa.E = E;
    fa.xq = xq;
    fa.xd = xd;
    fa.idx = idx;
    fa.w = wts;
    fa.cfg = to_cfg(L->router);
    fa.logits = lp;
    fa.bias = L->gate_bias;
    fa.loff = logits_in ? nullptr : L->gate_offset;
    fa.idx_user = idx_out;
    fa.w_user = w_out;
    fa.hq = reinterpret_cast<int8_t *>(base + ws.hq);
    fa.hd = reinterpret_cast<float *>(base + ws.hd);
    fa.obuf = reinterpret_cast<float *>(base + ws.obuf);
    fa.y = y;
    const int mfma_min = L->mfma_min_tokens;
    // the cache update and copies, once the batch's routing is in idx
    auto cache_step = [&]() {
      hipError_t ce = coli::launch_cache_plan(cache->st, idx, T * k, -1, s);
      if (ce == hipSuccess) ce = coli::launch_cache_fill(cache->st, cache->tier, s);
      return ce;
    };
    if (cache && T == 1) {
      // decode through the cache: logits (unless supplied), selection, cache
      // update and copies, then the layer on the supplied logits
      if (!logits_in) {
        e = coli::launch_front(L->qtype, x, L->gate_w, L->gate_offset, T, E, H, lp_dst, nullptr,
                               nullptr, s);
        if (e != hipSuccess) return COLI_ERR_DEVICE;
      }
      e = coli::launch_cache_route_plan(to_cfg(L->router), lp, L->gate_bias, cache->st, s);
      if (e == hipSuccess) e = coli::launch_cache_fill(cache->st, cache->tier, s);
      if (e != hipSuccess) return COLI_ERR_DEVICE;
      fa.loff = nullptr;
      e = coli::launch_decode_fused(fa, x, nullptr, lp, nullptr,
                                    reinterpret_cast<uint32_t *>(base + ws.ctr),
                                    reinterpret_cast<float *>(base + ws.hsh), s, kev(0));
      if (e != hipErrorNotSupported) return from_hip(e);
      e = coli::launch_front(L->qtype, x, nullptr, nullptr, T, E, H, nullptr, xq, xd, s, kev(0));
      if (e == hipSuccess) e = coli::launch_gateup(fa, false, mfma_min, s, kev(1));
      if (e == hipSuccess) e = coli::launch_down(fa, false, mfma_min, s, kev(2));
      return from_hip(e);
    }
    if (T == 1) {
      // decode: the whole layer in one kernel where that kernel is built for
      // the layer's row shapes
      e = coli::launch_decode_fused(fa, x, logits_in ? nullptr : L->gate_w, logits_in, logits_out,
                                    reinterpret_cast<uint32_t *>(base + ws.ctr),
                                    reinterpret_cast<float *>(base + ws.hsh), s, kev(0));
      if (e != hipErrorNotSupported) return from_hip(e);
    }
    if (!cache && T >= 2 && T <= 4) {
      // a small batch (an MTP verify): the whole layer in one kernel where
      // that kernel is built for the layer's shapes
      e = coli::launch_small_fused(fa, x, logits_in ? nullptr : L->gate_w, logits_in, logits_out,
                                   reinterpret_cast<uint32_t *>(base + ws.ctr),
                                   reinterpret_cast<float *>(base + ws.hsh), s, kev(0));
      if (e != hipErrorNotSupported) return from_hip(e);
    }
    // activations -> Q8_0 codes (union batches: their scales in binary64
    // too, for the matrix cores), and the router logits unless supplied
    double *xd64 = T >= 2 ? reinterpret_cast<double *>(base + ws.xd64) : nullptr;
    fa.xd64 = xd64;
    e = coli::launch_front(L->qtype, x, logits_in ? nullptr : L->gate_w, fa.loff, T, E, H, lp_dst,
                           xq, xd, s, kev(0), xd64);
    if (e != hipSuccess) return COLI_ERR_DEVICE;
    if (T == 1) {
      // decode on other shapes: each gate/up workgroup selects the experts itself
      e = coli::launch_gateup(fa, false, mfma_min, s, kev(1));
      if (e == hipSuccess) e = coli::launch_down(fa, false, mfma_min, s, kev(2));
      return from_hip(e);
    }
    e = coli::launch_route(to_cfg(L->router), lp, L->gate_bias, T, idx, wts, idx_out, w_out, s);
    if (e != hipSuccess) return COLI_ERR_DEVICE;
    if (cache && cache_step() != hipSuccess) return COLI_ERR_DEVICE;
    int32_t *counts = reinterpret_cast<int32_t *>(base + ws.counts);
    int32_t *offs = reinterpret_cast<int32_t *>(base + ws.offs);
    int32_t *perm = reinterpret_cast<int32_t *>(base + ws.perm);
    int32_t *uniq = reinterpret_cast<int32_t *>(base + ws.uniq);
    int32_t *nuniq = reinterpret_cast<int32_t *>(base + ws.nuniq);
    int32_t *mgofs = reinterpret_cast<int32_t *>(base + ws.mgofs);
    fa.disp = coli::Dispatch{counts, offs, perm, uniq, nuniq, mgofs};
    fa.mfma_min = mfma_min > 0 ? mfma_min : T >= coli::kMfmaAllTokens ? 1 : coli::kMfmaMinDefault;
    fa.mfma_min_shared = mfma_min > 0 ? mfma_min : coli::kMfmaMinSharedDefault;
    // no slot of a batch smaller than mfma_min tokens can reach the matrix cores
    const bool mfma = T >= fa.mfma_min;
    // every slot on the matrix cores: the dot-product kernels would only
    // launch workgroups that find nothing to do
    const bool dot = !(mfma && fa.mfma_min <= 1 && T >= fa.mfma_min_shared);
    // the union tables, and the matrix-core item tables in the same launch
    e = coli::launch_dispatch(idx, T, k, E, counts, offs, perm, uniq, nuniq, s,
                              mfma ? mgofs : nullptr, fa.mfma_min, fa.mfma_min_shared);
    if (e != hipSuccess) return COLI_ERR_DEVICE;
    if (dot) e = coli::launch_gateup(fa, true, mfma_min, s, kev(1));
    if (e == hipSuccess && mfma) e = coli::launch_gateup_mfma(fa, s, kev(3));
    if (e == hipSuccess && dot) e = coli::launch_down(fa, true, mfma_min, s, kev(2));
    if (e == hipSuccess && mfma) e = coli::launch_down_mfma(fa, s, kev(4));
    if (e == hipSuccess) e = coli::launch_combine(fa, s);
    return from_hip(e);
  });
}

}  // namespace

extern "C" {

coli_status coli_moe_forward_noalloc(const coli_moe_layer *L, const float *x, int32_t T,
                                     const float *logits_in, float *y, int32_t *idx_out,
                                     float *w_out, float *logits_out, int32_t *wait_status_out,
                                     void *stream) {
  return guarded([&] {
    if (!layer_ok(L) || T < 0 || T > kMaxTokens) return COLI_ERR_INVALID_ARG;
    if (wait_status_out && !aligned(wait_status_out, 4)) return COLI_ERR_INVALID_ARG;
    if (T == 0) return COLI_OK;
    if (ws_layout(L, T).total > (size_t)COLI_NOALLOC_SCRATCH_BYTES) return COLI_ERR_UNSUPPORTED;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return COLI_ERR_DEVICE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = scratch_ptr(dev, s);
    if (!ws) return COLI_ERR_DEVICE;
    const coli_status r = coli_moe_forward_profiled(L, x, T, logits_in, y, idx_out, w_out,
                                                    logits_out, ws, COLI_NOALLOC_SCRATCH_BYTES,
                                                    stream, nullptr, 0);
    if (r != COLI_OK || !wait_status_out) return r;
    return from_hip(coli::launch_workspace_status(static_cast<uint32_t *>(ws), wait_status_out, 1, s));
  });
}

coli_status coli_moe_workspace_status(void *workspace, int32_t *status_out, int32_t clear,
                                      void *stream) {
  return guarded([&] {
    if (!workspace || !aligned(workspace, 256) || !status_out || !aligned(status_out, 4))
      return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_workspace_status(static_cast<uint32_t *>(workspace), status_out,
                                                  clear ? 1 : 0, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_debug_decode_trace(const coli_moe_layer *L, const float *x, float *y,
                                    void *workspace, size_t workspace_bytes, uint64_t *trace,
                                    int32_t trace_wgs, int32_t *grid_out, void *stream) {
  return guarded([&] {
    if (!layer_ok(L) || !L->gate_w || !x || !y || !trace || trace_wgs < 1 || !grid_out)
      return COLI_ERR_INVALID_ARG;
#ifndef COLI_DECODE_TRACE
    // the ordinary build records nothing: libcoli_moe_trace.so does
    return COLI_ERR_UNSUPPORTED;
#endif
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(trace, 8)) return COLI_ERR_INVALID_ARG;
    const WsLayout ws = ws_layout(L, 1);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < ws.total)
      return COLI_ERR_WORKSPACE;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    char *base = static_cast<char *>(workspace);
    coli::FfnArgs fa{};
    fa.L = coli::LayerPtrs{L->hidden, L->inter, L->qtype, L->w_gate, L->w_up, L->w_down,
                           L->s_gate, L->s_up, L->s_down, L->sh_gate, L->sh_up, L->sh_down,
                           L->sh_s_gate, L->sh_s_up, L->sh_s_down};
    fa.T = 1;
    fa.k = L->router.top_k;
    fa.E = L->router.n_experts;
    fa.xq = reinterpret_cast<int8_t *>(base + ws.xq);
    fa.xd = reinterpret_cast<float *>(base + ws.xd);
    fa.idx = reinterpret_cast<int32_t *>(base + ws.idx);
    fa.w = reinterpret_cast<float *>(base + ws.w);
    fa.cfg = to_cfg(L->router);
    fa.logits = reinterpret_cast<float *>(base + ws.logits);
    fa.bias = L->gate_bias;
    fa.loff = L->gate_offset;
    fa.hq = reinterpret_cast<int8_t *>(base + ws.hq);
    fa.hd = reinterpret_cast<float *>(base + ws.hd);
    fa.y = y;
    int grid = 0;
    const hipError_t e = coli::launch_decode_fused(
        fa, x, L->gate_w, nullptr, nullptr, reinterpret_cast<uint32_t *>(base + ws.ctr),
        reinterpret_cast<float *>(base + ws.hsh), static_cast<hipStream_t>(stream), {}, trace,
        trace_wgs, &grid);
    if (e == hipErrorNotSupported) return COLI_ERR_UNSUPPORTED;
    *grid_out = grid;
    return from_hip(e);
  });
}

coli_status coli_debug_stream_read(const void *buf, size_t bytes, uint32_t *out,
                                   int32_t *grid_out, void *stream) {
  return guarded([&] {
    if (!buf || !out || !grid_out || bytes == 0 || bytes % 16 || !aligned(buf, 16) ||
        !aligned(out, 4))
      return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    int grid = 0;
    const hipError_t e = coli::launch_stream_read(buf, bytes, out, &grid,
                                                  static_cast<hipStream_t>(stream));
    *grid_out = grid;
    return from_hip(e);
  });
}

coli_status coli_debug_qgemv_blocks(int32_t qtype, const uint8_t *Wq, int32_t rows, int32_t cols,
                                    const int8_t *xq, int32_t T, int32_t *acc_out, void *stream) {
  return guarded([&] {
    if (!qtype_ok(qtype) || rows < 0 || cols < 64 || cols % 64 || T < 0 || T > 8 || !Wq || !xq ||
        !acc_out)
      return COLI_ERR_INVALID_ARG;
    if (!aligned(Wq, 16) || !aligned(xq, 4) || !aligned(acc_out, 4)) return COLI_ERR_INVALID_ARG;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    return from_hip(coli::launch_debug_blocks(qtype, Wq, rows, cols, xq, T, acc_out,
                                              static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_host_alloc(size_t bytes, void **ptr_out) {
  return guarded([&] {
    if (!ptr_out || bytes == 0) return COLI_ERR_INVALID_ARG;
    *ptr_out = nullptr;
    const coli_status st = check_device();
    if (st != COLI_OK) return st;
    void *p = nullptr;
    if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess || !p) {
      (void)hipGetLastError();
      return COLI_ERR_DEVICE;
    }
    // the copy kernel reads the host tier at its host address
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || d != p) {
      (void)hipGetLastError();
      (void)hipHostFree(p);
      return COLI_ERR_DEVICE;
    }
    {
      std::lock_guard<std::mutex> lock(g_host_mu);
      g_host_allocs[reinterpret_cast<uintptr_t>(p)] = bytes;
    }
    *ptr_out = p;
    return COLI_OK;
  });
}

coli_status coli_host_free(void *ptr) {
  return guarded([&] {
    if (!ptr) return COLI_OK;
    {
      std::lock_guard<std::mutex> lock(g_host_mu);
      auto it = g_host_allocs.find(reinterpret_cast<uintptr_t>(ptr));
      if (it == g_host_allocs.end()) return COLI_ERR_INVALID_ARG;
      g_host_allocs.erase(it);
    }
    return from_hip(hipHostFree(ptr));
  });
}

coli_status coli_expert_cache_layout_of(int32_t n_experts, int32_t n_slots,
                                        coli_expert_cache_layout *out) {
  if (!out || !cache_layout(n_experts, n_slots, out)) return COLI_ERR_INVALID_ARG;
  return COLI_OK;
}

coli_status coli_expert_cache_init(coli_expert_cache *C, void *stream) {
  return guarded([&] {
    coli::CacheState st;
    if (!C) return COLI_ERR_INVALID_ARG;
    C->n_pinned = 0;
    if (!cache_state(C, &st)) return COLI_ERR_INVALID_ARG;
    const coli_status ds = check_device();
    if (ds != COLI_OK) return ds;
    return from_hip(coli::launch_cache_init(st, static_cast<hipStream_t>(stream)));
  });
}

coli_status coli_expert_cache_repin(coli_expert_cache *C, const coli_moe_layer *L, int32_t n_pin,
                                    void *stream) {
  return guarded([&] {
    CacheRun run;
    if (!C || !layer_ok(L) || !cache_state(C, &run.st) || !cache_tier(L, C, &run.tier))
      return COLI_ERR_INVALID_ARG;
    if (n_pin < 0 || n_pin >= C->n_slots) return COLI_ERR_INVALID_ARG;
    const coli_status ds = check_device();
    if (ds != COLI_OK) return ds;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = coli::launch_cache_plan(run.st, nullptr, 0, n_pin, s);
    if (e == hipSuccess) e = coli::launch_cache_fill(run.st, run.tier, s);
    if (e != hipSuccess) return COLI_ERR_DEVICE;
    C->n_pinned = n_pin;
    return COLI_OK;
  });
}

coli_status coli_moe_forward_cached(const coli_moe_layer *L, const coli_expert_cache *C,
                                    const float *x, int32_t T, const float *logits_in, float *y,
                                    int32_t *idx_out, float *w_out, float *logits_out,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  return guarded([&] {
    CacheRun run;
    if (!layer_ok(L) || !cache_state(C, &run.st) || !cache_tier(L, C, &run.tier))
      return COLI_ERR_INVALID_ARG;
    if (T < 0 || T > kMaxTokens) return COLI_ERR_INVALID_ARG;
    // every expert the batch selects must find a slot
    const int64_t need = std::min<int64_t>(C->n_experts, (int64_t)T * L->router.top_k);
    if (need > C->n_slots - C->n_pinned) return COLI_ERR_UNSUPPORTED;
    return forward_impl(L, &run, x, T, logits_in, y, idx_out, w_out, logits_out, workspace,
                        workspace_bytes, stream, nullptr, 0);
  });
}

}  // extern "C"
