// kernels.hpp -- host-side launchers of the library's gfx950 kernels.  Each
// launcher enqueues on `st` and returns the launch status; shapes have been
// validated by the C-ABI layer (api.hip) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_ext.h>

#include "coli_moe.h"
#include "device.hpp"

namespace coli {

// Bytes at the start of the forward workspace that hold the single-kernel
// decode's counters (zero before first use, left zero by every call).
constexpr int kDecodeCounterBytes = COLI_WORKSPACE_COUNTER_BYTES;

// Optional per-kernel timing: events recorded by the launch itself at the
// kernel's start and end (hipExtLaunchKernelGGL), so their interval is the
// kernel's execution, as a kernel-trace profiler reports it.
struct KEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

#define COLI_LAUNCH(EV, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                  \
  do {                                                                                           \
    if ((EV).start || (EV).stop)                                                                 \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, (EV).start, (EV).stop, 0,        \
                            __VA_ARGS__);                                                        \
    else                                                                                         \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                       \
  } while (0)

// Router configuration as the kernels see it (a copy of the ABI struct).
struct RouterCfg {
  int E, k, n_group, topk_group, norm;
  float rsf, top_p;
  int renorm;
};

// Pointers of one layer's weights (device), stacked routed experts plus the
// shared expert.
struct LayerPtrs {
  int H, I, bits;
  const uint8_t *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;
  const uint8_t *sh_gate, *sh_up, *sh_down;
  const float *sh_s_gate, *sh_s_up, *sh_s_down;
  // expert cache: routed expert e lives in slot slot_of[e] of the routed
  // arrays (n_slots of them); null = every expert resident at index e
  const int32_t *slot_of;
  int n_slots;
};

// A layer's expert-cache state in device memory (layout in coli_moe.h).
constexpr int kCacheCtlWords = 64;
struct CacheState {
  uint32_t *ctl;
  int32_t *slot_of, *expert_of;
  uint32_t *last_use, *pinned, *use_count;
  int32_t *copy_list;
  int E, S;
};

// Where the cache copies from (host tier, device-visible) and to (the
// layer's routed slot arrays), with one expert's byte counts.
struct CacheTier {
  const uint8_t *hw_gate, *hw_up, *hw_down;
  const float *hs_gate, *hs_up, *hs_down;
  uint8_t *dw_gate, *dw_up, *dw_down;
  float *ds_gate, *ds_up, *ds_down;
  size_t gu_bytes, d_bytes;
  int I, H;
};

hipError_t launch_cache_init(const CacheState &c, hipStream_t st);
// repin < 0: a forward call's update from idx[0..n_pairs-1]; repin >= 0: pin
// the `repin` most-used experts.
hipError_t launch_cache_plan(const CacheState &c, const int32_t *idx, int n_pairs, int repin,
                             hipStream_t st);
// One token: selection from its logits (as every other path selects) and the
// cache update, in one launch.
hipError_t launch_cache_route_plan(const RouterCfg &cfg, const float *logits, const float *bias,
                                   const CacheState &c, hipStream_t st);
hipError_t launch_cache_fill(const CacheState &c, const CacheTier &t, hipStream_t st);

// Union bookkeeping living in the workspace.
struct Dispatch {
  const int32_t *counts;  // [E]
  const int32_t *offs;    // [E+1]
  const int32_t *perm;    // [T*k] entries t*k+j ordered by (expert, t, j)
  const int32_t *uniq;    // [E]
  const int32_t *n_uniq;  // [1]
  // matrix-core item tables: [2][E+2] first token group (64, then 32
  // tokens) of each union slot, then [2][mfma_gmax] union slot of each
  // group, then (from mfma_desc_off) the group counts {64, 32, n_uniq, 0}
  // and [2][mfma_gmax] group descriptors {expert (-1: shared), first pair
  // (-1: shared), first token, tokens}
  const int32_t *mgofs;
};

hipError_t launch_quant_pack(int bits, const float *w, int64_t rows, int64_t cols, uint8_t *q,
                             float *scale, hipStream_t st);
hipError_t launch_quant_pack_fp8(int bits, const uint8_t *w8, const float *bscale, int64_t rows,
                                 int64_t cols, uint8_t *q, float *scale, hipStream_t st);
hipError_t launch_gemv_f32act(int bits, const uint8_t *W, const float *scale, int64_t rows,
                              int64_t cols, const float *x, float *y, hipStream_t st);
constexpr int kMfmaGroup = 64;  // tokens per group in the matrix-core item table
// Token groups of `tok` tokens a union slot sends to the matrix cores (0:
// the dot-product path takes it).
__host__ __device__ inline int mfma_groups(int n_tok, int mfma_min, int tok) {
  return n_tok >= mfma_min ? (n_tok + tok - 1) / tok : 0;
}
// Bound of the matrix-core token groups of one batch (32-token groups: the
// routed pairs, one partial group per unique expert, the shared expert's).
__host__ __device__ inline int mfma_gmax(int T, int k, int E) {
  return (int)(((int64_t)T * k + 31) / 32 + E + (T + 31) / 32 + 1);
}
// Offset (int32 words, 16-byte aligned) of the group counts and descriptors
// in the matrix-core tables, and the tables' total size in words.
__host__ __device__ inline size_t mfma_desc_off(int T, int k, int E) {
  return ((2 * (size_t)(E + 2) + 2 * (size_t)mfma_gmax(T, k, E) + 3) / 4) * 4;
}
__host__ __device__ inline size_t mfma_table_words(int T, int k, int E) {
  return mfma_desc_off(T, k, E) + 4 + 8 * (size_t)mfma_gmax(T, k, E);
}
// Row stride of the binary64 copy of the Q8_0 block scales (d64, for the
// matrix-core gate/up): the blocks of a row rounded up to a multiple of 8.
__host__ __device__ inline int xd64_ld(int64_t n) { return (int)(((n / 32 + 7) / 8) * 8); }
hipError_t launch_act_quant(int layout_bits, const float *x, int64_t T, int64_t n, int8_t *q,
                            float *d, hipStream_t st, KEvents ev = {}, double *d64 = nullptr);

hipError_t launch_logits(const float *x, const float *gate_w, int T, int E, int H, float *logits,
                         hipStream_t st);
// Router logits (if gate_w) and Q8_0 activations in container BITS ordering
// (if xq), in as few launches as the batch allows.
// loff: optional [E] terms added to each computed logit.
// xd64: optional binary64 copy of xd (row stride xd64_ld(H)).
hipError_t launch_front(int bits, const float *x, const float *gate_w, const float *loff, int T,
                        int E, int H, float *logits, int8_t *xq, float *xd, hipStream_t st,
                        KEvents ev = {}, double *xd64 = nullptr);
hipError_t launch_route(const RouterCfg &cfg, const float *logits, const float *bias, int T,
                        int32_t *idx, float *w, int32_t *idx_copy, float *w_copy, hipStream_t st);
// Union tables (counts, offs, perm, uniq, n_uniq) from idx [T][k].  With
// mgofs, the same launch also writes the matrix-core item tables of the
// batch (layout at Dispatch::mgofs) for the slots with at least mfma_min
// tokens (the shared expert: mfma_min_shared).
hipError_t launch_dispatch(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offs,
                           int32_t *perm, int32_t *uniq, int32_t *n_uniq, hipStream_t st,
                           int32_t *mgofs = nullptr, int mfma_min = 0, int mfma_min_shared = 0);

// Expert FFN stages.  Slot lists: decode mode (T == 1) runs the k routed
// slots of token 0 (idx[0..k-1], -1 skipped) plus the shared expert as slot
// k; union mode runs every unique expert of the batch on its tokens plus the
// shared expert on all T tokens.  hq/hd rows: decode -> slot; union -> the
// pair's position in perm for routed pairs, n_routed + t for the shared one.
struct FfnArgs {
  LayerPtrs L;
  int T, k, E;
  const int8_t *xq;     // [T][H], ordering of L.bits
  const float *xd;      // [T][H/32]
  const double *xd64;   // union: xd in binary64, [T][xd64_ld(H)]
  int32_t *idx;         // [T][k] (decode: written by the gate/up kernel)
  float *w;             // [T][k]
  // decode mode: the gate/up kernel selects the experts itself
  RouterCfg cfg;
  const float *logits;  // [1][E]
  const float *bias;    // [E] or null
  const float *loff;    // [E] terms added to computed logits, or null
  int32_t *idx_user;    // optional copies for the caller
  float *w_user;
  Dispatch disp;        // union mode only
  int8_t *hq;           // [rows][I], ordering of L.bits
  float *hd;            // [rows][I/32]
  float *obuf;          // union: [T][k+1][H]
  float *y;             // [T][H]
  int mfma_min;         // union: routed slots with at least this many tokens run on the matrix cores
  int mfma_min_shared;  // union: the same for the shared expert (its tokens: the whole batch)
};

constexpr int kMfmaMinDefault = 8;  // default token count from which an expert runs on MFMA
// From this batch size on, the default sends every routed expert to the
// matrix cores: at 64-128 tokens the few-token experts the dot-product path
// would keep cost more there (measured at the GLM-5.2 shape: 64 tokens 1.33
// vs 1.19 ms, 128 tokens 1.86 vs 1.35 ms) than one matrix-core tile does.
constexpr int kMfmaAllTokens = 64;
// default for the shared expert, which receives the whole batch: one full
// 64-token group.  With fewer tokens it usually runs alone on the matrix
// cores (I/64 + H/64 workgroups), slower than on the dot-product path.
constexpr int kMfmaMinSharedDefault = 64;

hipError_t launch_gateup(const FfnArgs &a, bool union_mode, int mfma_min, hipStream_t st,
                         KEvents ev = {});
hipError_t launch_down(const FfnArgs &a, bool union_mode, int mfma_min, hipStream_t st,
                       KEvents ev = {});
hipError_t launch_combine(const FfnArgs &a, hipStream_t st);

// Union slots with at least a.mfma_min tokens run on the int8 matrix cores
// (mfma.hip), from the item tables launch_dispatch writes; the dot-product
// kernels skip those slots.
hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t st, KEvents ev = {});
hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t st, KEvents ev = {});

// The whole layer for one token in one kernel (decode.hip).  `ctr` is the
// workspace's state header (zero before the call; left zero after it).
// gate_w null: logits_in holds the supplied logits; else the computed logits
// are also written to logits_out when it is not null.  Returns
// hipErrorNotSupported for row shapes the kernel is not built for.
// trace: optional timeline records (coli_debug_decode_trace); grid_out
// (host) receives the grid size.
// hsh: [I] binary32 workspace for the shared expert's h.
hipError_t launch_decode_fused(const FfnArgs &f, const float *x, const float *gate_w,
                               const float *logits_in, float *logits_out, uint32_t *ctr,
                               float *hsh, hipStream_t st, KEvents ev = {},
                               uint64_t *trace = nullptr, int trace_wgs = 0,
                               int *grid_out = nullptr);

// A batch of 2 to 4 tokens (f.T) in one kernel: logits (or supplied ones),
// selection, the batch union, the combine (decode.hip).  The same header,
// waits and outputs as launch_decode_fused; idx/w: the workspace's [T][k]
// rows, through which the selections pass; hsh: [4][I] binary32; h rows of
// f.hq / f.hd: [T*k + T][...].  hipErrorNotSupported for other batch sizes
// and shapes.
hipError_t launch_small_fused(const FfnArgs &f, const float *x, const float *gate_w,
                              const float *logits_in, float *logits_out, uint32_t *ctr, float *hsh,
                              hipStream_t st, KEvents ev = {}, int *grid_out = nullptr);

// Plain streaming read of `bytes` (a multiple of 16, 16-byte aligned) with
// 16-byte non-temporal loads, one sum word per workgroup into out[grid]
// (keeps the loads live); *grid_out receives the grid size.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, int *grid_out,
                              hipStream_t st, KEvents ev = {});

// Copy the workspace header's sticky status word to out[0] (device), and
// clear it when `clear` is nonzero.
hipError_t launch_workspace_status(uint32_t *ctr, int32_t *out, int clear, hipStream_t st);

hipError_t launch_debug_blocks(int bits, const uint8_t *Wq, int rows, int cols, const int8_t *xq_perm,
                               int T, int32_t *acc, hipStream_t st);

}  // namespace coli
