/*
 * coli_moe.h -- C ABI of the routed-expert MoE layer library (libcoli_moe.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer is the one the colibrì pages describe for GLM-5.2 (colibrì README,
 * JustVugg/colibri, sections "思路" (Idea) and "已实现的功能" (Implemented
 * features)):
 *   - a DeepSeek-V3-like sigmoid router with the aux-loss-free ("noaux_tc")
 *     selection bias, group-limited top-k and routed_scaling_factor;
 *   - one always-on shared expert;
 *   - SwiGLU expert FFNs whose weights are int8, packed int4 or packed int2
 *     with one fp32 scale per row, dequantised on use against Q8_0-style
 *     int8 activations (integer dot products);
 *   - a batch-union dispatch: in a multi-token batch (prefill, MTP verify)
 *     each unique expert is read once and applied to every token routed to it.
 *
 * Memory: every data pointer is a DEVICE pointer on the current HIP device
 * unless marked "host".  The caller allocates and owns every buffer and keeps
 * it alive until the stream work that uses it has finished; the library
 * allocates only when asked to (coli_host_alloc) and keeps no per-call
 * state, so calls on different streams may run concurrently when their
 * buffers are disjoint (an expert cache's calls excepted: they share the
 * cache's state).
 *
 * Streams: `stream` is a hipStream_t passed as a plain pointer (NULL = the
 * null stream).  Every call only enqueues work on it and returns; outputs are
 * valid when that stream work completes.  Outputs are fully overwritten.
 *
 * Errors: all argument checks run before anything is enqueued; on a failed
 * check the call returns a code and enqueues nothing.  A failed launch (or no
 * usable gfx950 device) returns COLI_ERR_DEVICE.  Faults during execution
 * surface, as with any HIP work, at the caller's next synchronisation.  No
 * C++ exception crosses this interface.
 *
 * Layouts (the container reading; the pages give only "per-row scale"):
 *   - quantised weights: row-major [rows][cols*b/8] bytes, b = 8, 4 or 2;
 *     codes are two's complement, lowest bits first: int4 byte j holds
 *     element 2j in bits 0-3 and 2j+1 in bits 4-7; int2 byte j holds element
 *     4j+m in bits 2m..2m+1.  Scales are fp32 [rows].  Codes lie in
 *     [-qmax, qmax] with qmax = 127, 7, 1 (int2 is ternary).
 *   - Q8_0 activations: blocks of 32 consecutive values, int8 codes and one
 *     fp32 scale per block.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_ABI_VERSION 1

typedef enum {
  COLI_OK = 0,
  COLI_ERR_INVALID_ARG = 1, /* a pointer, size or configuration check failed */
  COLI_ERR_UNSUPPORTED = 2, /* valid request outside this build's limits */
  COLI_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  COLI_ERR_DEVICE = 4       /* no gfx950 device, or a launch failed */
} coli_status;

typedef enum { COLI_Q8 = 8, COLI_Q4 = 4, COLI_Q2 = 2 } coli_qtype; /* bits */

/* Router configuration (host struct).  Limits: n_experts <= 1024,
 * n_experts % n_group == 0, 1 <= topk_group <= n_group <= 64,
 * 1 <= top_k <= min(32, topk_group * n_experts / n_group). */
typedef struct {
  int32_t n_experts;           /* E: 256 for GLM-5.2 */
  int32_t top_k;               /* k: 8 */
  int32_t n_group;             /* contiguous groups of E/n_group experts: 8 */
  int32_t topk_group;          /* groups kept: 4 */
  int32_t norm_topk_prob;      /* 1: selected weights normalised to sum 1 */
  float routed_scaling_factor; /* 2.5 */
  float expert_top_p;          /* adaptive expert top-p; off unless 0<p<1 */
  int32_t top_p_renorm;        /* 1: renormalise the kept weights */
} coli_router_cfg;

/* One layer's weights (host struct of device pointers): the routed experts,
 * the shared expert and the router gate of one MoE layer (colibrì README,
 * "Implemented features": shared expert, sigmoid router; "Idea": 256 routed
 * experts of ~19 MB each at int4).
 * Routed experts are stacked: w_gate/w_up [E][I][H*b/8], s_gate/s_up [E][I],
 * w_down [E][H][I*b/8], s_down [E][H].  The shared expert has the same
 * per-expert layouts (E = 1).  Every weight row must start 16-byte aligned
 * (holds for any 16-byte aligned base since H*b/8 and I*b/8 are multiples of
 * 16).  H and I are multiples of 64 (one 16-byte chunk of an int2 row, and
 * a whole number of 32-row blocks in every kernel), at most 8192.
 * mfma_min_tokens: in a
 * batch of T >= 2 tokens, a unique expert (or the shared expert) receiving at
 * least this many tokens runs on the int8 matrix cores, one with fewer on the
 * integer dot-product GEMV; 0 selects the library defaults (a routed expert
 * with 8 tokens, or any routed expert in a batch of 64 tokens or more; the
 * shared expert, which receives the whole batch, from 64 tokens).
 * Both give the same results up to fp32 summation order.
 * gate_offset: NOT a step of the pages' layer -- an extension for synthetic
 * workloads.  Optional [E] fp32 per-expert terms added (one binary32
 * addition) to the logits computed from gate_w, before selection and
 * weighting; a synthetic gate uses it to give each layer a skewed (Zipf-like)
 * expert popularity, the regime in which the pages' learned expert cache
 * pays.  NULL = none (the layer as the pages define it); ignored when logits
 * are supplied, which already include any offset. */
typedef struct {
  int32_t hidden;   /* H: 6144 */
  int32_t inter;    /* I: 2048 */
  int32_t qtype;    /* coli_qtype */
  coli_router_cfg router;
  const float *gate_w;    /* [E][H] fp32; may be NULL if logits are supplied */
  const float *gate_bias; /* [E] fp32 selection bias; NULL = zero */
  const uint8_t *w_gate;
  const uint8_t *w_up;
  const uint8_t *w_down;
  const float *s_gate;
  const float *s_up;
  const float *s_down;
  const uint8_t *sh_gate;
  const uint8_t *sh_up;
  const uint8_t *sh_down;
  const float *sh_s_gate;
  const float *sh_s_up;
  const float *sh_s_down;
  int32_t mfma_min_tokens;
  const float *gate_offset; /* [E] fp32 or NULL */
} coli_moe_layer;

/* ABI version (COLI_ABI_VERSION) and a static message for a status.  Library
 * plumbing, not a step of the pages' layer.  coli_status_str takes any int32
 * (a coli_status value or not: unknown codes give "unknown status"). */
int coli_abi_version(void);
const char *coli_status_str(int32_t s);

/* Weight quantisation and packing (colibrì README, "Implemented features":
 * int8 / packed int4 / packed int2 containers, one scale per row; the
 * "convert" tool requantises a checkpoint into this container).
 * Per row r of w [rows][cols] fp32: amax = max|w|; s = amax/qmax (fp32,
 * correctly rounded); q = clamp(round_half_even(w/s), -qmax, qmax); s = 0
 * gives q = 0.  Writes q_out [rows][cols*qtype/8] bytes (layout above) and
 * scale_out [rows].  cols must be a positive multiple of 32; rows >= 0. */
coli_status coli_quant_pack(int32_t qtype, const float *w, int64_t rows,
                            int64_t cols, uint8_t *q_out, float *scale_out,
                            void *stream);

/* FP8 checkpoint requantisation (colibrì README, "Implemented features": the
 * offline FP8 -> int4 converter dequantises the 128x128 block-scaled FP8
 * checkpoint and requantises it into the engine's container).
 * w8 [rows][cols] OCP FP8 E4M3 codes without infinities (sign, 4-bit
 * exponent of bias 7, 3-bit mantissa; exponent 0 subnormal), block_scale
 * [ceil(rows/128)][ceil(cols/128)] fp32, the scale of each 128x128 tile
 * counted from row 0 and column 0 (edge tiles partial).  Each weight is
 * fl32(e4m3(code) * block_scale), and the rows are then quantised and packed
 * exactly as coli_quant_pack does, into q_out [rows][cols*qtype/8] and
 * scale_out [rows].  The result is bit-identical to coli_quant_pack of the
 * dequantised fp32 matrix.  cols a positive multiple of 32, rows >= 0;
 * w8 and q_out 16-byte aligned.  The two NaN codes (0x7F, 0xFF) are not
 * weights: a row holding one gets unspecified codes and scale. */
coli_status coli_quant_pack_fp8(int32_t qtype, const uint8_t *w8,
                                const float *block_scale, int64_t rows,
                                int64_t cols, uint8_t *q_out, float *scale_out,
                                void *stream);

/* f32-activation variant of the quantised product, for one token
 * (colibrì README, "Implemented features": for a single row the int4 kernel
 * keeps its activations in f32, which measured faster there than the
 * integer Q8_0 path).  y[r] = s_r * sum_c code[r][c] * x[c] with the codes
 * of w [rows][cols*qtype/8] (layout above, 16-byte aligned rows), scale
 * [rows], x [cols] fp32 (16-byte aligned), y [rows] fp32; sums in fp32.
 * cols*qtype must be a multiple of 128 (one 16-byte chunk) and at most
 * 65536, with cols <= 16384 (int8 8192, int4 and int2 16384 columns);
 * rows >= 0. */
coli_status coli_gemv_f32act(int32_t qtype, const uint8_t *w, const float *scale,
                             int64_t rows, int64_t cols, const float *x, float *y,
                             void *stream);

/* Q8_0-style activation quantisation (colibrì README, "Implemented
 * features": integer dot products against Q8_0-style int8 activations).
 * x [T][n] fp32 -> q [T][n] int8 (natural order) and d [T][n/32] fp32:
 * d = amax/127 per block of 32; q = clamp(round_half_even(x/d), -127, 127);
 * d = 0 gives q = 0.  n a positive multiple of 32; T >= 0. */
coli_status coli_quant_act_q8_0(const float *x, int32_t T, int32_t n,
                                int8_t *q, float *d, void *stream);

/* Router logits (colibrì README, "Implemented features": the
 * DeepSeek-V3-like router scores every routed expert from the token's hidden
 * state; its gate is the one fp32 weight of the layer).
 * logits [T][E] = x [T][H] . gate_w[E][H]^T, accumulated in fp64 and rounded
 * once to fp32.  x, gate_w 16-byte aligned; H a positive multiple of 32;
 * T >= 0 (0: no-op).  Writes logits [T][E]; reads nothing else. */
coli_status coli_moe_logits(const float *x, const float *gate_w, int32_t T,
                            int32_t E, int32_t H, float *logits, void *stream);

/* Routing (colibrì README, "Implemented features": sigmoid router,
 * noaux_tc, routed_scaling_factor; "Quick start": expert top-p).
 * For each of T tokens: sigma = fl32(1/(1+exp(-l))) evaluated in fp64;
 * c = sigma + bias (selection only); group score = sum of the two largest c
 * of the group; keep topk_group groups, then the top_k largest c of their
 * experts (ties: lower index first) -- the rank order of the outputs;
 * w = sigma/S * rsf with S the fp32 sum of the chosen sigma in rank order
 * (sigma * rsf when norm_topk_prob is 0).  With expert top-p the slots
 * outside the smallest weight-descending prefix whose normalised sum reaches
 * p get idx -1 and w 0 (kept weights renormalised if top_p_renorm).
 * logits [T][E] fp32, bias [E] or NULL; writes topk_idx [T][k] int32 and
 * topk_w [T][k] fp32. */
coli_status coli_moe_route(const coli_router_cfg *cfg, const float *logits,
                           const float *bias, int32_t T, int32_t *topk_idx,
                           float *topk_w, void *stream);

/* Batch-union tables (colibrì README, "Implemented features": batch-union
 * MoE).  From topk_idx [T][k] (entries -1 skipped): counts [E], offs [E+1]
 * (exclusive scan of counts), perm [T*k] = t*k+j of the routed pairs listed
 * by expert id, then token, then slot (entries past offs[E] are undefined),
 * uniq [E] = experts with nonzero count in increasing order (entries past
 * n_uniq undefined), n_uniq [1].  Bit-exact and deterministic.  The forward
 * call builds the same tables inside its workspace. */
coli_status coli_moe_dispatch(const int32_t *topk_idx, int32_t T, int32_t k,
                              int32_t E, int32_t *counts, int32_t *offs,
                              int32_t *perm, int32_t *uniq, int32_t *n_uniq,
                              void *stream);

/* Workspace bytes coli_moe_forward needs for up to max_tokens tokens with
 * this layer's shapes (0 if the descriptor is invalid).  The workspace holds
 * what the layer passes between its steps: the Q8_0 codes of x and h, the
 * routing, the batch-union tables (colibrì README, "Implemented features":
 * batch-union MoE, each unique expert read once per batch) and, for T >= 2,
 * one fp32 output row per (token, slot) that the combine sums in slot order.
 * It is a caller-owned device buffer, 256-byte aligned.  Its first
 * COLI_WORKSPACE_COUNTER_BYTES bytes are the state header of the
 * single-kernel decode path: they must be zero before the workspace is first
 * used (allocate it zeroed), and every call leaves them as it found them,
 * except the status word below.  One workspace serves one call at a time.
 *
 * Status word (uint32 at byte offset COLI_WORKSPACE_STATUS_OFFSET; sticky):
 * the decode kernel's waits for data other workgroups produce are bounded.
 * They assume the kernel's workgroups (no more than the GPU holds at once)
 * become resident together, which holds when it has the GPU to itself.  If
 * other work holds part of the GPU and a wait runs out of polling rounds,
 * the kernel ORs COLI_WAIT_SCORES (router scores) or COLI_WAIT_SLOTS (expert
 * gate/up results) into the word, and that call's y and routing outputs are
 * undefined.  The library never clears it; read and clear it with
 * coli_moe_workspace_status.  A header holding stale nonzero counters can
 * likewise only give undefined outputs, a set status bit, or both -- never a
 * hang or an access outside the buffers.
 *
 * Polling bound (uint32 at COLI_WORKSPACE_SPIN_LIMIT_OFFSET): a test hook.
 * If it is nonzero when a decode call starts, its bits 0-30 replace the
 * default bound on each wait's polling rounds (capped at the default) for
 * that call, which clears it; with bit 31 set every wait of the call also
 * treats its data as absent, runs the bound out and gives up.
 * Failure-handling tests set it to 0x80000001 so that waits give up
 * deterministically while every workgroup still exits normally. */
#define COLI_WORKSPACE_COUNTER_BYTES 20480
#define COLI_WORKSPACE_STATUS_OFFSET 10752
#define COLI_WORKSPACE_SPIN_LIMIT_OFFSET 11008
#define COLI_WAIT_SCORES 1u
#define COLI_WAIT_SLOTS 2u

size_t coli_moe_workspace_bytes(const coli_moe_layer *L, int32_t max_tokens);

/* The routed-expert MoE layer on T tokens (colibrì README, "Implemented
 * features": the DeepSeek-V3-like sigmoid router with noaux_tc and
 * routed_scaling_factor, the shared expert, int8 / packed int4 / packed int2
 * experts with per-row scales against Q8_0-style int8 activations, and the
 * batch-union MoE in which each unique expert of a batch is read once and
 * applied to every token routed to it; "Quick start": expert top-p).
 * y [T][H] fp32 = shared(x_t) + sum_j w_tj *
 * expert_{idx_tj}(x_t), the sum over kept slots in rank order, where
 * expert(x) = down( silu(gate . q(x)) * (up . q(x)) ) with both expert inputs
 * Q8_0-quantised and all three products integer dot products rescaled by the
 * row scale and the block scale.  No residual and no normalisation.
 * x [T][H] fp32.  logits_in [T][E] or NULL (then logits = x . gate_w^T).
 * Optional outputs (NULL to skip): idx_out [T][k], w_out [T][k],
 * logits_out [T][E].  T = 1 runs the decode path (one kernel); T >= 2 groups
 * the batch by expert (each unique expert's weights are read once).  T = 0
 * is a no-op.  x and y 16-byte aligned.  workspace must hold
 * coli_moe_workspace_bytes(L, T) bytes (see there for its header and status
 * word).  Errors: COLI_ERR_INVALID_ARG for a bad descriptor, pointer or T
 * (T < 0 or > 2^20), COLI_ERR_WORKSPACE for a missing, misaligned or short
 * workspace, COLI_ERR_DEVICE for no gfx950 device or a failed launch; on any
 * error nothing is enqueued. */
coli_status coli_moe_forward(const coli_moe_layer *L, const float *x,
                             int32_t T, const float *logits_in, float *y,
                             int32_t *idx_out, float *w_out, float *logits_out,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Profiling variant of coli_moe_forward: the same layer (colibrì README,
 * "Implemented features"; see coli_moe_forward), same work, same results,
 * for the benchmark.  stage_events holds n_stage_events caller-created hipEvent_t
 * handles (NULL entries skipped): [2i] and [2i+1] are recorded by the launch
 * of kernel i itself at its start and end (so their interval is that
 * kernel's execution time).  T = 1: kernel 0 is the single decode kernel
 * (for row shapes it is not built for: as below, kernels 0-2).  T >= 2:
 * kernel 0 the front kernel (activation quantisation + logits), 1 the
 * gate/up and 2 the down-projection kernel of the dot-product path, 3 the
 * gate/up and 4 the down-projection kernel of the matrix-core path (a
 * kernel with no work records an empty interval; the matrix-core kernels
 * are not launched, and their events not recorded, when T is below the
 * layer's mfma_min_tokens). */
coli_status coli_moe_forward_profiled(const coli_moe_layer *L, const float *x,
                                      int32_t T, const float *logits_in,
                                      float *y, int32_t *idx_out, float *w_out,
                                      float *logits_out, void *workspace,
                                      size_t workspace_bytes, void *stream,
                                      void *const *stage_events,
                                      int32_t n_stage_events);

/* coli_moe_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, kernels and results, with the workspace
 * replaced by the library's own static device scratch of
 * COLI_NOALLOC_SCRATCH_BYTES per GPU (allocated when the library's code is
 * loaded on that GPU and held until the process ends).  The call allocates
 * nothing.  The caller still passes x, y and the optional outputs, as for
 * coli_moe_forward.  T whose workspace (coli_moe_workspace_bytes) exceeds
 * the scratch returns COLI_ERR_UNSUPPORTED and enqueues nothing (about 128
 * tokens at the GLM-5.2 shape; 1 token always fits).  wait_status_out:
 * optional device int32 that receives the scratch's status word after the
 * call (0 = every bounded wait completed), which is then cleared.  Every call
 * on one GPU shares that GPU's scratch and keeps its contents until the next
 * call: calls that overlap on one GPU (other streams, other threads) race and
 * give undefined results; serialise them. */
#define COLI_NOALLOC_SCRATCH_BYTES (32u << 20)
coli_status coli_moe_forward_noalloc(const coli_moe_layer *L, const float *x,
                                     int32_t T, const float *logits_in,
                                     float *y, int32_t *idx_out, float *w_out,
                                     float *logits_out,
                                     int32_t *wait_status_out, void *stream);

/* ---------------------------------------------------------------------------
 * Tiered expert residency.  The pages treat device memory, host memory and
 * disk as one hierarchy and stream the routed experts a token needs from the
 * slower tier (CSDN feature, "把内存、显存和磁盘当成同一块蛋糕"), behind a
 * per-layer LRU cache of experts plus an optional pinned store of the hot
 * ones (colibrì README, "Idea"), where the pinned set is learned from the
 * experts actually used and can be re-chosen in session (labhub post,
 * "让它变得可以忍受的那些装置": the usage profile and --repin; CSDN
 * feature, "冷启动与热缓存的辩证法").  Here the cache is HBM and the slower
 * tier is pinned host memory read by the GPU over the host link.
 *
 * One layer's cache: S HBM slots for routed experts.  The layer descriptor's
 * routed arrays (w_gate, s_gate, w_up, s_up, w_down, s_down) are stacked over
 * the S slots instead of the E experts; the host tier holds every routed
 * expert, stacked over E in the same per-expert layouts.  Every forward
 * through the cache first routes the batch, then one workgroup updates the
 * cache state and lists the misses, then a copy kernel moves the missing
 * experts from the host tier into their slots, and then the layer runs with
 * each routed expert read from its slot.  All of it is enqueued on the
 * stream with no host round trip.  The cache moves bytes, not arithmetic:
 * outputs equal coli_moe_forward's on a fully resident layer.
 *
 * Replacement, per call: the experts the batch selects form the set R
 * (entries -1 skipped).  The clock advances by one; each routed pair adds 1
 * to use_count of its expert; each expert of R that is resident has its
 * slot's last_use set to the clock (a hit).  The missing experts of R, in
 * increasing expert order, take the unpinned slots not used by this call in
 * increasing (last_use, slot) order, evicting what those slots held (an
 * empty slot has last_use 0, so empty slots fill first).  A call needs
 * min(E, T*k) <= S - n_pinned, checked on the host.
 * ------------------------------------------------------------------------- */

/* Pinned host memory for a host tier (library plumbing: hipHostMalloc with
 * the default flags).  The returned address is valid on the host and on the
 * device.  The library records the allocation: a cache's host tier must lie
 * inside allocations made here, so a kernel never reads host memory the GPU
 * cannot reach.  coli_host_free(NULL) does nothing. */
coli_status coli_host_alloc(size_t bytes, void **ptr_out);
coli_status coli_host_free(void *ptr);

/* One layer's expert cache (host struct; E routed experts, S slots). */
typedef struct {
  int32_t n_experts; /* E, equal to the layer's router.n_experts */
  int32_t n_slots;   /* S, 1 <= S <= E */
  int32_t n_pinned;  /* slots pinned by the last coli_expert_cache_repin (0 after init) */
  int32_t reserved;
  /* host tier, inside coli_host_alloc allocations: w_gate/w_up [E][I][H*b/8],
   * s_gate/s_up [E][I], w_down [E][H][I*b/8], s_down [E][H] */
  const uint8_t *host_w_gate, *host_w_up, *host_w_down;
  const float *host_s_gate, *host_s_up, *host_s_down;
  void *state; /* device, coli_expert_cache_layout_of(E, S).total bytes, 256-byte aligned */
} coli_expert_cache;

/* Byte offsets inside a cache's device state, each 256-byte aligned:
 *   ctl        uint32[64]: [0] clock, [1] misses copied by the last call,
 *              [2] error bits (1: a call had more misses than free slots;
 *              its outputs are undefined), [4..5] hits, [6..7] misses
 *              (uint64, low word first; counted per unique expert per call)
 *   slot_of    int32[E]: slot of expert e, or -1
 *   expert_of  int32[S]: expert held by slot s, or -1
 *   last_use   uint32[S]: clock of the slot's last use (0: never)
 *   pinned     uint32[S]: 1 if the slot is pinned
 *   use_count  uint32[E]: routed pairs that selected expert e since init (the
 *              learned usage profile; a caller may save it and write it
 *              back after init to restore what an earlier run learned)
 *   copy_list  int32[S][2]: (expert, slot) of the last call's misses */
typedef struct {
  size_t ctl, slot_of, expert_of, last_use, pinned, use_count, copy_list, total;
} coli_expert_cache_layout;
coli_status coli_expert_cache_layout_of(int32_t n_experts, int32_t n_slots,
                                        coli_expert_cache_layout *out);

/* Empties the cache: every slot empty, usage, counters and clock zero.
 * Enqueued on the stream (a fill kernel, no memset); n_pinned set to 0. */
coli_status coli_expert_cache_init(coli_expert_cache *C, void *stream);

/* Pins the n_pin experts with the largest use_count (ties: lower expert
 * index) and unpins every other slot; pinned experts that are not resident
 * are copied in, through the same replacement as a forward call (the clock
 * advances; hits, misses and usage are not counted).  Sets C->n_pinned =
 * n_pin.  0 <= n_pin < S.  L is the layer whose slots the cache fills. */
coli_status coli_expert_cache_repin(coli_expert_cache *C,
                                    const coli_moe_layer *L, int32_t n_pin,
                                    void *stream);

/* coli_moe_forward through the cache: the same arguments and results, with
 * L's routed arrays stacked over C's S slots.  Routing runs first (logits
 * from gate_w plus gate_offset unless logits_in is given), then the cache
 * update and copies, then the layer.  T must satisfy min(E, T*k) <= S -
 * C->n_pinned (else COLI_ERR_UNSUPPORTED).  Calls on one cache must be
 * serialised (one stream). */
coli_status coli_moe_forward_cached(const coli_moe_layer *L,
                                    const coli_expert_cache *C, const float *x,
                                    int32_t T, const float *logits_in,
                                    float *y, int32_t *idx_out, float *w_out,
                                    float *logits_out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Adaptive speculation guard.  Verifying the MTP head's drafts in one batch
 * makes every draft route to more experts; on a cold cache the extra expert
 * loads can cost more than the accepted drafts save, which is why the pages
 * pair drafting with an adaptive guard and a DRAFT=0 switch (colibrì README,
 * "Implemented features", native MTP item; "Quick start": DRAFT=n).
 *
 * A host-side controller (no device work).  After every step the caller
 * reports the drafts it verified, how many were accepted and the step's
 * cost (any additive measure: microseconds, expert bytes read, host-link
 * bytes).  The guard keeps, per mode, an exponentially weighted average of
 * the step cost (weight ema for the newest step) and a slower one of the
 * tokens each step produces, 1 + accepted (weight 0.4 * ema: the accepted
 * count varies from step to step around a slowly moving rate, while the step
 * cost follows the cache); their ratio is that mode's cost per produced
 * token (a ratio of averages: an average of per-step ratios would overrate
 * drafting's cost when acceptance varies from step to step).  It answers
 * the drafts for the next step: max_draft while the drafting estimate is at
 * most (1 + margin) times the plain one, else 0.  Every probe_every steps it
 * runs one step in the mode not in use, so both estimates stay current
 * (the cache warming up makes drafting pay again).  Unknown estimates:
 * drafting starts on and the first probe measures plain decode.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t max_draft;   /* drafts per step while drafting (DRAFT=n), >= 1 */
  int32_t probe_every; /* steps between probes of the other mode, >= 2 */
  float ema;           /* weight of the newest step in the estimates, (0, 1] */
  float margin;        /* drafting kept while cost_draft <= cost_plain * (1 + margin) */
  /* state, written by init and step */
  double cost_draft, cost_plain; /* per produced token; negative: not yet measured */
  double sum_cost[2], sum_tokens[2]; /* averages per step of the cost and of the tokens, [0] plain, [1] drafting */
  int32_t next_draft;            /* drafts the next step should verify */
  int32_t since_probe;           /* steps since the last probe */
  int64_t steps, draft_steps, tokens;
} coli_spec_guard;

coli_status coli_spec_guard_init(coli_spec_guard *g, int32_t max_draft,
                                 int32_t probe_every, float ema, float margin);
/* Records one step (drafted in 0..max_draft, accepted in 0..drafted, cost
 * >= 0) and returns the drafts for the next step (also in g->next_draft);
 * a malformed report returns -1 and changes nothing. */
int32_t coli_spec_guard_step(coli_spec_guard *g, int32_t drafted,
                             int32_t accepted, double cost);

/* Status of the decode path's bounded waits (library plumbing, not a step
 * of the pages' layer; it reports when the outputs of coli_moe_forward are
 * undefined).  The workspace's status word (see coli_moe_workspace_bytes) copied to
 * status_out[0] (device int32) on the stream, then set to zero if clear is
 * nonzero.  0 means every bounded wait of every decode call since the last
 * clear completed.  workspace 256-byte aligned, status_out 4-byte aligned. */
coli_status coli_moe_workspace_status(void *workspace, int32_t *status_out,
                                      int32_t clear, void *stream);

/* Test export of the integer products (colibrì README, "Implemented
 * features": integer dot products of the int8 / packed int4 / packed int2
 * weights against Q8_0-style int8 activations), same device code as the forward:
 * acc_out [T][rows][cols/32] int32 = per-block sums of weight codes times
 * Q8_0 codes, exact.  Wq [rows][cols*qtype/8], xq [T][cols] int8 (natural
 * order).  cols a positive multiple of 64, T <= 8. */
coli_status coli_debug_qgemv_blocks(int32_t qtype, const uint8_t *Wq,
                                    int32_t rows, int32_t cols,
                                    const int8_t *xq, int32_t T,
                                    int32_t *acc_out, void *stream);

/* Diagnostics (library plumbing, not steps of the pages' layer).
 *
 * coli_debug_decode_trace: coli_moe_forward for one token with logits
 * computed from the gate, on the single-kernel decode path only
 * (COLI_ERR_UNSUPPORTED for row shapes it is not built for, and always in
 * libcoli_moe.so: only the timeline build of the library, libcoli_moe_trace.so,
 * compiles the records in), recording a timeline: trace [trace_wgs][COLI_TRACE_RECORDS][2] uint64 (device), for
 * workgroups below trace_wgs, record n = (code << 48 | value, s_memrealtime
 * ticks at 100 MHz) at phase and item boundaries (codes: 1 entry, 2 logit
 * slices done, 3 x quantised, 4 the workgroup's shared-expert rows done, 5 selection
 * begins, 6 router scores all read, 7 selection done, 8 routed gate/up item
 * done, 9 down item begins, 10 its h is ready, 11 down item done, 12 exit;
 * the value is the item's ticket).  Unused records keep their contents: zero
 * the buffer first.  *grid_out (host) receives the grid size.  Same results
 * as coli_moe_forward.
 *
 * coli_debug_stream_read: reads `bytes` (a positive multiple of 16) of the
 * 16-byte aligned device buffer `buf` with the plain streaming access
 * pattern of a bandwidth-bound kernel (16-byte non-temporal loads, eight in
 * flight per lane, grid-strided over as many workgroups as keep the GPU
 * full) and writes one xor word per workgroup to out [*grid_out] (device;
 * must hold 8 words per compute unit).  Its duration is the practical HBM
 * ceiling for that many bytes. */
#define COLI_TRACE_RECORDS 64
coli_status coli_debug_decode_trace(const coli_moe_layer *L, const float *x,
                                    float *y, void *workspace,
                                    size_t workspace_bytes, uint64_t *trace,
                                    int32_t trace_wgs, int32_t *grid_out,
                                    void *stream);
coli_status coli_debug_stream_read(const void *buf, size_t bytes,
                                   uint32_t *out, int32_t *grid_out,
                                   void *stream);

#ifdef __cplusplus
}
#endif
#endif /* COLI_MOE_H */
