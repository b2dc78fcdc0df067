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
// Every workgroup first computes its router logit slices (binary64 partial
// sums of gate rows; skipped if logits are given), quantises x into its LDS
// and requests its rows of the shared expert's gate/up, then selects the
// token's experts and finishes those rows.  Then work items, in ticket
// order:
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
//   workgroups, and per slot the finished gate/up items (routed 0 .. k-1)
//   or rows (shared, k);
//   the status word (sticky: give-ups of bounded waits, never cleared by the
//   kernel) and the polling bound override (test hook: if nonzero at the
//   start of a call, the bound on every wait's polling rounds; cleared by
//   the call);
//   then up to 1024 64-bit words of router logit partials: slice s = e * P + p
//   holds the complemented bits of the binary64 sum of x . gate_w[e] over the
//   p-th of P equal column ranges.  Zero means "not written yet" (no finite
//   binary64 value has all bits set), so consumers poll the words
//   themselves.
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
constexpr int kMaxSlices = 1024;  // logit partial words in the header
static_assert((kScoreWords + 2 * kMaxSlices) * 4 <= kDecodeCounterBytes,
              "decode state exceeds the workspace header");
static_assert(kCtrStatus * 4 == COLI_WORKSPACE_STATUS_OFFSET, "status word offset");
static_assert(kCtrSpin * 4 == COLI_WORKSPACE_SPIN_LIMIT_OFFSET, "polling bound offset");
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr uint32_t kSpinLimit = 1u << 19;  // ~100 ms of polling
constexpr int kMaxPartsPerRow = 4;         // logit slices per gate row at most
constexpr int kGuRows = 32;                // gate/up rows per GS/GR item
#ifndef COLI_DECODE_GU_PIPE
#define COLI_DECODE_GU_PIPE 1
#endif
constexpr int kGuPipe = COLI_DECODE_GU_PIPE;  // gate/up row passes in flight per wave
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
  int n_slice, n_part;   // logit slices (E * n_part, 0 with supplied logits) and parts per row
  float *hsh;            // [I] the shared expert's h in binary32 (workspace)
  int sh_rows;           // shared-expert gate/up rows of each workgroup
  int n_gr, n_down, total;  // items: GR, then D; total
  int down_rows;         // output rows per D item
  int slot_group;        // slots staged in LDS at a time by a D item
  int lds_x;             // byte offset of x's Q8_0 codes and scales in dynamic LDS
  int lds_l;             // byte offset of the token's logits kept for logits_out (-1: none)
  uint64_t *trace;       // optional timeline records [grid][COLI_TRACE_RECORDS][2], else null
  int trace_wgs;         // workgroups the trace buffer holds
  int *grid_out;         // host: receives the grid size when not null
};

// Timeline records (only when d.trace is set, by thread 0 of each
// workgroup): (code << 48 | value, s_memrealtime) at the boundaries of the
// kernel's phases and items; `n` counts the workgroup's records.
enum TraceCode : int {
  kTrEntry = 1, kTrSlices = 2, kTrXq = 3, kTrShDone = 4, kTrSelBegin = 5, kTrPollDone = 6,
  kTrSelEnd = 7, kTrGrEnd = 8, kTrDBegin = 9, kTrDReady = 10, kTrDEnd = 11, kTrExit = 12
};
// Compiled in only for the timeline build (COLI_DECODE_TRACE defined): in
// the library's ordinary build the records cost nothing.
__device__ __forceinline__ void trace_rec(const DecodeArgs &d, int &n, int code, int val) {
#ifdef COLI_DECODE_TRACE
  if (d.trace && threadIdx.x == 0 && n < COLI_TRACE_RECORDS && (int)blockIdx.x < d.trace_wgs) {
    uint64_t *p = d.trace + ((size_t)blockIdx.x * COLI_TRACE_RECORDS + n) * 2;
    p[0] = ((uint64_t)code << 48) | (uint32_t)val;
    p[1] = __builtin_amdgcn_s_memrealtime();
  }
  ++n;
#else
  (void)d, (void)n, (void)code, (void)val;
#endif
}

__device__ __forceinline__ uint32_t ld_ctr(const uint32_t *c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The thread index through an empty asm statement: address arithmetic on it
// stays inside the loop that uses it instead of being hoisted to the
// kernel's start, where its registers would be spilled for the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Every wave waits until its device-scope stores have completed, then one
// thread adds to the counter.
__device__ __forceinline__ void publish(uint32_t *c, uint32_t v) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polling rounds of a wait: the header's test-hook word, when nonzero, sets
// them (bits 0-30, at most the default `dflt`); with bit 31 set every wait
// of the call also treats its data as absent, so it runs the bound out and
// gives up (a failure forced from the host).  The result's bit 31 carries
// that flag.
__device__ __forceinline__ uint32_t spin_bound(const DecodeArgs &d, uint32_t dflt) {
  const uint32_t v = ld_ctr(d.ctr + kCtrSpin);
  if (v == 0u) return dflt;
  return min(v & 0x7FFFFFFFu, dflt & 0x7FFFFFFFu) | (v & 0x80000000u);
}
constexpr uint32_t kSpinForced = 0x80000000u;

// A bounded wait that ran out of polling rounds: record it (the call's
// outputs are undefined).
__device__ __forceinline__ void gave_up(const DecodeArgs &d, uint32_t what) {
  __hip_atomic_fetch_or(d.ctr + kCtrStatus, what, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Logit slice s = e * P + p: the binary64 sum of x[c] * gate_w[e][c] over
// the p-th of P equal column ranges, split over the waves (each lane's
// products summed in binary64, then the wave's lanes, then the waves in
// order), published as one 64-bit device-scope store.  issue() requests the
// slice's gate and x values; finish() sums and publishes.
struct SliceGate {
  static constexpr int kMaxPer = 4;  // float4 per lane: H / (P * 4 * waves * 64) <= 4 for H <= 8192
  float4 wv[kMaxPer], xv[kMaxPer];

  __device__ __forceinline__ void range(const DecodeArgs &d, int s, int &c0, int &cn) const {
    const int wave = threadIdx.x >> 6;
    const int P = d.n_part, pp = s % P;
    const int q4 = d.f.L.H / (4 * P);                  // float4 in the slice
    const int qw = (q4 + kDecWaves - 1) / kDecWaves;   // float4 per wave
    c0 = pp * q4 + wave * qw;
    cn = min(qw, q4 - wave * qw);                      // this wave's float4 (may be <= 0)
  }
  __device__ __forceinline__ void issue(const DecodeArgs &d, int s) {
    const int lane = threadIdx.x & 63;
    int c0, cn;
    range(d, s, c0, cn);
    const float4 *wr = reinterpret_cast<const float4 *>(d.gate_w + (size_t)(s / d.n_part) * d.f.L.H);
    const float4 *xr = reinterpret_cast<const float4 *>(d.x);
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (lane + 64 * i < cn) {
        wv[i] = wr[c0 + lane + 64 * i];
        xv[i] = xr[c0 + lane + 64 * i];
      }
    }
  }
  __device__ __forceinline__ void finish(const DecodeArgs &d, int s, double *part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int c0, cn;
    range(d, s, c0, cn);
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (lane + 64 * i < cn) {
        acc = fma((double)xv[i].x, (double)wv[i].x, acc);
        acc = fma((double)xv[i].y, (double)wv[i].y, acc);
        acc = fma((double)xv[i].z, (double)wv[i].z, acc);
        acc = fma((double)xv[i].w, (double)wv[i].w, acc);
      }
    }
    const double ws = wave_sum_f64(acc);
    if (lane == 0) part[wave] = ws;
    __syncthreads();
    if (threadIdx.x == 0) {
      double sum = part[0];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) sum += part[w];
      __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + s,
                         ~(uint64_t)__double_as_longlong(sum), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
};

// The token's router scores into LDS: the logits from the slices' partials
// polled in the header until every one has been written (bounded: a lost
// word leaves garbage, never a hang), added in column order in binary64 and
// rounded once (plus the layer's offset, if any), or the supplied logits;
// then sigma (binary64, rounded once) and c = sigma + bias.  issue()
// requests every partial of the thread's expert once (threads that call
// it); finish() requests the rest, polls what was absent, computes the
// scores, and ends with a barrier.  `lsave` (or null) keeps the logits for
// the caller.  Threads cover experts e, e + NT, ....  Token `tok` of a
// small batch: its logits row of the supplied ones, its partial words after
// those of the tokens before it.
struct ScorePoll {
  uint64_t v[kMaxPartsPerRow];

  bool have = false;  // the first round's words were requested by issue()

  __device__ __forceinline__ void issue(const DecodeArgs &d, int tok = 0) {
    const int e = threadIdx.x, P = d.n_part;
    if (d.logits_in || e >= d.f.cfg.E) return;
    have = true;
    const uint64_t *w = reinterpret_cast<const uint64_t *>(d.ctr + kScoreWords) + ((size_t)tok * d.f.cfg.E + e) * P;
#pragma unroll
    for (int p = 0; p < kMaxPartsPerRow; ++p)
      if (p < P) v[p] = __hip_atomic_load(w + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ __forceinline__ void finish(const DecodeArgs &d, SelInput &in, float *lsave, int tok = 0) {
    const RouterCfg &cfg = d.f.cfg;
    const int P = d.n_part;
    for (int e = threadIdx.x; e < cfg.E; e += kDecThreads) {
      float l;
      if (d.logits_in) {
        l = d.logits_in[(size_t)tok * cfg.E + e];
      } else {
        const uint64_t *w = reinterpret_cast<const uint64_t *>(d.ctr + kScoreWords) + ((size_t)tok * cfg.E + e) * P;
        if (e >= kDecThreads || !have) {  // words not requested by issue(): requested now
#pragma unroll
          for (int p = 0; p < kMaxPartsPerRow; ++p)
            if (p < P) v[p] = __hip_atomic_load(w + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t sb = spin_bound(d, kSpinLimit);
        const uint32_t spin = sb & ~kSpinForced;
        const bool forced = (sb & kSpinForced) != 0u;
        double sum = 0.0;
#pragma unroll
        for (int p = 0; p < kMaxPartsPerRow; ++p) {
          if (p < P) {
            uint32_t it = 0;
            while ((v[p] == 0ull || forced) && it < spin) {
              __builtin_amdgcn_s_sleep(2);
              v[p] = __hip_atomic_load(w + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              ++it;
            }
            if (v[p] == 0ull || forced) gave_up(d, COLI_WAIT_SCORES);
            const double part = __longlong_as_double((long long)~v[p]);
            sum = p == 0 ? part : sum + part;
          }
        }
        l = (float)sum;
        if (d.f.loff) l += d.f.loff[e];
      }
      if (lsave) lsave[e] = l;
      const float sg = sigmoid_f64(l);
      in.sg[e] = sg;
      in.c[e] = sg + (d.f.bias ? d.f.bias[e] : 0.f);
    }
    __syncthreads();
  }
};

// The token's experts and weights into LDS (sidx, sw) from the scores in
// `in`, by the whole workgroup (select_fast, else select_wg: the same total
// order and binary32 operations as select_token); slots that are not valid
// expert ids become -1.
__device__ __forceinline__ void select_local(const DecodeArgs &d, const SelInput &in,
                                             unsigned char *sel, int32_t *sidx, float *sw) {
  const RouterCfg &cfg = d.f.cfg;
  if (select_fast_ok(cfg.E, cfg.n_group, cfg.topk_group, cfg.k, kDecThreads))
    select_fast<kDecThreads>(cfg, in, *reinterpret_cast<SelFastScratch *>(sel), sidx, sw);
  else
    select_wg<kDecThreads>(cfg, in, *reinterpret_cast<SelWgScratch *>(sel), sidx, sw);
  for (int j = threadIdx.x; j < d.f.k; j += kDecThreads)
    if ((unsigned)sidx[j] >= (unsigned)cfg.E) sidx[j] = -1;  // never index outside the experts
  __syncthreads();
}

// The shared expert's gate/up rows [r0, r0 + nr) of this workgroup, in
// passes of RPP rows per wave: g and u summed in binary64 and rounded once,
// h = SwiGLU, stored in binary32 to hsh with device-scope stores.  The
// shared expert needs no routing, so issue() requests the first pass's
// weights before the router's scores are polled and the experts selected,
// and finish() computes (and loads any further pass) once the selection is
// done: the rows stream while the selection's latency runs.  The workgroup
// counts its rows in the shared slot's counter once its stores have
// completed (with its first gate/up item's counter, or on its own), and
// every D item quantises the shared h to Q8_0 itself.
template <int BITS, int LPR, int CPL>
struct SharedRows {
  static constexpr int RPP = 64 / LPR;
  uint4 wg[CPL], wu[CPL];

  __device__ __forceinline__ void load(const DecodeArgs &d, int row) {
    const int H = d.f.L.H, gl = (threadIdx.x & 63) % LPR;
    const int nchunks = H * BITS / 128;
    const size_t row_bytes = (size_t)H * BITS / 8;
    const ExpertPtrs ep = expert_ptrs(d.f.L, -1);
    const uint4 *gp = reinterpret_cast<const uint4 *>(ep.wg + (size_t)row * row_bytes);
    const uint4 *up = reinterpret_cast<const uint4 *>(ep.wu + (size_t)row * row_bytes);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = min(gl + LPR * i, nchunks - 1);
      wg[i] = ld_nt(gp + c);
      wu[i] = ld_nt(up + c);
    }
  }
  // a row past the range recomputes the last, unused
  __device__ __forceinline__ int row_of(const DecodeArgs &d, int r0, int rp) const {
    return min(r0 + rp + (int)(threadIdx.x & 63) / LPR, d.f.L.I - 1);
  }
  __device__ __forceinline__ void issue(const DecodeArgs &d, int r0, int nr) {
    const int rp = (int)(threadIdx.x >> 6) * RPP;
    if (rp < nr) load(d, row_of(d, r0, rp));
  }
  __device__ __forceinline__ void finish(const DecodeArgs &d, int r0, int nr, const int8_t *xq,
                                         const float *xd) {
    const int H = d.f.L.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gl = lane % LPR, rsub = lane / LPR;
    const int nchunks = H * BITS / 128;
    const ExpertPtrs ep = expert_ptrs(d.f.L, -1);
    Act<BITS> act[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + LPR * i;
      if (c < nchunks) load_act<BITS>(act[i], xq, xd, c);
      else zero_act<BITS>(act[i]);
    }
    for (int rp = wave * RPP; rp < nr; rp += kDecWaves * RPP) {
      const int row = row_of(d, r0, rp);
      if (rp != wave * RPP) load(d, row);
      double pg = 0.0, pu = 0.0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        pg += chunk_part_f64<BITS>(wg[i], act[i]);
        pu += chunk_part_f64<BITS>(wu[i], act[i]);
      }
      pg = group_sum_f64<LPR>(pg);
      pu = group_sum_f64<LPR>(pu);
      if (lane == group_sum_lane<LPR>(lane) && rp + rsub < nr) {
        const float h = swiglu_h(row_out(pg, ep.sg[row]), row_out(pu, ep.su[row]));
        st_dev(reinterpret_cast<uint32_t *>(d.hsh) + row, __float_as_uint(h));
      }
    }
  }
};

// The shared expert's h (binary32, hsh, complete) as Q8_0 codes in the
// container ordering and block scales, into LDS: 4 values per thread, the 8
// threads of a 32-value block together (amax, then amax / 127 and the codes
// rounded to nearest even, as every other Q8_0 step of the layer).
template <int BITS>
__device__ __forceinline__ void quantize_shared_h(const DecodeArgs &d, int8_t *q, float *dsc) {
  const int I = d.f.L.I;
  const int tid = opaque_tid();
  const int part = tid & 7;
  for (int i0 = 4 * tid; i0 < I; i0 += 4 * kDecThreads) {
    const uint64_t *src = reinterpret_cast<const uint64_t *>(d.hsh + i0);
    const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float e[4] = {__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                        __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
    float m = fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3])));
    m = group_max<8>(m);
    const float db = m / 127.f;
    const int blk = i0 / 32;
    if (part == 0) dsc[blk] = db;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c = 0.f;
      if (db != 0.f) c = fminf(fmaxf(rintf(e[j] / db), -127.f), 127.f);
      q[(size_t)blk * 32 + perm_dst<BITS>(4 * part + j)] = (int8_t)c;
    }
  }
}

// D item: output rows [r0, r0 + down_rows).  Wave w owns rows
// r0 + w*PR .. r0 + w*PR + PR-1 (PR = NPASS * RPP) for every slot, so it
// combines y = o_shared + sum_j w_j * o_j itself: each lane accumulates its
// chunks' share of every slot (shared first, then slots 0 .. k-1), and the
// lanes of a row are summed once at the end -- a fixed order, so the result
// is reproducible.
template <int BITS, int LPR, int CPL, int NPASS, int SG>
__device__ __forceinline__ void down_rows(const DecodeArgs &d, int r0, int8_t *lds_q, float *lds_d,
                                          const int32_t *sidx, const float *sw, int &trn) {
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
    // once every gate/up item of the group's slots is done (the shared
    // slot: every row of h), stage their h codes and scales in LDS
    // (device-scope loads, all in flight together); the shared h is
    // quantised here from binary32
    if ((int)threadIdx.x < gn) {
      const int q = threadIdx.x;
      const int sl = g0 + q == 0 ? k : g0 + q - 1;
      const uint32_t *c = d.ctr + kCtrSlot0 + sl * kCtrStride;
      const uint32_t target = (uint32_t)(sl == k ? I : I / kGuRows);
      const uint32_t sb = spin_bound(d, 8u * kSpinLimit);
      const uint32_t spin = sb & ~kSpinForced;
      const bool forced = (sb & kSpinForced) != 0u;
      uint32_t it = 0, v;
      while (((v = ld_ctr(c)) < target || forced) && it < spin) {
        __builtin_amdgcn_s_sleep(8);
        ++it;
      }
      if (v < target || forced) gave_up(d, COLI_WAIT_SLOTS);
    }
    __syncthreads();
    if (g0 == 0) trace_rec(d, trn, kTrDReady, r0);
    // the staged slots: [q_lo, gn) (slot 0 of the first group is the shared
    // expert's, quantised below)
    const int q_lo = g0 == 0 ? 1 : 0;
    if (I % 128 == 0) {
      // straight into LDS: 16-byte loads with the cache policy of the
      // device-scope loads (sc1), all in flight at once and no registers.
      // One wave instruction fills 64 consecutive 16-byte LDS chunks.
      const int cq = I / 16, cd = I / 128;  // chunks of codes / of scales per slot
      const int nA = (gn - q_lo) * cq, nB = (gn - q_lo) * cd;
      const int nwA = (nA + 63) / 64, nwB = (nB + 63) / 64;
      for (int ii = wave; ii < nwA + nwB; ii += kDecWaves) {
        const bool codes = ii < nwA;
        const int base = (codes ? ii : ii - nwA) * 64;
        const int c = base + lane, per = codes ? cq : cd;
        unsigned char *dst = (codes ? reinterpret_cast<unsigned char *>(lds_q)
                                    : reinterpret_cast<unsigned char *>(lds_d)) +
                             ((size_t)q_lo * per + base) * 16;
        if (c < (codes ? nA : nB)) {
          const int q = q_lo + c / per, r = c - (q - q_lo) * per;
          const int sl = g0 + q == 0 ? k : g0 + q - 1;
          const unsigned char *src =
              codes ? reinterpret_cast<const unsigned char *>(a.hq) + (size_t)sl * I + r * 16
                    : reinterpret_cast<const unsigned char *>(a.hd) + (size_t)sl * (I / 8) + r * 16;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0,
                                           kLoadSc1);
        }
      }
      if (q_lo) quantize_shared_h<BITS>(d, lds_q, lds_d);
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      if (q_lo) quantize_shared_h<BITS>(d, lds_q, lds_d);
      // 64-bit device-scope loads, kStage per thread issued before any is
      // written to LDS
      constexpr int kStage = 2;
      const int wq = I / 8, wd = I / 64;  // 8-byte words of codes and scales per slot
      const int n = (gn - q_lo) * (wq + wd);
      const int tid = opaque_tid();
      for (int i0 = 0; i0 < n; i0 += kStage * kDecThreads) {
        uint64_t v[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
          const int i = i0 + j * kDecThreads + tid;
          v[j] = 0;
          if (i < n) {
            const int q = q_lo + i / (wq + wd), r = i - (q - q_lo) * (wq + wd);
            const int sl = g0 + q == 0 ? k : g0 + q - 1;
            const uint64_t *src = r < wq ? reinterpret_cast<const uint64_t *>(a.hq + (size_t)sl * I) + r
                                         : reinterpret_cast<const uint64_t *>(a.hd + (size_t)sl * (I / 32)) + (r - wq);
            v[j] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
          const int i = i0 + j * kDecThreads + tid;
          if (i < n) {
            const int q = q_lo + i / (wq + wd), r = i - (q - q_lo) * (wq + wd);
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

// Persistent: the grid is at most the workgroups the GPU holds at once.
// Every workgroup first computes its logit slices, quantises x into its LDS
// and requests its share of the shared expert's gate/up rows (none of which
// needs the routing), then selects the token's experts itself, finishes the
// shared rows and takes tickets: GR items (with a full grid, exactly one
// per workgroup), then D items.  A D item stages h in the region the
// selection scratch used.
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
  // dynamic LDS: [selection scratch, later a D item's staged h | x's Q8_0
  // codes and scales | the logits kept for the caller]
  extern __shared__ __align__(16) unsigned char dyn[];
  const FfnArgs &a = d.f;
  const int k = a.k, I = a.L.I, H = a.L.H;
  const int n_rb = I / kGuRows;
  const int b_d = d.n_gr;
  int8_t *xq_lds = reinterpret_cast<int8_t *>(dyn + d.lds_x);
  float *xd_lds = reinterpret_cast<float *>(dyn + d.lds_x + H);
  float *lsave = d.lds_l >= 0 ? reinterpret_cast<float *>(dyn + d.lds_l) : nullptr;

  // Work queue q = b % 8 holds items q, q + 8, ...; consecutive workgroups
  // go to consecutive XCDs, so each XCD streams an equal share of every
  // kind of item.  Within a queue the items keep their global order.
  // A workgroup's first item is its own index (queue q's nq workgroups take
  // its first nq items in order), which saves the first atomic round trip;
  // later tickets come from the queue's counter, offset by nq.
  const int q = blockIdx.x % kQueues;
  const int nq = ((int)gridDim.x - q + kQueues - 1) / kQueues;
  // A counter value past the queue's items (a header the caller did not
  // zero) ends the loop: the item index is formed in 64 bits and clamped,
  // so no value of the header can yield an index outside [0, total].
  auto next_ticket = [&]() -> int {
    if (threadIdx.x == 0)
      s_ticket = (int)__hip_atomic_fetch_add(d.ctr + kCtrTicket + q * kCtrStride, 1u,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t tk = (uint32_t)uniform_i32(s_ticket);
    const long long tt = (long long)q + (long long)kQueues * ((long long)nq + (long long)tk);
    __syncthreads();
    return tt < (long long)d.total ? (int)tt : d.total;
  };

  int trn = 0;
  trace_rec(d, trn, kTrEntry, 0);
  // router logits first: this workgroup's slices
  {
    SliceGate sg;
    for (int sl = (int)blockIdx.x; sl < d.n_slice; sl += gridDim.x) {
      sg.issue(d, sl);
      sg.finish(d, sl, lpart);
    }
  }
  trace_rec(d, trn, kTrSlices, 0);
  // then x's Q8_0 codes into LDS, this workgroup's rows of the shared expert
  // (which needs no routing), the router's scores and the token's experts,
  // by the whole workgroup
  SelInput &in = *reinterpret_cast<SelInput *>(dyn);
  {
    ActRow<BITS, kDecThreads> xr;
    xr.load(d.x, H);
    xr.quantize(H, xq_lds, xd_lds);
  }
  __syncthreads();
  trace_rec(d, trn, kTrXq, 0);
  // this workgroup's rows of the shared expert stream while the scores are
  // polled and the experts selected
  const int sh_r0 = (int)blockIdx.x * d.sh_rows;
  const int sh_nr = max(0, min(d.sh_rows, I - sh_r0));
  SharedRows<BITS, GLPR, GCPL> shr;
  shr.issue(d, sh_r0, sh_nr);
  trace_rec(d, trn, kTrSelBegin, 0);
  {
    ScorePoll sp;
    sp.issue(d);
    sp.finish(d, in, lsave);
  }
  trace_rec(d, trn, kTrPollDone, 0);
  select_local(d, in, dyn + sizeof(SelInput), sidx, sw);
  trace_rec(d, trn, kTrSelEnd, 0);
  shr.finish(d, sh_r0, sh_nr, xq_lds, xd_lds);
  trace_rec(d, trn, kTrShDone, 0);

  // the shared rows are counted once their stores have completed: with the
  // first gate/up item's counter, else on their own before the D items
  bool sh_counted = sh_nr == 0;
  int t = (int)blockIdx.x;
  // GR: routed slot u, rows [kGuRows rb, +kGuRows)
  for (; t < b_d; t = next_ticket()) {
    const int u = t / n_rb, rb = t % n_rb;
    if (u == 0 && rb == 0) {
      for (int j = threadIdx.x; j < k; j += kDecThreads) {
        if (a.idx_user) a.idx_user[j] = sidx[j];
        if (a.w_user) a.w_user[j] = sw[j];
      }
      if (lsave && d.logits_out)
        for (int e = threadIdx.x; e < a.E; e += kDecThreads) d.logits_out[e] = lsave[e];
    }
    const int e = uniform_i32(sidx[u]);
    if (e >= 0) {
      TokList s{1, -1, u, false};
      gateup_body<BITS, GLPR, GCPL, 1, kDecWaves, true, BLK, kGuPipe>(a, false, expert_ptrs(a.L, e), s,
                                                                     BLK * rb, hs, xq_lds, xd_lds);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(d.ctr + kCtrSlot0 + u * kCtrStride, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      if (!sh_counted)
        __hip_atomic_fetch_add(d.ctr + kCtrSlot0 + k * kCtrStride, (uint32_t)sh_nr,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    sh_counted = true;
    trace_rec(d, trn, kTrGrEnd, t);
  }
  if (!sh_counted) publish(d.ctr + kCtrSlot0 + k * kCtrStride, (uint32_t)sh_nr);
  // D: output rows of D item t - b_d; the staged h overlays the selection
  // scratch, which is no longer needed by then
  int8_t *lds_q = reinterpret_cast<int8_t *>(dyn);
  float *lds_d = reinterpret_cast<float *>(dyn + (size_t)d.slot_group * I);
  for (; t < d.total; t = next_ticket()) {
    trace_rec(d, trn, kTrDBegin, t);
    down_rows<BITS, DLPR, DCPL, DNPASS, DSG>(d, (t - b_d) * d.down_rows, lds_q, lds_d, sidx, sw,
                                            trn);
    trace_rec(d, trn, kTrDEnd, t);
  }
  trace_rec(d, trn, kTrExit, 0);

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
    for (int sl = threadIdx.x; sl < d.n_slice; sl += kDecThreads)
      __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + sl, (uint64_t)0,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ===========================================================================
// Small batches (2 to 4 tokens: an MTP verify of the current token and its
// drafts) as ONE kernel, the batch union of the decode kernel's design.
//
// colibrì README, "Implemented features", native MTP item: the drafts are
// verified in one batched forward, where each unique expert of the batch is
// read once for every token that picked it (batch-union item).
//
// Per call, in order:
//   logit slices (computed logits): one gate row per slice for every token
//     (P = 1), each token's binary64 partial in its own header word;
//   workgroup t < T: token t's scores and experts (select_local), written to
//     the workspace's idx / w rows and counted in the selection counter
//     (first, so the union waits as little as possible for it);
//   every workgroup: the tokens' Q8_0 codes into LDS, then, once T
//     selections are counted, the batch's union in LDS: the (token, slot)
//     pairs sorted by (expert, pair), so the experts' runs are consecutive
//     and each pair's h row is its position;
//   tickets: GR items (a 32-row block of the shared expert for every token,
//     then of each unique expert u for the tokens of u), then D items (a
//     block of output rows for every token: the shared expert first, then
//     the unique experts in order, each token's contributions weighted and
//     summed in that fixed order).
// Slot counters: unique expert u on line u, the shared expert on line
// kSelMaxK; the waits, give-ups, status word and header reset are the
// decode kernel's.
// ===========================================================================
constexpr int kSmallMaxT = 4;
constexpr int kSmallPipe = 1;  // gate/up row passes in flight per wave
// D items: row passes per wave, experts whose weights are in flight together
constexpr int small_dpass(int dcpl) { return dcpl == 1 ? 2 : 1; }
// D items: units (an expert's rows) per group, whose weights are in flight
// together, and the h rows staged for them (at most 12, so two workgroups
// still fit a CU's LDS)
constexpr int small_dsg(int dcpl, int t) { return dcpl == 1 ? 6 : 2; }
constexpr int small_drows(int dcpl, int t) { return dcpl == 1 ? 12 : 2 * t; }
constexpr int kCtrSel = kCtrSpin + 16;  // selections published (a word of the polling-bound line)
constexpr int kShLine = kSelMaxK;       // the shared expert's slot counter line

// The batch union, built by every workgroup from the published selections.
struct SmallUnion {
  int n_pairs, n_valid, U;
  int pidx[kSelMaxK];    // expert of pair l = t * k + j (-1: none)
  float pw[kSelMaxK];    // weight of pair l
  int sorted[kSelMaxK];  // pair at h row r
  int ue[kSelMaxK + 1];  // where unique u's weights are stored (expert_store)
  int ufirst[kSelMaxK + 1];  // first h row of unique u (ufirst[U] = n_valid)
};

template <int T>
__device__ __forceinline__ void small_union(const DecodeArgs &d, SmallUnion &su) {
  const FfnArgs &a = d.f;
  const int n = T * a.k, E = a.E;
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < n) {
    const int e = (int)ld_dev(reinterpret_cast<const uint32_t *>(a.idx) + tid);
    su.pidx[tid] = (e >= 0 && e < E) ? e : -1;
    su.pw[tid] = __uint_as_float(ld_dev(reinterpret_cast<const uint32_t *>(a.w) + tid));
  }
  __syncthreads();
  if (tid < 64) {
    // rank of pair l among keys (expert, l), invalid pairs last
    const bool in = lane < n;
    const int e = in ? su.pidx[lane] : -1;
    const int key = in ? (e >= 0 ? e * 64 + lane : E * 64 + lane) : 0x7FFFFFFF;
    int rank = 0;
    for (int m = 0; m < n; ++m) {
      const int em = su.pidx[m];
      const int km = em >= 0 ? em * 64 + m : E * 64 + m;
      rank += km < key ? 1 : 0;
    }
    if (in) su.sorted[rank] = lane;
  }
  __syncthreads();
  if (tid < 64) {
    const bool in = lane < n;
    const int e = in ? su.pidx[su.sorted[lane]] : -1;
    const int ep = (in && lane > 0) ? su.pidx[su.sorted[lane - 1]] : -2;
    const bool valid = e >= 0;
    const bool first = valid && e != ep;
    const uint64_t bf = __ballot(first), bv = __ballot(valid);
    const int u = __popcll(bf & ((1ull << lane) - 1ull));
    if (first) {
      su.ue[u] = expert_store(a.L, e);
      su.ufirst[u] = lane;
    }
    if (lane == 0) {
      su.U = __popcll(bf);
      su.n_valid = __popcll(bv);
      su.n_pairs = n;
      su.ufirst[__popcll(bf)] = __popcll(bv);
    }
  }
  __syncthreads();
}

// Logit slice e (P = 1): the binary64 sums x_t . gate_w[e] of every token,
// split over the waves as SliceGate does.
template <int T>
__device__ __forceinline__ void small_slice(const DecodeArgs &d, int e, double (*part)[kDecWaves]) {
  constexpr int kMaxPer = SliceGate::kMaxPer;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = d.f.L.H, E = d.f.cfg.E;
  const int q4 = H / 4, qw = (q4 + kDecWaves - 1) / kDecWaves;
  const int c0 = wave * qw, cn = min(qw, q4 - wave * qw);
  const float4 *wr = reinterpret_cast<const float4 *>(d.gate_w + (size_t)e * H);
  float4 wv[kMaxPer], xv[T][kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    if (lane + 64 * i < cn) {
      wv[i] = wr[c0 + lane + 64 * i];
#pragma unroll
      for (int t = 0; t < T; ++t)
        xv[t][i] = reinterpret_cast<const float4 *>(d.x + (size_t)t * H)[c0 + lane + 64 * i];
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (lane + 64 * i < cn) {
        acc = fma((double)xv[t][i].x, (double)wv[i].x, acc);
        acc = fma((double)xv[t][i].y, (double)wv[i].y, acc);
        acc = fma((double)xv[t][i].z, (double)wv[i].z, acc);
        acc = fma((double)xv[t][i].w, (double)wv[i].w, acc);
      }
    }
    const double ws = wave_sum_f64(acc);
    if (lane == 0) part[t][wave] = ws;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    double sum = part[t][0];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) sum += part[t][w];
    __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + (size_t)t * E + e,
                       ~(uint64_t)__double_as_longlong(sum), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// D item: output rows [r0, r0 + down_rows) for every token.  "Experts" in
// order: x = 0 the shared one (its T rows at k*T), then unique u = x - 1
// (its pairs' rows ufirst[u] .. ufirst[u+1]-1).  They are taken in groups
// of at most SG units of at most SG*T staged h rows in all (a unit: some
// consecutive rows of one expert; an expert normally has at most T pairs,
// but a token may repeat an expert); wave w owns rows r0 + w*PR .. for
// every expert and token.  Each (token, slot) output
// row is the union path's: its lanes' chunk products summed, times the row
// scale; they are kept in LDS (ob) and combined per token in slot order as
// the union path's combine does, so both paths give the same bits.
constexpr int kSmallObRows = 32;  // output rows per D item, at most
template <int BITS, int LPR, int CPL, int NPASS, int SG, int RW, int T>
__device__ __forceinline__ void small_down_rows(const DecodeArgs &d, const SmallUnion &su, int r0,
                                                int8_t *lds_q, float *lds_d, int *srow,
                                                float (*ob)[kSmallObRows]) {
  const int tid = opaque_tid();
  constexpr int RPP = 64 / LPR;
  const FfnArgs &a = d.f;
  const int I = a.L.I, H = a.L.H, k = a.k, hr0 = k * T;
  const int lane = tid & 63, wave = tid >> 6;
  const int gl = lane % LPR, rsub = lane / LPR;
  const int nchunks = I * BITS / 128;
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int nx = su.U + 1;
  const int wrow0 = r0 + wave * NPASS * RPP;
  static_assert(kDecWaves * NPASS * RPP <= kSmallObRows, "output rows per D item");

  constexpr int R = RW;  // staged rows per group
  int nxt = 0, nxr = 0;      // next expert and its next row
  while (nxt < nx) {
    // the next group: units (expert ux[q], its rows [rbeg[q], + rcnt[q]))
    int ux[SG], rbeg[SG], rcnt[SG], nrows = 0, gn = 0;
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      ux[q] = 0;
      rbeg[q] = 0;
      rcnt[q] = 0;
      if (nxt < nx && nrows < R) {
        const int cnt = nxt == 0 ? T : su.ufirst[nxt] - su.ufirst[nxt - 1];
        const int take = min(cnt - nxr, R - nrows);
        ux[q] = nxt;
        rbeg[q] = (nxt == 0 ? hr0 : su.ufirst[nxt - 1]) + nxr;
        rcnt[q] = take;
        nrows += take;
        gn = q + 1;
        nxr += take;
        if (nxr == cnt) {
          ++nxt;
          nxr = 0;
        }
      }
    }
    uint4 wv[SG][NPASS][CPL];
    float sdv[SG][NPASS];
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      if (q < gn) {
        const int x = ux[q];
        const ExpertPtrs ep = expert_ptrs_at(a.L, x == 0 ? -1 : su.ue[x - 1]);
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
    if (tid < gn) {
      int x = 0;
#pragma unroll
      for (int q = 0; q < SG; ++q)
        if (q == tid) x = ux[q];
      const uint32_t *c = d.ctr + kCtrSlot0 + (x == 0 ? kShLine : x - 1) * kCtrStride;
      const uint32_t target = (uint32_t)(I / kGuRows);
      const uint32_t sb = spin_bound(d, 8u * kSpinLimit);
      const uint32_t spin = sb & ~kSpinForced;
      const bool forced = (sb & kSpinForced) != 0u;
      uint32_t it = 0, v;
      while (((v = ld_ctr(c)) < target || forced) && it < spin) {
        __builtin_amdgcn_s_sleep(8);
        ++it;
      }
      if (v < target || forced) gave_up(d, COLI_WAIT_SLOTS);
    }
    if (tid == 0) {
      int n = 0;
#pragma unroll
      for (int q = 0; q < SG; ++q)
        for (int r = 0; r < rcnt[q]; ++r) srow[n++] = rbeg[q] + r;
    }
    __syncthreads();
    {
      // staged rows g = 0 .. nrows-1: codes then scales, 16-byte pieces
      // straight into LDS with the device-scope loads' cache policy
      const int cq = I / 16, cd = I / 128;
      const int nA = nrows * cq, nB = nrows * cd;
      const int nwA = (nA + 63) / 64, nwB = (nB + 63) / 64;
      for (int ii = wave; ii < nwA + nwB; ii += kDecWaves) {
        const bool codes = ii < nwA;
        const int base = (codes ? ii : ii - nwA) * 64;
        const int c = base + lane, per = codes ? cq : cd;
        unsigned char *dst = (codes ? reinterpret_cast<unsigned char *>(lds_q)
                                    : reinterpret_cast<unsigned char *>(lds_d)) + (size_t)base * 16;
        if (c < (codes ? nA : nB)) {
          const int g = c / per, r = c - g * per;
          const int hrow = srow[g];
          const unsigned char *src =
              codes ? reinterpret_cast<const unsigned char *>(a.hq) + (size_t)hrow * I + r * 16
                    : reinterpret_cast<const unsigned char *>(a.hd) + (size_t)hrow * (I / 8) + r * 16;
          __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0,
                                           kLoadSc1);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    int g = 0;
#pragma unroll
    for (int q = 0; q < SG; ++q) {
      for (int r = 0; r < rcnt[q]; ++r, ++g) {
        // the pair's token and slot (the shared expert: token r, slot k)
        const int x = ux[q];
        const int pair = x == 0 ? -1 : su.sorted[rbeg[q] + r];
        const int tok = x == 0 ? rbeg[q] - hr0 + r : pair / k;
        const int slot = x == 0 ? k : pair % k;
        Act<BITS> act[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = gl + LPR * i;
          if (c < nchunks) load_act<BITS>(act[i], lds_q + (size_t)g * I, lds_d + g * (I / 32), c);
          else zero_act<BITS>(act[i]);
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) acc += chunk_part<BITS>(wv[q][p][i], act[i]);
          acc = group_sum<LPR>(acc);
          if (lane == group_sum_lane<LPR>(lane))
            ob[tok * (k + 1) + slot][wrow0 - r0 + p * RPP + rsub] = acc * sdv[q][p];
        }
      }
    }
    __syncthreads();
  }
  // y = o_shared + the kept slots' w * o in slot order, one thread per
  // (token, row)
  const int rows = kDecWaves * NPASS * RPP;
  for (int i = tid; i < T * rows; i += kDecThreads) {
    const int t = i / rows, rl = i % rows;
    float y = ob[t * (k + 1) + k][rl];
    for (int j = 0; j < k; ++j) {
      if (su.pidx[t * k + j] < 0) continue;
      y += su.pw[t * k + j] * ob[t * (k + 1) + j][rl];
    }
    a.y[(size_t)t * H + r0 + rl] = y;
  }
  __syncthreads();
}

// GR item: unique expert u's gate/up rows [32 rb, +32) for its n tokens
// (h rows ufirst[u] ..), or with u < 0 the shared expert's for all n_sh
// tokens (h rows k * n_sh + t): the gate/up body with the tokens in a runtime loop
// whose activations are re-read from LDS per row pass, so a pass holds only
// its rows' weights (PIPE passes in flight) -- few registers at any n.
template <int BITS, int LPR, int CPL, int PIPE>
__device__ __forceinline__ void small_gateup(const DecodeArgs &d, const SmallUnion &su, int u, int rb,
                                             float (*hs)[kGuRows], float (*hu)[kGuRows],
                                             int8_t (*hcode)[kGuRows], const int8_t *xq,
                                             const float *xd, int n_sh) {
  const int tid = opaque_tid();
  static_assert(kGuRows == 32, "one Q8_0 block of h per item");
  constexpr int RPP = 64 / LPR;
  constexpr int ROWS_PER_WAVE = kGuRows / kDecWaves;
  constexpr int PASSES = ROWS_PER_WAVE / RPP;
  const FfnArgs &a = d.f;
  const int H = a.L.H, I = a.L.I;
  const int lane = tid & 63, wave = tid >> 6;
  const int gl = lane % LPR, rsub = lane / LPR;
  const int nchunks = H * BITS / 128;
  const size_t row_bytes = (size_t)H * BITS / 8;
  const int xblocks = H / 32;
  const bool shared = u < 0;
  const int h0 = shared ? a.k * n_sh : su.ufirst[u];
  const int n_tok = shared ? n_sh : su.ufirst[u + 1] - h0;
  const ExpertPtrs ep = expert_ptrs_at(a.L, shared ? -1 : su.ue[u]);
  const int srow = rb * 32 + wave * ROWS_PER_WAVE + min(lane, ROWS_PER_WAVE - 1);
  const float sgv = ep.sg[srow], suv = ep.su[srow];
  uint4 wg[PIPE][CPL], wu[PIPE][CPL];
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
    const int rl = wave * ROWS_PER_WAVE + p * RPP + rsub;
    const float sg = row_scale<RPP>(sgv, p, rsub), su_ = row_scale<RPP>(suv, p, rsub);
    for (int n = 0; n < n_tok; ++n) {
      const int t = shared ? n : su.sorted[h0 + n] / a.k;
      const int8_t *xqt = xq + (size_t)t * H;
      const float *xdt = xd + (size_t)t * xblocks;
      double pg = 0.0, pu = 0.0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = gl + LPR * i;
        Act<BITS> act;
        if (c < nchunks) load_act<BITS>(act, xqt, xdt, c);
        else zero_act<BITS>(act);
        pg += chunk_part_f64<BITS>(wg[buf][i], act);
        pu += chunk_part_f64<BITS>(wu[buf][i], act);
      }
      pg = group_sum_f64<LPR>(pg);
      pu = group_sum_f64<LPR>(pu);
      if (lane == group_sum_lane<LPR>(lane)) {
        hs[n][rl] = row_out(pg, sg);
        hu[n][rl] = row_out(pu, su_);
      }
    }
    if (PIPE == 1 && p + 1 < PASSES) load_rows(p + 1, 0);
  }
  __syncthreads();
  // SwiGLU and Q8_0 of each token's 32 values of h: 32 threads per token
  for (int n0 = 0; n0 < n_tok; n0 += kDecThreads / 32) {
    const int n = n0 + (tid >> 5), i = tid & 31;
    if (n < n_tok) {
      const float h = swiglu_h(hs[n][i], hu[n][i]);
      float amax = group_max<32>(fabsf(h));
      amax = __shfl(amax, (lane & 32) | 31, 64);
      const float db = amax / 127.f;
      float c = 0.f;
      if (db != 0.f) c = fminf(fmaxf(rintf(h / db), -127.f), 127.f);
      hcode[n][perm_dst<BITS>(i)] = (int8_t)c;
      if (i == 0)
        st_dev(reinterpret_cast<uint32_t *>(a.hd) + (size_t)(h0 + n) * (I / 32) + rb, __float_as_uint(db));
    }
  }
  __syncthreads();
  {
    const int n = tid >> 3, i = tid & 7;
    if (n < n_tok)
      st_dev(reinterpret_cast<uint32_t *>(a.hq + (size_t)(h0 + n) * I + rb * 32) + i,
             reinterpret_cast<const uint32_t *>(hcode[n])[i]);
  }
}

template <int BITS, int GLPR, int GCPL, int DLPR, int DCPL, int T>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(BITS == 4 ? 4 : 2))) void k_small_fused(DecodeArgs d) {
  constexpr int DNPASS = small_dpass(DCPL);
  constexpr int DSG = small_dsg(DCPL, T);
  __shared__ SmallUnion su;
  // a GR item's g, u and h codes: one row per pair of its expert (at most
  // every pair of the batch, if the tokens repeat an expert)
  __shared__ float hs[kSelMaxK][kGuRows], hu[kSelMaxK][kGuRows];
  __shared__ __align__(16) int8_t hcode[kSelMaxK][kGuRows];
  __shared__ double lpart[kSmallMaxT][kDecWaves];
  __shared__ int s_ticket;
  constexpr int DRW = small_drows(DCPL, T);
  __shared__ int srow[DRW];
  __shared__ float ob[kSelMaxK + kSmallMaxT][kSmallObRows];  // a D item's (token, slot) rows
  __shared__ int32_t sidx[kSelMaxK];
  __shared__ float sw[kSelMaxK];
  // dynamic LDS: [selection scratch, later a D item's staged h | the tokens'
  // Q8_0 codes and scales | one token's logits kept for the caller]
  extern __shared__ __align__(16) unsigned char dyn[];
  const FfnArgs &a = d.f;
  const int k = a.k, I = a.L.I, H = a.L.H, E = a.E;
  const int n_rb = I / kGuRows;
  int8_t *xq_lds = reinterpret_cast<int8_t *>(dyn + d.lds_x);
  float *xd_lds = reinterpret_cast<float *>(dyn + d.lds_x + T * H);
  float *lsave = d.lds_l >= 0 ? reinterpret_cast<float *>(dyn + d.lds_l) : nullptr;

  // logit slices: gate row e for every token; workgroup t < T then selects
  // token t's experts; then the tokens' Q8_0 codes, the loads of up to three
  // tokens in flight together
  for (int e = (int)blockIdx.x; e < d.n_slice; e += gridDim.x) small_slice<T>(d, e, lpart);
  if ((int)blockIdx.x < T) {
    // token blockIdx.x: scores, experts, weights, published
    const int t = blockIdx.x;
    SelInput &in = *reinterpret_cast<SelInput *>(dyn);
    ScorePoll sp;
    sp.issue(d, t);
    sp.finish(d, in, lsave, t);
    select_local(d, in, dyn + sizeof(SelInput), sidx, sw);
    for (int j = threadIdx.x; j < k; j += kDecThreads) {
      st_dev(reinterpret_cast<uint32_t *>(a.idx) + t * k + j, (uint32_t)sidx[j]);
      st_dev(reinterpret_cast<uint32_t *>(a.w) + t * k + j, __float_as_uint(sw[j]));
      if (a.idx_user) a.idx_user[t * k + j] = sidx[j];
      if (a.w_user) a.w_user[t * k + j] = sw[j];
    }
    if (lsave && d.logits_out)
      for (int e = threadIdx.x; e < E; e += kDecThreads) d.logits_out[(size_t)t * E + e] = lsave[e];
    publish(d.ctr + kCtrSel, 1u);
    __syncthreads();
  }
  {
    constexpr int XB = T == 4 ? 2 : T;
#pragma unroll
    for (int t0 = 0; t0 < T; t0 += XB) {
      ActRow<BITS, kDecThreads> xr[XB];
#pragma unroll
      for (int t = 0; t < XB; ++t) xr[t].load(d.x + (size_t)(t0 + t) * H, H);
#pragma unroll
      for (int t = 0; t < XB; ++t)
        xr[t].quantize(H, xq_lds + (size_t)(t0 + t) * H, xd_lds + (size_t)(t0 + t) * (H / 32));
    }
  }
  __syncthreads();
  // every token's selection, then the union
  if (threadIdx.x == 0) {
    const uint32_t sb = spin_bound(d, kSpinLimit);
    const uint32_t spin = sb & ~kSpinForced;
    const bool forced = (sb & kSpinForced) != 0u;
    uint32_t it = 0, v;
    while (((v = ld_ctr(d.ctr + kCtrSel)) < (uint32_t)T || forced) && it < spin) {
      __builtin_amdgcn_s_sleep(2);
      ++it;
    }
    if (v < (uint32_t)T || forced) gave_up(d, COLI_WAIT_SCORES);
  }
  __syncthreads();
  small_union<T>(d, su);
  // GR items: the shared expert's row blocks (x = 0), then each unique
  // expert's (x = u + 1)
  const int n_gr = (su.U + 1) * n_rb;
  const int total = n_gr + d.n_down;

  const int q = blockIdx.x % kQueues;
  const int nq = ((int)gridDim.x - q + kQueues - 1) / kQueues;
  auto next_ticket = [&]() -> int {
    if (threadIdx.x == 0)
      s_ticket = (int)__hip_atomic_fetch_add(d.ctr + kCtrTicket + q * kCtrStride, 1u,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t tk = (uint32_t)uniform_i32(s_ticket);
    const long long tt = (long long)q + (long long)kQueues * ((long long)nq + (long long)tk);
    __syncthreads();
    return tt < (long long)total ? (int)tt : total;
  };

  int t = (int)blockIdx.x < total ? (int)blockIdx.x : total;
  for (; t < n_gr; t = next_ticket()) {
    const int u = t / n_rb - 1, rb = t % n_rb;
    small_gateup<BITS, GLPR, GCPL, kSmallPipe>(d, su, u, rb, hs, hu, hcode, xq_lds, xd_lds, T);
    publish(d.ctr + kCtrSlot0 + (u < 0 ? kShLine : u) * kCtrStride, 1u);
  }
  int8_t *lds_q = reinterpret_cast<int8_t *>(dyn);
  float *lds_d = reinterpret_cast<float *>(dyn + (size_t)DRW * I);
  for (; t < total; t = next_ticket())
    small_down_rows<BITS, DLPR, DCPL, DNPASS, DSG, DRW, T>(d, su, (t - n_gr) * d.down_rows, lds_q, lds_d, srow, ob);

  // the last workgroup out clears the header for the next call
  __syncthreads();
  if (threadIdx.x == 0)
    s_ticket = (int)__hip_atomic_fetch_add(d.ctr + kCtrExit, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (uniform_i32(s_ticket) == (int)gridDim.x - 1) {
    const int nc = kCtrSlot0 / kCtrStride + kSelMaxK + 1;
    for (int i = threadIdx.x; i < nc; i += kDecThreads)
      __hip_atomic_store(d.ctr + i * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      __hip_atomic_store(d.ctr + kCtrSpin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(d.ctr + kCtrSel, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int sl = threadIdx.x; sl < T * d.n_slice; sl += kDecThreads)
      __hip_atomic_store(reinterpret_cast<uint64_t *>(d.ctr + kScoreWords) + sl, (uint64_t)0,
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
  const int I = d.f.L.I, H = d.f.L.H, E = d.f.E;
  d.down_rows = kDecWaves * DNPASS * (64 / DLPR);
  if (H % d.down_rows) return hipErrorNotSupported;
  d.n_down = H / d.down_rows;
  // dynamic LDS: [max(selection scratch, staged h: I code bytes + I/32
  // scales a slot) | x's codes and scales | the logits kept for the caller]
  const int per_slot = I + (I / 32) * 4;
  d.slot_group = DSG;
  while (d.slot_group > 1 && d.slot_group * per_slot > 24 * 1024) --d.slot_group;
  const size_t sel =
      (sizeof(SelInput) + std::max(sizeof(SelWgScratch), sizeof(SelFastScratch)) + 15) / 16 * 16;
  const size_t reg_a = (std::max(sel, (size_t)d.slot_group * per_slot) + 15) / 16 * 16;
  d.lds_x = (int)reg_a;
  const size_t reg_x = ((size_t)H + (size_t)(H / 32) * 4 + 15) / 16 * 16;
  d.lds_l = d.logits_out ? (int)(reg_a + reg_x) : -1;
  const size_t shmem = reg_a + reg_x + (d.logits_out ? (size_t)E * 4 : 0);
  // as many workgroups as the GPU holds at once
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
  const int cap = std::max(per_cu * n_cu, kQueues);
  d.total = d.n_gr + d.n_down;
  // every queue that holds an item has a workgroup (grid >= min(total, 8))
  const int grid = std::min(d.total, cap);
  // the shared expert's gate/up rows, spread evenly over the grid
  d.sh_rows = (I + grid - 1) / grid;
  // logit slices: P parts per gate row, as many as fit the grid and the
  // header's partial words (the columns of a part a whole number of float4)
  if (d.gate_w) {
    int P = 1;
    while (P * 2 <= kMaxPartsPerRow && E * P * 2 <= std::min(grid, kMaxSlices) && (H / (P * 2)) % 4 == 0)
      P *= 2;
    if (E * P > kMaxSlices) return hipErrorNotSupported;
    d.n_part = P;
    d.n_slice = E * P;
  } else {
    d.n_part = 1;
    d.n_slice = 0;
  }
  if (d.grid_out) *d.grid_out = grid;
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

template <int BITS, int GLPR, int GCPL, int DLPR, int DCPL, int T>
static hipError_t launch_small_t(DecodeArgs d, hipStream_t st, KEvents ev) {
  constexpr int DNPASS = small_dpass(DCPL);
  const int I = d.f.L.I, H = d.f.L.H, E = d.f.E, k = d.f.k;
  d.down_rows = kDecWaves * DNPASS * (64 / DLPR);
  if (H % d.down_rows || I % kGuRows || T * k > kSelMaxK || (d.gate_w && T * E > kMaxSlices) ||
      (H / 4 + kDecWaves - 1) / kDecWaves > 64 * SliceGate::kMaxPer || H > 8192)
    return hipErrorNotSupported;
  d.n_down = H / d.down_rows;
  // dynamic LDS: [max(selection scratch, staged h of DSG experts' rows) |
  // the tokens' codes and scales | one token's logits kept for the caller]
  const size_t per_row = (size_t)I + (size_t)(I / 32) * 4;
  const size_t sel =
      (sizeof(SelInput) + std::max(sizeof(SelWgScratch), sizeof(SelFastScratch)) + 15) / 16 * 16;
  const size_t reg_a = (std::max(sel, (size_t)small_drows(DCPL, T) * per_row) + 15) / 16 * 16;
  d.lds_x = (int)reg_a;
  const size_t reg_x = ((size_t)T * H + (size_t)T * (H / 32) * 4 + 15) / 16 * 16;
  d.lds_l = d.logits_out ? (int)(reg_a + reg_x) : -1;
  const size_t shmem = reg_a + reg_x + (d.logits_out ? (size_t)E * 4 : 0);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(&k_small_fused<BITS, GLPR, GCPL, DLPR, DCPL, T>),
          kDecThreads, shmem) != hipSuccess ||
      per_cu <= 0)
    return hipErrorNotSupported;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  const int cap = std::max(per_cu * n_cu, kQueues);
  d.total = (T * k + 1) * (I / kGuRows) + d.n_down;  // items at most (every pair its own expert)
  const int grid = std::min(d.total, cap);
  d.n_part = 1;
  d.n_slice = d.gate_w ? E : 0;
  if (d.grid_out) *d.grid_out = grid;
  COLI_LAUNCH(ev, (k_small_fused<BITS, GLPR, GCPL, DLPR, DCPL, T>), dim3(grid), dim3(kDecThreads),
              shmem, st, d);
  return hipGetLastError();
}

template <int BITS, int GL, int GC, int DL, int DC>
static hipError_t launch_small_shape(DecodeArgs d, int T, hipStream_t st, KEvents ev) {
  switch (T) {
    case 2: return launch_small_t<BITS, GL, GC, DL, DC, 2>(d, st, ev);
    case 3: return launch_small_t<BITS, GL, GC, DL, DC, 3>(d, st, ev);
    case 4: return launch_small_t<BITS, GL, GC, DL, DC, 4>(d, st, ev);
    default: return hipErrorNotSupported;
  }
}

// The single-kernel small batch is built for the decode kernel's row shapes.
template <int BITS>
static hipError_t launch_small_bits(DecodeArgs d, int T, hipStream_t st, KEvents ev) {
  const int gn = d.f.L.H * BITS / 128, dn = d.f.L.I * BITS / 128;
  const int gl = dec_lpr(gn), gc = dec_cpl(gn, gl), dl = dec_lpr(dn), dc = dec_cpl(dn, dl);
#define COLI_SMALL_CASE(GL, GC, DL, DC) \
  if (gl == GL && gc == GC && dl == DL && dc == DC) return launch_small_shape<BITS, GL, GC, DL, DC>(d, T, st, ev);
  COLI_SMALL_CASE(64, 1, 64, 1)
  if constexpr (BITS == 8) { COLI_SMALL_CASE(64, 6, 64, 2) }
  if constexpr (BITS == 4) { COLI_SMALL_CASE(64, 3, 64, 1) }
  if constexpr (BITS == 2) { COLI_SMALL_CASE(32, 3, 32, 1) }
#undef COLI_SMALL_CASE
  return hipErrorNotSupported;
}

hipError_t launch_small_fused(const FfnArgs &f, const float *x, const float *gate_w,
                              const float *logits_in, float *logits_out, uint32_t *ctr, float *hsh,
                              hipStream_t st, KEvents ev, int *grid_out) {
  if (f.T < 2 || f.T > kSmallMaxT) return hipErrorNotSupported;
  DecodeArgs d{};
  d.grid_out = grid_out;
  d.f = f;
  d.x = x;
  d.gate_w = gate_w;
  d.logits_in = gate_w ? nullptr : logits_in;
  d.logits_out = gate_w ? logits_out : nullptr;
  d.ctr = ctr;
  d.hsh = hsh;
  switch (f.L.bits) {
    case 8: return launch_small_bits<8>(d, f.T, st, ev);
    case 4: return launch_small_bits<4>(d, f.T, st, ev);
    case 2: return launch_small_bits<2>(d, f.T, st, ev);
    default: return hipErrorInvalidValue;
  }
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
                               float *hsh, hipStream_t st, KEvents ev, uint64_t *trace,
                               int trace_wgs, int *grid_out) {
  DecodeArgs d{};
  d.trace = trace;
  d.trace_wgs = trace_wgs;
  d.grid_out = grid_out;
  d.f = f;
  d.x = x;
  d.gate_w = gate_w;
  d.logits_in = gate_w ? nullptr : logits_in;
  d.logits_out = gate_w ? logits_out : nullptr;
  d.ctr = ctr;
  d.hsh = hsh;
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
