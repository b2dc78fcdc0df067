// ffn.hip -- the expert FFNs of the routed-MoE layer on the integer
// dot-product path (gfx950 v_dot4_i32_i8), decode and batch-union modes.
//
// colibrì README, "Implemented features": expert weights are int8 / packed
// int4 / packed int2 with one scale per row, dequantised on use against
// Q8_0-style int8 activations; the MoE is DeepSeek-V3-like (SwiGLU experts
// plus a shared expert); in a batch each unique expert is read once and
// applied to every position routed to it.
//
// Work split.  A "chunk" is 16 bytes of packed weights (device.hpp).  LPR
// lanes share a weight row, lane c of the group loading chunks c, c+LPR, ...
// (CPL chunks at most), so every wave-wide load is a run of contiguous
// 16-byte pieces; the fp32 partial sums of a row are reduced across its LPR
// lanes with DPP.  Each block partial is scaled by its Q8_0 scale d in fp32
// and the row sum by the row scale s.
//
// Gate/up: a workgroup owns 32 consecutive intermediate rows of one expert
// (exactly one Q8_0 block of h), computes g and u for every token of the
// expert, h = silu(g) * u, and quantises the 32 values of h per token to
// one Q8_0 block -- so the down projection's input never leaves int8.
//
// Down: decode mode spreads the k+1 slots of the token over the waves of a
// workgroup and combines w_j * o_j in a fixed slot order through LDS; union
// mode runs one expert over its tokens and writes o into a per-(token, slot)
// buffer that a combine kernel reduces in the same fixed order.  No
// floating-point atomics: results are bit-reproducible.
#include <algorithm>

#include "ffn_common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace coli {

// Decode (T == 1): grid.x = (k+1) * (I/32).  Slot u < k is the u-th routed
// expert of the token, which every routed workgroup selects itself from the
// logits (one wave, select.hpp) -- no separate routing launch; workgroup
// (0, 0) also stores the routing for the down kernel and the caller.  Slot k
// is the shared expert, which needs no routing and starts at once.
template <int BITS, int LPR, int CPL>
__global__ __launch_bounds__(256) void k_gateup_decode(FfnArgs a) {
  __shared__ float hs[1][32];
  __shared__ SelScratch sc;
  __shared__ int32_t sidx[kSelMaxK];
  __shared__ float sw[kSelMaxK];
  const int n_rb = a.L.I / 32;
  const int u = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
  int e = -1;
  if (u < a.k) {
    if (threadIdx.x < 64) select_token(a.cfg, a.logits, a.bias, sc, sidx, sw);
    __syncthreads();
    if (u == 0 && rb == 0 && (int)threadIdx.x < a.k) {
      const int j = threadIdx.x;
      a.idx[j] = sidx[j];
      a.w[j] = sw[j];
      if (a.idx_user) a.idx_user[j] = sidx[j];
      if (a.w_user) a.w_user[j] = sw[j];
    }
    e = sidx[u];
    if (e < 0) return;  // dropped by expert top-p
  }
  TokList s;
  s.n_tok = 1;
  s.p0 = -1;
  s.slot = u;
  s.shared = (u == a.k);
  gateup_body<BITS, LPR, CPL, 1>(a, false, expert_ptrs(a.L, e), s, rb, hs, a.xq, a.xd);
}

// Union (T >= 2): items (union slot u, 32-row block rb) for u up to the
// largest possible slot count, grid-strided (slots the matrix-core kernels
// take, or past the last unique expert, are skipped).
template <int BITS, int LPR, int CPL, int NT>
__global__ __launch_bounds__(256) void k_gateup_union(FfnArgs a, int n_items) {
  __shared__ float hs[NT][32];
  const int n_rb = a.L.I / 32;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = item / n_rb, rb = item % n_rb;
    int e;
    TokList s;
    if (!union_item(a, u, e, s)) continue;
    gateup_body<BITS, LPR, CPL, NT>(a, true, expert_ptrs(a.L, e), s, rb, hs, a.xq, a.xd);
  }
}

// ---------------------------------------------------------------------------
// Down, decode mode (T == 1).  grid.x = H / ROWS; block = 64 * NW waves with
// NW = min(k+1, 12).  Wave w handles slots w, w+NW, ... of [routed 0..k-1,
// shared k]: ROWS rows of w_j * o_j (o for the shared slot) into LDS, all
// ROWS row loads in flight at once; then the rows are summed in the order
// shared, 0, 1, ..., k-1.
// ---------------------------------------------------------------------------
template <int BITS, int LPR, int CPL>
__global__ __launch_bounds__(768) void k_down_decode(FfnArgs a) {
  constexpr int RPP = 64 / LPR;
  constexpr int PASSES = CPL == 1 ? 16 : CPL == 2 ? 8 : CPL <= 4 ? 4 : 2;  // ~16 loads in flight
  constexpr int ROWS = PASSES * RPP;
  constexpr int kMaxSlots = kSelMaxK + 1;
  __shared__ float part[kMaxSlots][ROWS];
  const int I = a.L.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int gl = lane % LPR, rsub = lane / LPR;
  const int nchunks = I * BITS / 128;
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int r0 = blockIdx.x * ROWS;
  const int nslots = a.k + 1;

  for (int sl = wave; sl < nslots; sl += nw) {
    const bool shared = (sl == a.k);
    const int e = shared ? -1 : a.idx[sl];
    if (!shared && e < 0) {
      for (int r = lane; r < ROWS; r += 64) part[sl][r] = 0.f;
      continue;
    }
    const ExpertPtrs ep = expert_ptrs(a.L, e);
    const float wgt = shared ? 1.f : a.w[sl];
    uint4 wv[PASSES][CPL];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPP + rsub;
      const uint4 *wp = reinterpret_cast<const uint4 *>(ep.wd + (size_t)row * row_bytes);
#pragma unroll
      for (int i = 0; i < CPL; ++i) wv[p][i] = ld_nt(wp + min(gl + LPR * i, nchunks - 1));
    }
    const float sdv = ep.sd[r0 + min(lane, ROWS - 1)];  // lane i: scale of row r0 + i
    Act<BITS> act[CPL];
    const int8_t *hq = a.hq + (size_t)sl * I;
    const float *hd = a.hd + (size_t)sl * (I / 32);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = gl + LPR * i;
      if (c < nchunks) load_act<BITS>(act[i], hq, hd, c);
      else zero_act<BITS>(act[i]);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc += chunk_part<BITS>(wv[p][i], act[i]);
      acc = group_sum<LPR>(acc);
      const int rl = p * RPP + rsub;
      const float sd = row_scale<RPP>(sdv, p, rsub);
      if (lane == group_sum_lane<LPR>(lane)) {
        const float o = acc * sd;
        part[sl][rl] = shared ? o : wgt * o;
      }
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < ROWS; r += blockDim.x) {
    float y = part[a.k][r];
    for (int j = 0; j < a.k; ++j) y += part[j][r];
    a.y[r0 + r] = y;
  }
}

// ---------------------------------------------------------------------------
// Down, union mode.  Items (slot, block of 4*ROWS rows), grid-strided; each
// wave owns ROWS rows of one expert and runs every token of the expert on
// them (NT at a time), writing o to obuf[t][j][row].
// ---------------------------------------------------------------------------
template <int BITS, int LPR, int CPL, int NT, int ROWS>
__device__ __forceinline__ void down_union_item(const FfnArgs &a, int item) {
  constexpr int RPP = 64 / LPR;
  constexpr int PASSES = ROWS / RPP;
  const int H = a.L.H, I = a.L.I;
  const int n_rb = H / (4 * ROWS);
  const int u = item / n_rb, rb = item % n_rb;
  int e;
  TokList s;
  if (!union_item(a, u, e, s)) return;
  const ExpertPtrs ep = expert_ptrs(a.L, e);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % LPR, rsub = lane / LPR;
  const int nchunks = I * BITS / 128;
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int r0 = rb * 4 * ROWS + wave * ROWS;

  uint4 wv[PASSES][CPL];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP + rsub;
    const uint4 *wp = reinterpret_cast<const uint4 *>(ep.wd + (size_t)row * row_bytes);
#pragma unroll
    for (int i = 0; i < CPL; ++i) wv[p][i] = ld_nt(wp + min(gl + LPR * i, nchunks - 1));
  }
  const float sdv = ep.sd[r0 + min(lane, ROWS - 1)];  // lane i: scale of row r0 + i
  for (int t0 = 0; t0 < s.n_tok; t0 += NT) {
    Act<BITS> act[CPL][NT];
    int tok[NT], slot[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      int t = 0, hrow = 0, j = 0;
      const bool tv = t0 + tt < s.n_tok;
      if (tv) tok_at(a, true, s, t0 + tt, t, hrow, j);
      tok[tt] = tv ? t : -1;
      slot[tt] = j;
      const int8_t *hq = a.hq + (size_t)hrow * I;
      const float *hd = a.hd + (size_t)hrow * (I / 32);
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = gl + LPR * i;
        if (tv && c < nchunks) load_act<BITS>(act[i][tt], hq, hd, c);
        else zero_act<BITS>(act[i][tt]);
      }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = r0 + p * RPP + rsub;
      float acc[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        acc[tt] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[tt] += chunk_part<BITS>(wv[p][i], act[i][tt]);
        acc[tt] = group_sum<LPR>(acc[tt]);
      }
      const float sd = row_scale<RPP>(sdv, p, rsub);
      if (lane == group_sum_lane<LPR>(lane)) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
          if (tok[tt] >= 0)
            a.obuf[((size_t)tok[tt] * (a.k + 1) + slot[tt]) * H + row] = acc[tt] * sd;
      }
    }
  }
}

template <int BITS, int LPR, int CPL, int NT, int ROWS>
__global__ __launch_bounds__(256) void k_down_union(FfnArgs a, int n_items) {
  for (int item = blockIdx.x; item < n_items; item += gridDim.x)
    down_union_item<BITS, LPR, CPL, NT, ROWS>(a, item);
}

// y[t][r] = o_shared + sum over kept slots j (in order) of w_tj * o_tj.
// The rows of 8 slots at a time are requested before any is added (every
// slot's row exists in obuf; a dropped slot's is read and not used).
__global__ __launch_bounds__(256) void k_combine(FfnArgs a) {
  constexpr int kGroup = 8;
  const int H = a.L.H, k = a.k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  if (i >= (int64_t)a.T * (H / 4)) return;
  const int t = (int)(i / (H / 4)), r4 = (int)(i % (H / 4));
  const float4 *ob = reinterpret_cast<const float4 *>(a.obuf + (size_t)t * (k + 1) * H);
  const int32_t *ti = a.idx + (size_t)t * k;
  const float *tw = a.w + (size_t)t * k;
  float4 y = ob[(size_t)k * (H / 4) + r4];
  for (int j0 = 0; j0 < k; j0 += kGroup) {
    float4 o[kGroup];
    int id[kGroup];
    float wj[kGroup];
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      const int j = j0 + jj;
      if (j < k) {
        id[jj] = ti[j];
        wj[jj] = tw[j];
        o[jj] = ob[(size_t)j * (H / 4) + r4];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kGroup; ++jj) {
      if (j0 + jj >= k || id[jj] < 0) continue;
      const float w = wj[jj];
      y.x += w * o[jj].x;
      y.y += w * o[jj].y;
      y.z += w * o[jj].z;
      y.w += w * o[jj].w;
    }
  }
  reinterpret_cast<float4 *>(a.y + (size_t)t * H)[r4] = y;
}

// ---------------------------------------------------------------------------
// Launch helpers.  LPR is 32 when a row has an odd multiple of 32 chunks,
// else 64; CPL is the chunk count per lane rounded up to 1, 2, 4 or 8.
// ---------------------------------------------------------------------------
static int pick_lpr(int nchunks) { return (nchunks % 64 != 0 && nchunks % 32 == 0) ? 32 : 64; }

static int pick_cpl(int nchunks, int lpr) {
  const int c = (nchunks + lpr - 1) / lpr;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 3 ? 3 : c <= 4 ? 4 : c <= 6 ? 6 : c <= 8 ? 8 : -1;
}

#define COLI_CPL_SWITCH(CPLV, ...)                        \
  switch (CPLV) {                                         \
    case 1: { constexpr int CPL = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int CPL = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int CPL = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int CPL = 4; __VA_ARGS__; } break; \
    case 6: { constexpr int CPL = 6; __VA_ARGS__; } break; \
    case 8: { constexpr int CPL = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                 \
  }

#define COLI_LPR_SWITCH(LPRV, ...)                          \
  if ((LPRV) == 32) { constexpr int LPR = 32; __VA_ARGS__; } \
  else { constexpr int LPR = 64; __VA_ARGS__; }

#define COLI_BITS_SWITCH(BV, ...)                          \
  switch (BV) {                                            \
    case 8: { constexpr int BITS = 8; __VA_ARGS__; } break; \
    case 4: { constexpr int BITS = 4; __VA_ARGS__; } break; \
    case 2: { constexpr int BITS = 2; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                  \
  }

// Tokens per register batch of the union kernels: every lane keeps the
// activations of NT tokens for its CPL chunks in registers, so NT shrinks as
// a chunk's activation (Act<BITS>) grows, keeping that set within ~100
// registers (the kernels then need no spill registers).
template <int BITS, int CPL>
constexpr int union_nt() {
  constexpr int regs = CPL * (Act<BITS>::kInts + Act<BITS>::kD);
  return regs * 4 <= 100 ? 4 : regs * 2 <= 100 ? 2 : 1;
}

// Workgroups of a union GEMV launch (8 per CU); more items are strided.
constexpr int kUnionGrid = 2048;

static int union_slots(const FfnArgs &a) {
  const long routed = (long)a.T * a.k;
  return (int)((routed < a.E ? routed : a.E) + 1);
}

hipError_t launch_gateup(const FfnArgs &a, bool union_mode, int /*mfma_min*/, hipStream_t st,
                         KEvents ev) {
  const int nch = a.L.H * a.L.bits / 128;
  const int lpr = pick_lpr(nch), cpl = pick_cpl(nch, lpr);
  const int slots = union_mode ? union_slots(a) : a.k + 1;
  const int n_items = slots * (a.L.I / 32);
  const dim3 grid((unsigned)(union_mode ? std::min(n_items, kUnionGrid) : n_items)), block(256);
  COLI_BITS_SWITCH(a.L.bits, COLI_LPR_SWITCH(lpr, COLI_CPL_SWITCH(cpl, {
    if (union_mode)
      COLI_LAUNCH(ev, (k_gateup_union<BITS, LPR, CPL, union_nt<BITS, CPL>()>), grid, block, 0, st, a,
                  n_items);
    else
      COLI_LAUNCH(ev, (k_gateup_decode<BITS, LPR, CPL>), grid, block, 0, st, a);
  })));
  return hipGetLastError();
}

hipError_t launch_down(const FfnArgs &a, bool union_mode, int /*mfma_min*/, hipStream_t st,
                       KEvents ev) {
  const int nch = a.L.I * a.L.bits / 128;
  const int lpr = pick_lpr(nch), cpl = pick_cpl(nch, lpr);
  if (!union_mode) {
    const int nw = a.k + 1 < 12 ? a.k + 1 : 12;
    const int passes = cpl == 1 ? 16 : cpl == 2 ? 8 : cpl <= 4 ? 4 : 2;
    const int rows = passes * (64 / lpr);
    const dim3 grid((unsigned)(a.L.H / rows)), block(64 * nw);
    COLI_BITS_SWITCH(a.L.bits, COLI_LPR_SWITCH(lpr, COLI_CPL_SWITCH(cpl, {
      COLI_LAUNCH(ev, (k_down_decode<BITS, LPR, CPL>), grid, block, 0, st, a);
    })));
  } else {
    constexpr int ROWS = 8;
    const int slots = union_slots(a);
    const int n_items = slots * (a.L.H / (4 * ROWS));
    const dim3 grid((unsigned)std::min(n_items, kUnionGrid)), block(256);
    COLI_BITS_SWITCH(a.L.bits, COLI_LPR_SWITCH(lpr, COLI_CPL_SWITCH(cpl, {
      COLI_LAUNCH(ev, (k_down_union<BITS, LPR, CPL, union_nt<BITS, CPL>(), ROWS>), grid, block, 0, st, a,
                  n_items);
    })));
  }
  return hipGetLastError();
}

hipError_t launch_combine(const FfnArgs &a, hipStream_t st) {
  const int64_t n = (int64_t)a.T * (a.L.H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Test export: exact int32 block sums through the same chunk products.
// xq is in natural order; the kernel reorders each chunk's codes into the
// container's ordering before the product.  Thread per (t, row, chunk).
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void k_debug_blocks(const uint8_t *__restrict__ Wq, int rows,
                                                      int cols, const int8_t *__restrict__ xq,
                                                      int T, int32_t *__restrict__ acc) {
  const int nch = cols * BITS / 128;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * rows * nch) return;
  const int c = (int)(i % nch);
  const int r = (int)((i / nch) % rows);
  const int t = (int)(i / ((int64_t)nch * rows));
  const uint4 w = reinterpret_cast<const uint4 *>(Wq + (size_t)r * cols * BITS / 8)[c];
  constexpr int E = Q<BITS>::kElems;
  int words[E / 4];
  const int8_t *xs = xq + (size_t)t * cols + (size_t)c * E;
#pragma unroll
  for (int m = 0; m < E / 4; ++m) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) v |= (uint32_t)(uint8_t)xs[perm_src<BITS>(4 * m + b)] << (8 * b);
    words[m] = (int)v;
  }
  const int nb = cols / 32;
  int32_t *out = acc + ((size_t)t * rows + r) * nb;
  if constexpr (BITS == 8) {
    // two chunks per block: the even chunk writes, the odd one adds later --
    // instead each thread owns one half and the block sum is formed by the
    // even-chunk thread reading its partner's codes.
    if ((c & 1) == 0) {
      const uint4 w2 = reinterpret_cast<const uint4 *>(Wq + (size_t)r * cols)[c + 1];
      int words2[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= (uint32_t)(uint8_t)xs[16 + 4 * m + b] << (8 * b);
        words2[m] = (int)v;
      }
      out[c >> 1] = chunk_dot_q8(w, words) + chunk_dot_q8(w2, words2);
    }
  } else if constexpr (BITS == 4) {
    out[c] = chunk_dot_q4(w, words);
  } else {
    int b0, b1;
    chunk_dot_q2(w, words, b0, b1);
    out[2 * c] = b0;
    out[2 * c + 1] = b1;
  }
}

hipError_t launch_debug_blocks(int bits, const uint8_t *Wq, int rows, int cols, const int8_t *xq,
                               int T, int32_t *acc, hipStream_t st) {
  const int64_t n = (int64_t)T * rows * (cols * bits / 128);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (bits) {
    case 8: hipLaunchKernelGGL(k_debug_blocks<8>, grid, block, 0, st, Wq, rows, cols, xq, T, acc); break;
    case 4: hipLaunchKernelGGL(k_debug_blocks<4>, grid, block, 0, st, Wq, rows, cols, xq, T, acc); break;
    case 2: hipLaunchKernelGGL(k_debug_blocks<2>, grid, block, 0, st, Wq, rows, cols, xq, T, acc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
