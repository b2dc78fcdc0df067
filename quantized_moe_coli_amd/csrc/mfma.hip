// mfma.hip -- the batch-union expert FFNs on the gfx950 int8 matrix cores,
// for the experts of a batch that receive many tokens (prefill, long
// verify batches).
//
// colibrì README, "Implemented features": int8 / packed int4 / packed int2
// expert weights with one scale per row, dequantised on use against
// Q8_0-style int8 activations, and a batch-union MoE in which each unique
// expert is read once for all of its tokens.  With many tokens per expert
// the dot-product GEMV (ffn.hip) turns ALU-bound; here the products run on
// v_mfma_i32_16x16x32_i8, whose K = 32 is exactly one Q8_0 block, so every
// MFMA result is one block's exact int32 sum, scaled in fp32 by the token's
// block scale before it is accumulated.
//
// Operands (16 x 16 x 32): lane l holds 8 int8 values of row l % 16 of A
// and of column l % 16 of B, at k = 8 (l / 16) .. 8 (l / 16) + 7; the
// result row 4 (l / 16) + r, column l % 16 is in element r.  A is 16
// weight rows, B is 16 tokens.  The packed weights are widened to int8 by
// masking each code into the high bits of a byte (codes x16 for int4, x64
// for int2), which yields the k order the activations are already stored in
// (the container ordering of coli_quant_act_q8_0's forward copy); the int32
// results are shifted back exactly.
//
// Work items: a (union slot, token group of 64, 64-row block) each; the
// item table (prefix of token groups over the slots that run here) is built
// on the device after the dispatch tables, so the grid is a host-side upper
// bound and surplus workgroups exit at once.
#include <type_traits>

#include "ffn_common.hpp"
#include "kernels.hpp"

namespace coli {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 64;  // weight rows per workgroup (16 per wave)
constexpr int kMfmaTiles = kMfmaTokens / 16;

// Tokens a union slot sends to the matrix cores (0: the dot-product path
// takes it).
__device__ __forceinline__ int mfma_groups(int n_tok, int mfma_min) {
  return n_tok >= mfma_min ? (n_tok + kMfmaTokens - 1) / kMfmaTokens : 0;
}

// mgofs[u] = first token group of union slot u (slots 0 .. n_uniq-1 are the
// unique routed experts, slot n_uniq the shared expert); mgofs[n_uniq + 1]
// is the total.  One workgroup; slots <= 1025.
__global__ __launch_bounds__(1024) void k_mfma_items(FfnArgs a, int32_t *__restrict__ mgofs) {
  __shared__ int sc[2][1024];
  const int tid = threadIdx.x;
  const int nu = *a.disp.n_uniq;
  const int slots = nu + 1;
  // thread i sums slots 2i, 2i+1
  int g0 = 0, g1 = 0;
  if (2 * tid < slots) {
    const int u = 2 * tid;
    g0 = u < nu ? mfma_groups(a.disp.counts[a.disp.uniq[u]], a.mfma_min)
               : mfma_groups(a.T, a.mfma_min_shared);
  }
  if (2 * tid + 1 < slots) {
    const int u = 2 * tid + 1;
    g1 = u < nu ? mfma_groups(a.disp.counts[a.disp.uniq[u]], a.mfma_min)
               : mfma_groups(a.T, a.mfma_min_shared);
  }
  int cur = 0;
  sc[0][tid] = g0 + g1;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = sc[cur][tid] + (tid >= d ? sc[cur][tid - d] : 0);
    sc[cur ^ 1][tid] = v;
    cur ^= 1;
    __syncthreads();
  }
  const int incl = sc[cur][tid];  // inclusive prefix of the pair sums
  const int excl = incl - (g0 + g1);
  if (2 * tid < slots) mgofs[2 * tid] = excl;
  if (2 * tid + 1 < slots) mgofs[2 * tid + 1] = excl + g0;
  if (tid == 1023) mgofs[slots] = incl;  // total (slots <= 2048)
}

// A operand, in two steps so a block's raw loads can all be issued before
// any is used: wraw loads the packed bytes of k-group g of block b of a
// weight row; wop widens them to int8 (x16 for int4, x64 for int2).
template <int BITS>
using WRaw = typename std::conditional<BITS == 8, uint64_t, uint32_t>::type;

template <int BITS>
__device__ __forceinline__ WRaw<BITS> wraw(const uint8_t *row, int b, int g) {
  if constexpr (BITS == 8) return *reinterpret_cast<const uint64_t *>(row + 32 * b + 8 * g);
  else if constexpr (BITS == 4) return *reinterpret_cast<const uint32_t *>(row + 16 * b + 4 * g);
  else return *reinterpret_cast<const uint32_t *>(row + 8 * b + 4 * (g >> 1));
}

template <int BITS>
__device__ __forceinline__ long wop(WRaw<BITS> w, int g) {
  if constexpr (BITS == 8) {
    return (long)w;
  } else if constexpr (BITS == 4) {
    const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
    return (long)(((uint64_t)hi << 32) | lo);
  } else {
    uint32_t p0, p1;
    if (g & 1) {
      p0 = (w << 2) & 0xC0C0C0C0u;
      p1 = w & 0xC0C0C0C0u;
    } else {
      p0 = (w << 6) & 0xC0C0C0C0u;
      p1 = (w << 4) & 0xC0C0C0C0u;
    }
    return (long)(((uint64_t)p1 << 32) | p0);
  }
}

template <int BITS>
__device__ __forceinline__ long wop(const uint8_t *row, int b, int g) {
  return wop<BITS>(wraw<BITS>(row, b, g), g);
}

template <int BITS>
constexpr int wshift() {
  return BITS == 8 ? 0 : BITS == 4 ? 4 : 6;
}

// The work item of this workgroup: union slot, token group, and row block.
struct MfmaItem {
  int e;      // expert (-1: shared)
  TokList s;  // the slot's tokens
  int n0, nt; // first token of the group, tokens in it
  int rb;     // row block
};

__device__ __forceinline__ bool mfma_item(const FfnArgs &a, int n_rb, MfmaItem &it) {
  const int G = blockIdx.x / n_rb;
  it.rb = blockIdx.x % n_rb;
  const int nu = *a.disp.n_uniq;
  const int32_t *gofs = a.disp.mgofs;
  if (G >= gofs[nu + 1]) return false;
  int lo = 0, hi = nu;  // last slot whose first group is <= G
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gofs[mid] <= G) lo = mid;
    else hi = mid - 1;
  }
  const bool shared = lo == nu;
  it.e = shared ? -1 : a.disp.uniq[lo];
  it.s.slot = -1;
  it.s.shared = shared;
  it.s.n_tok = shared ? a.T : a.disp.counts[it.e];
  it.s.p0 = shared ? -1 : a.disp.offs[it.e];
  it.n0 = (G - gofs[lo]) * kMfmaTokens;
  it.nt = min(kMfmaTokens, it.s.n_tok - it.n0);
  return it.nt > 0;
}

// ---------------------------------------------------------------------------
// The block-scaled int8 GEMM core shared by both kernels.  A workgroup of 4
// waves multiplies NMAT weight matrices (16 rows per wave each) by up to 64
// token rows of Q8_0 codes, over K in chunks of CH blocks of 32.  Each chunk
// is loaded with 16-byte coalesced loads into registers one chunk ahead,
// stored to LDS, then read back in the MFMA operand layout (a 16-byte load
// per lane of a weight row holds whole blocks, while an operand holds a
// quarter block of each of 16 rows, so the reshuffle goes through LDS).
// acc[m][tt][r]: matrix m, token tile tt, row 4 g + r of the wave, token
// 16 tt + li (lane = 16 g + li).
// ---------------------------------------------------------------------------
template <int BITS>
struct MfmaGeo {
  static constexpr int CH = BITS == 8 ? 8 : 16;           // blocks per chunk
  static constexpr int RBC = CH * 32 * BITS / 8;          // weight bytes per row per chunk
  static constexpr int WST = RBC + 16;                    // LDS stride of a weight row
  static constexpr int XST = CH * 32 + 16;                // LDS stride of a token row
  static constexpr int XPT = kMfmaTokens * CH * 2 / 256;  // 16-byte code loads per thread
  static constexpr int DPT = kMfmaTokens * CH / 256;      // scales per thread
};

template <int BITS, int NMAT>
struct MfmaLds {
  using G = MfmaGeo<BITS>;
  int8_t xs[kMfmaTokens * G::XST];    // token codes of the chunk
  float ds[kMfmaTokens][G::CH + 1];   // their block scales
  uint8_t ws[4][NMAT * 16 * G::WST];  // each wave's weight rows of the chunk
  int trow[kMfmaTokens];              // activation row of each token
};

template <int BITS, int NMAT, typename Acc>
__device__ __forceinline__ void mfma_core(const uint8_t *const *wbase, size_t row_bytes,
                                          const int8_t *act, const float *actd, int K, int nt,
                                          MfmaLds<BITS, NMAT> &L, Acc (*acc)[kMfmaTiles][4]) {
  using G = MfmaGeo<BITS>;
  constexpr int SH = wshift<BITS>();
  constexpr int PPR = G::RBC / 16;             // 16-byte pieces per weight row
  constexpr int WPL = NMAT * 16 * PPR / 64;    // 16-byte weight loads per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int nbk = K / 32, nch = (nbk + G::CH - 1) / G::CH;
  const int ntt = (nt + 15) >> 4;
  const v4i zero = {0, 0, 0, 0};
  uint4 xr[G::XPT], wr[WPL];
  float dr[G::DPT];

  auto load_chunk = [&](int c) {
    const int b0 = c * G::CH, cb = min(G::CH, nbk - b0);
#pragma unroll
    for (int i = 0; i < G::XPT; ++i) {
      const int p = threadIdx.x + 256 * i, tok = p / (2 * G::CH), pc = p % (2 * G::CH);
      xr[i] = make_uint4(0, 0, 0, 0);
      if (tok < nt && pc < 2 * cb)
        xr[i] = *reinterpret_cast<const uint4 *>(act + (size_t)L.trow[tok] * K + b0 * 32 + 16 * pc);
    }
#pragma unroll
    for (int i = 0; i < G::DPT; ++i) {
      const int p = threadIdx.x + 256 * i, tok = p / G::CH, bb = p % G::CH;
      dr[i] = 0.f;
      if (tok < nt && bb < cb) dr[i] = actd[(size_t)L.trow[tok] * nbk + b0 + bb];
    }
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const int p = lane + 64 * i, r = p / PPR, pc = p % PPR;
      wr[i] = make_uint4(0, 0, 0, 0);
      if (pc * 16 < cb * 32 * BITS / 8)
        wr[i] = ld_nt(reinterpret_cast<const uint4 *>(wbase[r / 16] + (size_t)(r % 16) * row_bytes +
                                                      (size_t)b0 * 32 * BITS / 8) + pc);
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < G::XPT; ++i) {
      const int p = threadIdx.x + 256 * i, tok = p / (2 * G::CH), pc = p % (2 * G::CH);
      *reinterpret_cast<uint4 *>(L.xs + tok * G::XST + 16 * pc) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < G::DPT; ++i) {
      const int p = threadIdx.x + 256 * i;
      L.ds[p / G::CH][p % G::CH] = dr[i];
    }
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const int p = lane + 64 * i, r = p / PPR, pc = p % PPR;
      *reinterpret_cast<uint4 *>(L.ws[wave] + r * G::WST + 16 * pc) = wr[i];
    }
  };

  load_chunk(0);
  for (int c = 0; c < nch; ++c) {
    __syncthreads();  // the previous chunk's operands are no longer read
    store_chunk();
    if (c + 1 < nch) load_chunk(c + 1);
    __syncthreads();
    const int cb = min(G::CH, nbk - c * G::CH);
#pragma unroll 4
    for (int b = 0; b < cb; ++b) {
      long aw[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const uint8_t *wrow = L.ws[wave] + (m * 16 + li) * G::WST;
        if constexpr (BITS == 8) aw[m] = *reinterpret_cast<const long *>(wrow + 32 * b + 8 * g);
        else if constexpr (BITS == 4)
          aw[m] = wop<4>(*reinterpret_cast<const uint32_t *>(wrow + 16 * b + 4 * g), g);
        else aw[m] = wop<2>(*reinterpret_cast<const uint32_t *>(wrow + 8 * b + 4 * (g >> 1)), g);
      }
#pragma unroll
      for (int tt = 0; tt < kMfmaTiles; ++tt) {
        if (tt < ntt) {
          const long bx = *reinterpret_cast<const long *>(L.xs + (16 * tt + li) * G::XST + 32 * b + 8 * g);
          const Acc dj = (Acc)L.ds[16 * tt + li][b];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            const v4i cm = __builtin_amdgcn_mfma_i32_16x16x32_i8(aw[m], bx, zero, 0, 0, 0);
            // the block's exact int32 sum times the token's block scale
            // (exact in binary64; one rounding per step in binary32)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][tt][r] += (Acc)(cm[r] >> SH) * dj;
          }
        }
      }
    }
  }
  __syncthreads();  // LDS free for the caller
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + Q8_0(h): rows [64 rb, +64) of gate and up for up to 64
// tokens of one expert.  Wave w owns rows 16 w .. 16 w + 15 of both.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void k_gateup_mfma(FfnArgs a) {
  __shared__ __align__(16) MfmaLds<BITS, 2> L;
  const int H = a.L.H, I = a.L.I;
  MfmaItem it;
  if (!mfma_item(a, I / kMfmaRows, it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const ExpertPtrs ep = expert_ptrs(a.L, it.e);
  const size_t row_bytes = (size_t)H * BITS / 8;
  const int row0 = it.rb * kMfmaRows + wave * 16;
  for (int n = threadIdx.x; n < kMfmaTokens; n += 256) {
    int t = 0, hrow, j;
    if (n < it.nt) tok_at(a, true, it.s, it.n0 + n, t, hrow, j);
    L.trow[n] = t;
  }
  __syncthreads();
  const uint8_t *wb[2] = {ep.wg + (size_t)row0 * row_bytes, ep.wu + (size_t)row0 * row_bytes};
  // g and u accumulate in binary64 (the expert definition's sum, rounded
  // once), so h -- and its Q8_0 codes -- are those of that definition
  double acc[2][kMfmaTiles][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int tt = 0; tt < kMfmaTiles; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][tt][r] = 0.0;
  mfma_core<BITS, 2>(wb, row_bytes, a.xq, a.xd, H, it.nt, L, acc);

  // h = silu(g) * u for rows 4 g + r of the wave, token 16 tt + li, staged
  // in LDS (over the operand tiles) for the Q8_0 step
  static_assert(sizeof(float) * kMfmaTokens * (kMfmaRows + 1) <= sizeof(L.xs) + sizeof(L.ds),
                "h tile exceeds the operand tiles");
  float(*hs)[kMfmaRows + 1] = reinterpret_cast<float(*)[kMfmaRows + 1]>(L.xs);
  const int ntt = (it.nt + 15) >> 4;
  float sg[4], su[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sg[r] = ep.sg[row0 + 4 * g + r];
    su[r] = ep.su[row0 + 4 * g + r];
  }
#pragma unroll
  for (int tt = 0; tt < kMfmaTiles; ++tt)
    if (tt < ntt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hs[16 * tt + li][wave * 16 + 4 * g + r] =
            swiglu_h(row_out(acc[0][tt][r], sg[r]), row_out(acc[1][tt][r], su[r]));
  __syncthreads();
  // Q8_0 of each token's two 32-row blocks of h: 32 threads per block
  for (int q = threadIdx.x; q < it.nt * kMfmaRows; q += 256) {
    const int tl = q / kMfmaRows, bb = (q / 32) & 1, i = q & 31;
    const float h = hs[tl][bb * 32 + i];
    float amax = group_max<32>(fabsf(h));
    amax = __shfl(amax, (lane & 32) | 31, 64);
    int t, hrow, j;
    tok_at(a, true, it.s, it.n0 + tl, t, hrow, j);
    const float db = amax / 127.f;
    float c = 0.f;
    if (db != 0.f) c = fminf(fmaxf(rintf(h / db), -127.f), 127.f);
    const int blk = it.rb * (kMfmaRows / 32) + bb;
    a.hq[(size_t)hrow * I + blk * 32 + perm_dst<BITS>(i)] = (int8_t)c;
    if (i == 0) a.hd[(size_t)hrow * (I / 32) + blk] = db;
  }
}

// ---------------------------------------------------------------------------
// Down projection: output rows [64 rb, +64) for up to 64 tokens of one
// expert, o into the per-(token, slot) buffer the combine kernel reduces.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void k_down_mfma(FfnArgs a) {
  __shared__ __align__(16) MfmaLds<BITS, 1> L;
  const int H = a.L.H, I = a.L.I;
  MfmaItem it;
  if (!mfma_item(a, H / kMfmaRows, it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const ExpertPtrs ep = expert_ptrs(a.L, it.e);
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int row0 = it.rb * kMfmaRows + wave * 16;
  for (int n = threadIdx.x; n < kMfmaTokens; n += 256) {
    int t = 0, hrow = 0, j;
    if (n < it.nt) tok_at(a, true, it.s, it.n0 + n, t, hrow, j);
    L.trow[n] = hrow;
  }
  __syncthreads();
  const uint8_t *wb[1] = {ep.wd + (size_t)row0 * row_bytes};
  float acc[1][kMfmaTiles][4];
#pragma unroll
  for (int tt = 0; tt < kMfmaTiles; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[0][tt][r] = 0.f;
  mfma_core<BITS, 1>(wb, row_bytes, a.hq, a.hd, I, it.nt, L, acc);

  const int ntt = (it.nt + 15) >> 4;
  float sd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sd[r] = ep.sd[row0 + 4 * g + r];
#pragma unroll
  for (int tt = 0; tt < kMfmaTiles; ++tt) {
    const int n = 16 * tt + li;
    if (tt < ntt && n < it.nt) {
      int t, hrow, j;
      tok_at(a, true, it.s, it.n0 + n, t, hrow, j);
      float4 o;
      o.x = acc[0][tt][0] * sd[0];
      o.y = acc[0][tt][1] * sd[1];
      o.z = acc[0][tt][2] * sd[2];
      o.w = acc[0][tt][3] * sd[3];
      *reinterpret_cast<float4 *>(a.obuf + ((size_t)t * (a.k + 1) + j) * H + row0 + 4 * g) = o;
    }
  }
}

// Upper bound of the token groups a batch can send here: routed pairs in
// groups of 64 plus one partial group per unique expert that can reach
// mfma_min tokens (at most pairs / mfma_min of them), plus the shared
// expert's groups when the batch reaches its threshold.
static int mfma_group_bound(const FfnArgs &a) {
  const long pairs = (long)a.T * a.k;
  long cap = pairs < a.E ? pairs : a.E;
  if (pairs / a.mfma_min < cap) cap = pairs / a.mfma_min;
  const long shared = a.T >= a.mfma_min_shared ? (a.T + kMfmaTokens - 1) / kMfmaTokens : 0;
  return (int)((pairs + kMfmaTokens - 1) / kMfmaTokens + cap + shared);
}

hipError_t launch_mfma_items(const FfnArgs &a, int32_t *mgofs, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_items, dim3(1), dim3(1024), 0, st, a, mgofs);
  return hipGetLastError();
}

hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t st, KEvents ev) {
  const dim3 grid((unsigned)(mfma_group_bound(a) * (a.L.I / kMfmaRows))), block(256);
  switch (a.L.bits) {
    case 8: COLI_LAUNCH(ev, k_gateup_mfma<8>, grid, block, 0, st, a); break;
    case 4: COLI_LAUNCH(ev, k_gateup_mfma<4>, grid, block, 0, st, a); break;
    case 2: COLI_LAUNCH(ev, k_gateup_mfma<2>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t st, KEvents ev) {
  const dim3 grid((unsigned)(mfma_group_bound(a) * (a.L.H / kMfmaRows))), block(256);
  switch (a.L.bits) {
    case 8: COLI_LAUNCH(ev, k_down_mfma<8>, grid, block, 0, st, a); break;
    case 4: COLI_LAUNCH(ev, k_down_mfma<4>, grid, block, 0, st, a); break;
    case 2: COLI_LAUNCH(ev, k_down_mfma<2>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
