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
// MFMA result is one block's exact int32 sum, scaled by the token's block
// scale before it is accumulated (binary64 for gate/up, binary32 for down).
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
// Work items: a (union slot, token group of 64, 128-row block) each; the
// item table (prefix of token groups over the slots that run here) is built
// on the device with the dispatch tables (k_dispatch), so the grid is a
// host-side upper bound and surplus workgroups exit at once.
#include <type_traits>

#include "ffn_common.hpp"
#include "kernels.hpp"

namespace coli {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 128;   // weight rows per workgroup (16 per wave)
constexpr int kMfmaThreads = 512;  // threads per workgroup (8 waves)
constexpr int kMfmaWaves = kMfmaThreads / 64;
constexpr int kMaxStages = 8;

// A kernel's geometry by the workgroups it keeps resident per CU (WG).  Two
// halve each one's LDS ring, its tokens per item and its stage rows, and cap
// it at 128 VGPRs, so four waves share a SIMD instead of two: the binary32
// down projection gains from that, the binary64 gate/up does not.
template <int WG>
struct MfmaCfg {
  static constexpr int TOK = kMfmaGroup / WG;             // tokens per work item (group)
  static constexpr int TILES = TOK / 16;                  // 16-token tiles
  static constexpr int ROWB = 128 / WG;                   // weight bytes per row per stage (at most)
  static constexpr int RING = 160 * 1024 / WG - 2048;     // LDS for the stage ring
};

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

// ---------------------------------------------------------------------------
// Work items: (union slot, token group of up to 64 or 32 tokens, block of
// weight rows), numbered G * n_rb + rb over the token groups G of the slots
// that run here (mgofs), one per workgroup; the hardware hands each CU the
// next workgroup as soon as one finishes, which balances items of unequal
// cost.  Workgroup b takes item n_items - 1 - b: the shared expert's groups
// (the last slot, full groups when it runs here) start first instead of
// forming the tail.  Items of one (slot, row block) with several token
// groups are n_rb apart, so their re-reads of the weights run at about the
// same time.
//
// Workgroup b runs on XCD b mod 8, each XCD with its own L2.  In plain order
// an XCD takes the same row blocks of every group (n_rb a multiple of 8):
// each weight row block is fetched once, but every group's activations by
// all eight XCDs.  Runs of 8 groups of 8 different slots (experts with one
// group each, most of a prefill's) are taken transposed instead: XCD x
// runs every row block of one group, so its activations are fetched once
// too, and so are the weights, which no other group uses.
//
// A workgroup finds its item in two dependent loads: the group counts, then
// the group descriptors (expert, first pair, first token, tokens) and the
// run's end slots together, all written by the dispatch kernel.
// ---------------------------------------------------------------------------
struct MfmaItem {
  int e;      // expert (-1: shared)
  TokList s;  // the slot's tokens
  int n0, nt; // first token of the item, tokens in it
  int rb;     // row block
};

template <int WG>
__device__ __forceinline__ bool mfma_item(const FfnArgs &a, int n_rb, MfmaItem &it) {
  using C = MfmaCfg<WG>;
  const int gmax = mfma_gmax(a.T, a.k, a.E);
  const bool g64 = C::TOK == kMfmaGroup;
  const int32_t *gslot = a.disp.mgofs + 2 * (a.E + 2) + (g64 ? 0 : gmax);
  const int4 *hdr = reinterpret_cast<const int4 *>(a.disp.mgofs + mfma_desc_off(a.T, a.k, a.E));
  const int4 *desc = hdr + 1 + (g64 ? 0 : gmax);
  const int4 h = *hdr;
  const int n_items = (g64 ? h.x : h.y) * n_rb;
  if ((int)blockIdx.x >= n_items) return false;
  const int i = n_items - 1 - (int)blockIdx.x;
  const int run = 8 * n_rb, r0 = i / run;
  // both candidate groups' descriptors and the run's end slots, loaded together
  const bool full = (r0 + 1) * run <= n_items;
  const int4 dp = desc[i / n_rb];
  int4 dt = dp;
  int s0 = 0, s7 = 0;
  if (full) {
    s0 = gslot[8 * r0];
    s7 = gslot[8 * r0 + 7];
    dt = desc[8 * r0 + i % 8];
  }
  const bool transposed = full && s7 - s0 == 7;
  const int4 d = transposed ? dt : dp;
  it.rb = transposed ? (i % run) / 8 : i % n_rb;
  it.e = d.x;
  it.s.slot = -1;
  it.s.shared = d.x < 0;
  it.s.p0 = d.y;
  it.n0 = d.z;
  it.nt = d.w;
  it.s.n_tok = d.z + d.w;
  return it.nt > 0;
}

// ---------------------------------------------------------------------------
// The block-scaled int8 GEMM core shared by both kernels.  A workgroup of 8
// waves multiplies NMAT weight matrices (128 rows each, 16 per wave) by up
// to 64 token rows of Q8_0 codes, over K in stages of CH blocks of 32.
//
// Stages go straight from memory into a ring of as many LDS buffers as fit, with
// global_load_lds (16-byte pieces for weights and codes, 4-byte ones for
// the block scales), so all other stages are in flight while one is
// multiplied, and no register holds them on the way.  Every wave issues the
// same number of load instructions per stage, so one s_waitcnt vmcnt(N)
// waits for exactly the oldest stage; a bare s_barrier (no fence, which
// would wait for every load in flight) then makes it visible to all waves.
//
// LDS layouts are XOR-swizzled in 16-byte pieces (scales in 4-byte words):
// the lanes of a wave read a 16 x 32 operand (16 rows or tokens at one k
// offset) from 64 distinct banks, and the global reads behind each load
// instruction stay contiguous per row.  Pieces past a row's end, rows past
// the matrix and tokens past the item are clamped to valid addresses; what
// they bring in is never used.
//
// The token tile count NTT is a template parameter (one loop per count), so
// a full stage's eight blocks unroll with no runtime branch.
// acc[m][tt][r]: matrix m, token tile tt, row 4 g + r of the wave's 16,
// token 16 tt + li (lane = 16 g + li).
// ---------------------------------------------------------------------------
template <int BITS, int WG>
struct MfmaGeo {
  static constexpr int CH0 = MfmaCfg<WG>::ROWB * 8 / (32 * BITS);
  static constexpr int CH = CH0 < 8 ? CH0 : 8;          // blocks per stage
  static constexpr int RB = CH * 32 * BITS / 8;         // weight bytes per row per stage
  static constexpr int PPR = RB / 16;                   // 16-byte pieces per weight row
  static constexpr int XR = CH * 32;                    // code bytes per token per stage
  static constexpr int XPR = XR / 16;                   // pieces per token
  static constexpr int KW = 256 / RB;                   // weight rows per 256 bytes of LDS
  static constexpr int KX = 256 / XR;                   // token rows per 256 bytes
};

// Swizzled positions (pieces, or words for the scales).
template <int BITS, int WG>
__device__ __forceinline__ int wkey(int r) {
  using G = MfmaGeo<BITS, WG>;
  return (r / G::KW) & (G::PPR - 1);
}
template <int BITS, int WG>
__device__ __forceinline__ int xkey(int t) {
  using G = MfmaGeo<BITS, WG>;
  return (t / G::KX) & (G::XPR - 1);
}
// The block scales of a stage, binary32 (4-byte words) or binary64 (16-byte
// pieces of two): per token CH scales in SPT pieces of PB bytes; the lanes
// reading one block's scale for 16 tokens hit distinct banks.
template <int CH, typename SC>
struct ScaleGeo {
  static constexpr bool F64 = sizeof(SC) == 8;
  static constexpr int PB = F64 ? 16 : 4;               // bytes per load piece
  static constexpr int SPT = CH * (int)sizeof(SC) / PB;  // pieces per token
  static constexpr int KD = F64 ? 256 / (CH * 8) : 8;   // tokens per key step
  __device__ static int key(int t) {
    if constexpr (F64) return (t / KD) & (SPT - 1);
    else return CH == 8 ? (t >> 3) & 7 : 0;
  }
  // LDS byte offset of token t's scale of block b within the stage's scales
  __device__ static int at(int t, int b) {
    if constexpr (F64) return t * CH * 8 + 16 * ((b >> 1) ^ key(t)) + 8 * (b & 1);
    else return (t * CH + (b ^ key(t))) * 4;
  }
};

// A stage of the ring for TS staged tokens (the item's token tiles; fewer
// tokens leave room for more stages in flight).
template <int BITS, int NMAT, int WG, typename SC, int TS = MfmaCfg<WG>::TOK>
struct MfmaStage {
  using G = MfmaGeo<BITS, WG>;
  using SG = ScaleGeo<G::CH, SC>;
  static constexpr int TOK = TS;
  static constexpr int W = NMAT * kMfmaRows * G::RB;   // weight bytes
  static constexpr int X = TOK * G::XR;                // code bytes
  static constexpr int D = TOK * G::CH * (int)sizeof(SC);  // scale bytes
  static constexpr int DPW = D / SG::PB / kMfmaWaves;  // scale pieces per wave (one instruction)
  static constexpr int BYTES = W + X + D;
  // ring depth: as many stages as fit, all but one in flight
  static constexpr int RING = MfmaCfg<WG>::RING;
  static constexpr int STAGES = RING / BYTES < kMaxStages ? RING / BYTES : kMaxStages;
  static_assert(STAGES >= 3, "ring depth");
  // load instructions per wave per stage
  static constexpr int NW = W / 16 / kMfmaThreads;
  // code pieces: NX instructions of XPW lanes each per wave
  static constexpr int PX = X / 16;
  static constexpr int NX = PX >= kMfmaThreads ? PX / kMfmaThreads : 1;
  static constexpr int XPW = PX >= kMfmaThreads ? 64 : PX / kMfmaWaves;
  static constexpr int NL = NW + NX + 1;
  static_assert(W % (16 * kMfmaThreads) == 0 && NX * kMfmaWaves * XPW == PX, "stage split");
  static_assert(DPW <= 64 && DPW * kMfmaWaves * SG::PB == D, "one scale instruction per wave");
};

// Whether a stage of TS tokens splits into whole load instructions per wave.
template <int BITS, int NMAT, int WG, typename SC, int TS>
constexpr bool stage_fits() {
  using G = MfmaGeo<BITS, WG>;
  constexpr int PX = TS * G::XR / 16;
  constexpr int NX = PX >= kMfmaThreads ? PX / kMfmaThreads : 1;
  constexpr int XPW = PX >= kMfmaThreads ? 64 : PX / kMfmaWaves;
  constexpr int D = TS * G::CH * (int)sizeof(SC);
  constexpr int PB = sizeof(SC) == 8 ? 16 : 4;
  constexpr int DPW = D / PB / kMfmaWaves;
  return NX * kMfmaWaves * XPW == PX && XPW >= 1 && DPW >= 1 && DPW <= 64 &&
         DPW * kMfmaWaves * PB == D;
}
// Tokens staged per stage for NTT token tiles: the tiles' tokens where that
// splits evenly, else the full group.
template <int BITS, int NMAT, int WG, typename SC, int NTT>
constexpr int stage_tokens() {
  return stage_fits<BITS, NMAT, WG, SC, 16 * NTT>() ? 16 * NTT : MfmaCfg<WG>::TOK;
}

template <int BITS, int NMAT, int WG, typename SC>
struct MfmaLds {
  __align__(16) unsigned char ring[MfmaCfg<WG>::RING];  // stages of any token count
  int trow[MfmaCfg<WG>::TOK];  // activation row of each token slot (clamped past the item)
  int orow[MfmaCfg<WG>::TOK];  // output row of each token slot (h row, or obuf row)
  float rsc[2 * kMfmaRows];    // the scales of the item's rows (two 128-row matrices)
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt untouched), gfx9 field layout.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Wait until at most `later` stages of NL loads each are in flight (later
// <= L): the oldest stage has landed.
template <int NL, int L>
__device__ __forceinline__ void wait_stages_left(int later) {
  if constexpr (L == 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (later >= L) wait_vm_lgkm0<NL * L>();
    else wait_stages_left<NL, L - 1>(later);
  }
}

// nrows[m]: rows of matrix m that exist (>= 1; rows past it load its last).
// act_rows bounds the activation rows the item's tokens name (trow); actd
// holds each row's block scales at a stride of sld.  The results are the
// sums of the widened (x 2^wshift) codes: the caller scales them back.
template <int BITS, int NMAT, int NTT, int WG, typename Acc, typename SC>
__device__ __forceinline__ void mfma_core(const uint8_t *const *wbase, const int *nrows,
                                          size_t row_bytes, const int8_t *act, const SC *actd,
                                          int sld, int K, int act_rows,
                                          MfmaLds<BITS, NMAT, WG, SC> &L,
                                          Acc (*acc)[MfmaCfg<WG>::TILES][4]) {
  using G = MfmaGeo<BITS, WG>;
  using ST = MfmaStage<BITS, NMAT, WG, SC, stage_tokens<BITS, NMAT, WG, SC, NTT>()>;
  using SG = typename ST::SG;
  static_assert(ST::STAGES * ST::BYTES <= (int)sizeof(L.ring) && 16 * NTT <= ST::TOK, "ring");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int nbk = K / 32, nst = (nbk + G::CH - 1) / G::CH;
  const v4i zero = {0, 0, 0, 0};
  // the accumulators live here, sized for the item, and go to acc at the end
  Acc ac[NMAT][NTT][4];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ac[m][tt][r] = (Acc)0;

  // Each lane's byte offset for every load instruction, from a base that
  // only the stage moves (so a full stage's loads need no address
  // arithmetic per lane): weight row and swizzled piece, token row and
  // piece, token row and swizzled scale word.  The matrix of weight
  // instruction i is the same for every wave.
  static_assert((kMfmaRows * G::PPR) % (kMfmaWaves * 64) == 0, "one matrix per weight instruction");
  const bool lane_offs = (uint64_t)act_rows * (uint64_t)K < (1ull << 31);
  uint32_t woff[ST::NW], xoff[ST::NX], doff = 0;
#pragma unroll
  for (int i = 0; i < ST::NW; ++i) {
    const int q = (i * kMfmaWaves + wave) * 64 + lane;
    const int m = (i * kMfmaWaves * 64) / (kMfmaRows * G::PPR);
    const int r = (q / G::PPR) % kMfmaRows, pl = q % G::PPR;
    woff[i] = (uint32_t)((size_t)min(r, nrows[m] - 1) * row_bytes) + 16u * (uint32_t)(pl ^ wkey<BITS, WG>(r));
  }
#pragma unroll
  for (int i = 0; i < ST::NX; ++i) {
    const int q = min((i * kMfmaWaves + wave) * ST::XPW + lane, ST::PX - 1);
    const int t = q / G::XPR, pl = q % G::XPR;
    xoff[i] = (uint32_t)L.trow[t] * (uint32_t)K + 16u * (uint32_t)(pl ^ xkey<BITS, WG>(t));
  }
  {
    const int q = wave * ST::DPW + lane;
    const int t = min(q / SG::SPT, ST::TOK - 1), p = q % SG::SPT;
    doff = (uint32_t)L.trow[t] * (uint32_t)(sld * sizeof(SC)) + (uint32_t)(SG::PB * (p ^ SG::key(t)));
  }

  // one stage's loads: every wave issues ST::NL instructions
  auto issue = [&](int c) {
    unsigned char *buf = L.ring + (size_t)(c % ST::STAGES) * ST::BYTES;
    if (lane_offs && (c + 1) * G::CH <= nbk) {
      // a full stage: wave-uniform bases plus the lanes' fixed offsets
#pragma unroll
      for (int i = 0; i < ST::NW; ++i) {
        const int m = (i * kMfmaWaves * 64) / (kMfmaRows * G::PPR);
        const uint8_t *src = wbase[m] + (size_t)c * G::RB + woff[i];
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + (size_t)(i * kMfmaWaves + wave) * 64 * 16),
                                         16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < ST::NX; ++i) {
        const int8_t *src = act + (size_t)c * G::XR + xoff[i];
        if (ST::XPW == 64 || lane < ST::XPW)
          __builtin_amdgcn_global_load_lds(
              src, (lds_void *)(buf + ST::W + (size_t)(i * kMfmaWaves + wave) * ST::XPW * 16), 16, 0, 0);
      }
      if (lane < ST::DPW) {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(actd + (size_t)c * G::CH) + doff;
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + ST::W + ST::X + (size_t)wave * ST::DPW * SG::PB),
                                         SG::PB, 0, 0);
      }
      return;
    }
    // the last, partial stage (or activation offsets past 31 bits): clamped
    const int valid_w = min(G::RB, (int)(row_bytes - (size_t)c * G::RB));  // bytes of this stage in a row
    const int valid_x = min(G::XR, K - c * G::XR);
#pragma unroll
    for (int i = 0; i < ST::NW; ++i) {
      const int q0 = (i * kMfmaWaves + wave) * 64, q = q0 + lane;
      const int m = q / (kMfmaRows * G::PPR), r = (q / G::PPR) % kMfmaRows, pl = q % G::PPR;
      const int gp = min(pl ^ wkey<BITS, WG>(r), valid_w / 16 - 1);
      const int rr = min(r, nrows[m] - 1);
      const uint8_t *src = wbase[m] + (size_t)rr * row_bytes + (size_t)c * G::RB + 16 * gp;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + (size_t)q0 * 16), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < ST::NX; ++i) {
      const int q0 = (i * kMfmaWaves + wave) * ST::XPW, q = min(q0 + lane, ST::PX - 1);
      const int t = q / G::XPR, pl = q % G::XPR;
      const int gp = min(pl ^ xkey<BITS, WG>(t), valid_x / 16 - 1);
      const int8_t *src = act + (size_t)L.trow[t] * K + (size_t)c * G::XR + 16 * gp;
      if (ST::XPW == 64 || lane < ST::XPW)
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + ST::W + (size_t)q0 * 16), 16, 0, 0);
    }
    {
      // the scales: wave w loads pieces [w * DPW, (w + 1) * DPW) of the
      // stage (binary64 rows are padded to whole stages: no clamp)
      const int q = wave * ST::DPW + lane;
      if (lane < ST::DPW) {
        const int t = q / SG::SPT, p = q % SG::SPT;
        size_t off;
        if constexpr (SG::F64) {
          off = (size_t)L.trow[t] * sld * 8 + (size_t)c * G::CH * 8 + SG::PB * (p ^ SG::key(t));
        } else {
          off = ((size_t)L.trow[t] * sld + min(c * G::CH + (p ^ SG::key(t)), nbk - 1)) * 4;
        }
        const uint8_t *src = reinterpret_cast<const uint8_t *>(actd) + off;
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + ST::W + ST::X + (size_t)wave * ST::DPW * SG::PB),
                                         SG::PB, 0, 0);
      }
    }
  };

  // The A operand of block b, matrix m: the packed word(s) as stored, then
  // widened to int8.
  auto a_raw = [&](const unsigned char *buf, int b, int m) -> WRaw<BITS> {
    const int r = 16 * wave + li;
    const unsigned char *wrow = buf + (size_t)(m * kMfmaRows + r) * G::RB;
    const int key = wkey<BITS, WG>(r);
    if constexpr (BITS == 8) {
      const int pc = (2 * b + (g >> 1)) ^ key;
      return *reinterpret_cast<const uint64_t *>(wrow + 16 * pc + 8 * (g & 1));
    } else if constexpr (BITS == 4) {
      return *reinterpret_cast<const uint32_t *>(wrow + 16 * (b ^ key) + 4 * g);
    } else {
      const int pc = (b >> 1) ^ key;
      return *reinterpret_cast<const uint32_t *>(wrow + 16 * pc + 8 * (b & 1) + 4 * (g >> 1));
    }
  };
  // B operand (token tile tt's codes) and the tokens' block scale
  auto b_op = [&](const unsigned char *buf, int b, int tt) -> long {
    const int t = 16 * tt + li;
    const int pc = (2 * b + (g >> 1)) ^ xkey<BITS, WG>(t);
    return *reinterpret_cast<const long *>(buf + ST::W + (size_t)t * G::XR + 16 * pc + 8 * (g & 1));
  };
  auto b_scale = [&](const unsigned char *buf, int b, int tt) -> SC {
    return *reinterpret_cast<const SC *>(buf + ST::W + ST::X + SG::at(16 * tt + li, b));
  };
  // the block's exact int32 sums (of the widened codes, below 2^24 in
  // magnitude, so exact in either type) times the token's block scale
  auto scale_acc = [&](Acc *a4, const v4i &cm, SC dj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a4[r] += (Acc)cm[r] * (Acc)dj;
  };

  auto block_step = [&](const unsigned char *buf, int b) {
    long aw[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) aw[m] = wop<BITS>(a_raw(buf, b, m), g);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const long bx = b_op(buf, b, tt);
      const SC dj = b_scale(buf, b, tt);
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const v4i cm = __builtin_amdgcn_mfma_i32_16x16x32_i8(aw[m], bx, zero, 0, 0, 0);
        scale_acc(ac[m][tt], cm, dj);
      }
    }
  };

  // NB blocks from b0, software-pipelined: every LDS operand of the NB
  // blocks is read first, then each MFMA is issued LAG products ahead of
  // the scaling of its result, so neither the LDS latency nor the MFMA's
  // is waited for product by product.
  constexpr int LAG = 2;
  auto blocks_piped = [&](auto nb_c, const unsigned char *buf, int b0) {
    constexpr int NB = decltype(nb_c)::value;
    constexpr int NM = NB * NTT * NMAT;
    WRaw<BITS> raw[NB][NMAT];
    long bx[NB][NTT];
    SC dj[NB][NTT];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) raw[b][m] = a_raw(buf, b0 + b, m);
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        bx[b][tt] = b_op(buf, b0 + b, tt);
        dj[b][tt] = b_scale(buf, b0 + b, tt);
      }
    }
    v4i cm[LAG + 1];
#pragma unroll
    for (int i = 0; i < NM + LAG; ++i) {
      if (i < NM) {
        const int b = i / (NTT * NMAT), tt = (i / NMAT) % NTT, m = i % NMAT;
        cm[i % (LAG + 1)] =
            __builtin_amdgcn_mfma_i32_16x16x32_i8(wop<BITS>(raw[b][m], g), bx[b][tt], zero, 0, 0, 0);
      }
      if (i >= LAG) {
        const int j = i - LAG;
        const int b = j / (NTT * NMAT), tt = (j / NMAT) % NTT, m = j % NMAT;
        scale_acc(ac[m][tt], cm[j % (LAG + 1)], dj[b][tt]);
      }
    }
  };

#pragma unroll
  for (int c = 0; c < ST::STAGES - 1; ++c)
    if (c < nst) issue(c);
  // stage c's data: this wave's loads of it are done once at most the later
  // stages' remain; the barrier makes every wave's visible and frees stage
  // c - 1, whose buffer then takes stage c + STAGES - 1
  auto stage_ready = [&](int c) -> const unsigned char * {
    wait_stages_left<ST::NL, ST::STAGES - 2>(min(ST::STAGES - 2, nst - 1 - c));
    __builtin_amdgcn_s_barrier();
    if (c + ST::STAGES - 1 < nst) issue(c + ST::STAGES - 1);
    return L.ring + (size_t)(c % ST::STAGES) * ST::BYTES;
  };
  // the full stages, each in one pipelined run (one or two token tiles) or
  // in runs of two blocks (more tiles: operands and accumulators leave no
  // room for more); the partial last stage, if any, after the loop, so the
  // loop body has one path and the accumulators stay in place across it
  const int nfull = nbk / G::CH;
  for (int c = 0; c < nfull; ++c) {
    const unsigned char *buf = stage_ready(c);
    if constexpr (NTT <= 2) {
      blocks_piped(std::integral_constant<int, G::CH>(), buf, 0);
    } else {
      for (int b0 = 0; b0 < G::CH; b0 += 2) blocks_piped(std::integral_constant<int, 2>(), buf, b0);
    }
  }
  if (nfull < nst) {
    const unsigned char *buf = stage_ready(nfull);
    for (int b = 0; b < nbk - nfull * G::CH; ++b) block_step(buf, b);
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][tt][r] = ac[m][tt][r];
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring (no load is in flight)
}

template <int BITS, int NMAT, int WG, typename Acc, typename SC>
__device__ __forceinline__ void mfma_core_ntt(int ntt, const uint8_t *const *wbase, const int *nrows,
                                              size_t row_bytes, const int8_t *act, const SC *actd,
                                              int sld, int K, int act_rows,
                                              MfmaLds<BITS, NMAT, WG, SC> &L,
                                              Acc (*acc)[MfmaCfg<WG>::TILES][4]) {
  constexpr int TILES = MfmaCfg<WG>::TILES;
  if (ntt <= 1) {
    mfma_core<BITS, NMAT, 1, WG>(wbase, nrows, row_bytes, act, actd, sld, K, act_rows, L, acc);
  } else if (ntt == 2 || TILES == 2) {
    mfma_core<BITS, NMAT, 2, WG>(wbase, nrows, row_bytes, act, actd, sld, K, act_rows, L, acc);
  } else if constexpr (TILES >= 4) {
    if (ntt == 3) mfma_core<BITS, NMAT, 3, WG>(wbase, nrows, row_bytes, act, actd, sld, K, act_rows, L, acc);
    else mfma_core<BITS, NMAT, 4, WG>(wbase, nrows, row_bytes, act, actd, sld, K, act_rows, L, acc);
  }
}

// Token slots of an item: activation row of each (clamped past nt), into LDS.
// The item's token rows (activations in, outputs out) and the scales of its
// weight rows (s0[0 .. c0), s1[0 .. c1), clamped), into LDS at the start, so
// the epilogue needs no further round trip to memory.
template <int TOK>
__device__ __forceinline__ void item_rows(const FfnArgs &a, const MfmaItem &it, bool hrows, int *trow,
                                          int *orow, float *rsc, const float *s0, int c0,
                                          const float *s1, int c1) {
  for (int n = threadIdx.x; n < TOK; n += kMfmaThreads) {
    int t = 0, hrow = 0, j = 0;
    tok_at(a, true, it.s, it.n0 + min(n, it.nt - 1), t, hrow, j);
    trow[n] = hrows ? hrow : t;
    orow[n] = hrows ? t * (a.k + 1) + j : hrow;
  }
  for (int i = threadIdx.x; i < 2 * kMfmaRows; i += kMfmaThreads)
    rsc[i] = i < kMfmaRows ? s0[min(i, c0 - 1)] : s1[min(i - kMfmaRows, c1 - 1)];
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + Q8_0(h): rows [128 rb, +128) of gate and up for up to
// 32 tokens (64 at int2) of one expert.  Wave w owns rows 16 w .. 16 w + 15
// of both.
// ---------------------------------------------------------------------------
// Workgroups resident per CU: two (each with half the LDS ring and 32-token
// items), so one's item start and h epilogue overlap the other's stages;
// int2's core would not fit the 128 VGPRs that leaves, so it keeps one.
template <int BITS>
constexpr int gateup_wg() { return BITS == 2 ? 1 : 2; }

template <int BITS>
__global__ __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(2 * gateup_wg<BITS>()))) void k_gateup_mfma(FfnArgs a) {
  constexpr int WG = gateup_wg<BITS>();
  constexpr int TOK = MfmaCfg<WG>::TOK, TILES = MfmaCfg<WG>::TILES;
  __shared__ MfmaLds<BITS, 2, WG, double> L;
  const int H = a.L.H, I = a.L.I;
  MfmaItem it;
  if (!mfma_item<WG>(a, (I + kMfmaRows - 1) / kMfmaRows, it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const ExpertPtrs ep = expert_ptrs(a.L, it.e);
  const size_t row_bytes = (size_t)H * BITS / 8;
  const int rb0 = it.rb * kMfmaRows, nrows = min(kMfmaRows, I - rb0);
  item_rows<TOK>(a, it, false, L.trow, L.orow, L.rsc, ep.sg + rb0, nrows, ep.su + rb0, nrows);
  const uint8_t *wb[2] = {ep.wg + (size_t)rb0 * row_bytes, ep.wu + (size_t)rb0 * row_bytes};
  const int nr[2] = {nrows, nrows};
  // g and u accumulate in binary64 (the expert definition's sum, rounded
  // once), so h -- and its Q8_0 codes -- are those of that definition
  double acc[2][TILES][4];
  const int ntt = (it.nt + 15) >> 4;
  mfma_core_ntt<BITS, 2, WG>(ntt, wb, nr, row_bytes, a.xq, a.xd64, xd64_ld(H), H, a.T, L, acc);

  // h = silu(g) * u for rows 4 g + r of the wave, token 16 tt + li, staged
  // in LDS (over the ring) for the Q8_0 step
  static_assert(sizeof(float) * TOK * (kMfmaRows + 1) <= sizeof(L.ring), "h tile");
  float(*hs)[kMfmaRows + 1] = reinterpret_cast<float(*)[kMfmaRows + 1]>(L.ring);
  const int rw = 16 * wave + 4 * g;  // the lane's first row in the block
  // the sums are of codes widened by 2^wshift: a power of two, undone exactly
  constexpr double unw = 1.0 / (double)(1 << wshift<BITS>());
  float sg[4], su[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = min(rw + r, nrows - 1);
    sg[r] = L.rsc[row];
    su[r] = L.rsc[kMfmaRows + row];
  }
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt)
    if (tt < ntt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hs[16 * tt + li][rw + r] = swiglu_h(row_out(acc[0][tt][r] * unw, sg[r]), row_out(acc[1][tt][r] * unw, su[r]));
  __syncthreads();
  // Q8_0 of each token's 32-row blocks of h: 32 threads per block
  const int nblk = nrows / 32;
  for (int q = threadIdx.x; q < it.nt * kMfmaRows; q += kMfmaThreads) {
    const int tl = q / kMfmaRows, bb = (q / 32) % (kMfmaRows / 32), i = q & 31;
    const float h = hs[tl][bb * 32 + i];
    float amax = group_max<32>(fabsf(h));
    amax = __shfl(amax, (lane & 32) | 31, 64);
    if (bb < nblk) {
      const int hrow = L.orow[tl];
      const float db = amax / 127.f;
      float c = 0.f;
      if (db != 0.f) c = fminf(fmaxf(rintf(h / db), -127.f), 127.f);
      const int blk = rb0 / 32 + bb;
      a.hq[(size_t)hrow * I + blk * 32 + perm_dst<BITS>(i)] = (int8_t)c;
      if (i == 0) a.hd[(size_t)hrow * (I / 32) + blk] = db;
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection: output rows [256 rb, +256) for up to 32 tokens (64 at
// int2) of one expert (two 128-row halves, the core's two matrices), o into the
// per-(token, slot) buffer the combine kernel reduces.
// ---------------------------------------------------------------------------
constexpr int kDownRows = 2 * kMfmaRows;

// two resident workgroups, except for int2 (whose core would not fit 128 VGPRs)
template <int BITS>
constexpr int down_wg() { return BITS == 2 ? 1 : 2; }

template <int BITS>
__global__ __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(2 * down_wg<BITS>()))) void k_down_mfma(FfnArgs a) {
  constexpr int WG = down_wg<BITS>();
  constexpr int TOK = MfmaCfg<WG>::TOK, TILES = MfmaCfg<WG>::TILES;
  __shared__ MfmaLds<BITS, 2, WG, float> L;
  const int H = a.L.H, I = a.L.I;
  MfmaItem it;
  if (!mfma_item<WG>(a, (H + kDownRows - 1) / kDownRows, it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const ExpertPtrs ep = expert_ptrs(a.L, it.e);
  const size_t row_bytes = (size_t)I * BITS / 8;
  const int rb0 = it.rb * kDownRows, nrows = min(kDownRows, H - rb0);
  item_rows<TOK>(a, it, true, L.trow, L.orow, L.rsc, ep.sd + rb0, min(nrows, kMfmaRows),
                 ep.sd + rb0 + (nrows > kMfmaRows ? kMfmaRows : 0), max(1, nrows - kMfmaRows));
  // half 1 may not exist at the matrix edge: its loads then read half 0's rows
  const int nr[2] = {min(nrows, kMfmaRows), max(1, nrows - kMfmaRows)};
  const uint8_t *wb[2] = {ep.wd + (size_t)rb0 * row_bytes,
                          ep.wd + (size_t)(nrows > kMfmaRows ? rb0 + kMfmaRows : rb0) * row_bytes};
  float acc[2][TILES][4];
  const int ntt = (it.nt + 15) >> 4;
  mfma_core_ntt<BITS, 2, WG>(ntt, wb, nr, row_bytes, a.hq, a.hd, I / 32, I, a.T * (a.k + 1), L, acc);

  const int rw = 16 * wave + 4 * g;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int row = m * kMfmaRows + rw;  // first of the lane's 4 rows in the block
    if (row >= nrows) continue;          // rows past the matrix: whole quads
    constexpr float unw = 1.0f / (float)(1 << wshift<BITS>());
    float sd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sd[r] = L.rsc[row + r];
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      const int n = 16 * tt + li;
      if (tt < ntt && n < it.nt) {
        float4 o;
        o.x = acc[m][tt][0] * unw * sd[0];
        o.y = acc[m][tt][1] * unw * sd[1];
        o.z = acc[m][tt][2] * unw * sd[2];
        o.w = acc[m][tt][3] * unw * sd[3];
        *reinterpret_cast<float4 *>(a.obuf + (size_t)L.orow[n] * H + rb0 + row) = o;
      }
    }
  }
}

// Upper bound of the token groups a batch can send here: routed pairs in
// groups of tok plus one partial group per unique expert that can reach
// mfma_min tokens (at most pairs / mfma_min of them), plus the shared
// expert's groups when the batch reaches its threshold.
static int mfma_group_bound(const FfnArgs &a, int tok) {
  const long pairs = (long)a.T * a.k;
  long cap = pairs < a.E ? pairs : a.E;
  if (pairs / a.mfma_min < cap) cap = pairs / a.mfma_min;
  const long shared = a.T >= a.mfma_min_shared ? (a.T + tok - 1) / tok : 0;
  return (int)((pairs + tok - 1) / tok + cap + shared);
}

// Grid: one workgroup per item (an upper bound; surplus workgroups exit).
template <int WG>
static dim3 mfma_grid(const FfnArgs &a, int n_rb) {
  return dim3((unsigned)(mfma_group_bound(a, MfmaCfg<WG>::TOK) * n_rb));
}


hipError_t launch_gateup_mfma(const FfnArgs &a, hipStream_t st, KEvents ev) {
  const int n_rb = (a.L.I + kMfmaRows - 1) / kMfmaRows;
  const dim3 block(kMfmaThreads);
  switch (a.L.bits) {
    case 8: COLI_LAUNCH(ev, k_gateup_mfma<8>, mfma_grid<gateup_wg<8>()>(a, n_rb), block, 0, st, a); break;
    case 4: COLI_LAUNCH(ev, k_gateup_mfma<4>, mfma_grid<gateup_wg<4>()>(a, n_rb), block, 0, st, a); break;
    case 2: COLI_LAUNCH(ev, k_gateup_mfma<2>, mfma_grid<gateup_wg<2>()>(a, n_rb), block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_mfma(const FfnArgs &a, hipStream_t st, KEvents ev) {
  const int n_rb = (a.L.H + kDownRows - 1) / kDownRows;
  const dim3 block(kMfmaThreads);
  switch (a.L.bits) {
    case 8: COLI_LAUNCH(ev, k_down_mfma<8>, mfma_grid<down_wg<8>()>(a, n_rb), block, 0, st, a); break;
    case 4: COLI_LAUNCH(ev, k_down_mfma<4>, mfma_grid<down_wg<4>()>(a, n_rb), block, 0, st, a); break;
    case 2: COLI_LAUNCH(ev, k_down_mfma<2>, mfma_grid<down_wg<2>()>(a, n_rb), block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
