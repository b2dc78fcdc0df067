// device.hpp -- gfx950 device helpers shared by the library's kernels:
// wave reductions over DPP, integer dot products of one 16-byte weight chunk
// against Q8_0 activation codes, and the activation orderings that make the
// in-register unpacking of packed int4 / int2 codes cheap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Cross-lane moves.  DPP control codes (GCN/CDNA "DPP" instruction modifier):
//   quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
//   row_mirror = 0x140, row_half_mirror = 0x141,
//   row_bcast:15 = 0x142, row_bcast:31 = 0x143.
// A lane outside row_mask keeps `old` (here 0).
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over aligned groups of L lanes (L in 1,2,4,...,64).  For L <= 16 every
// lane of the group ends with the group sum; for L = 32 the sum is valid in
// lane 31 of each half; for L = 64 in lane 63.  Fixed pattern, so results are
// bit-reproducible run to run.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (L >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (L >= 8) v += dpp_f32<0x141>(v);
  if constexpr (L >= 16) v += dpp_f32<0x140>(v);
  if constexpr (L >= 32) v += dpp_f32<0x142, 0xA>(v);
  if constexpr (L >= 64) v += dpp_f32<0x143, 0xC>(v);
  return v;
}

// Lane holding the group sum after group_sum<L> for the group of `lane`.
template <int L>
__device__ __forceinline__ int group_sum_lane(int lane) {
  if constexpr (L <= 16) return lane;
  else if constexpr (L == 32) return (lane & 32) | 31;
  else return 63;
}

template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 2) v = fmaxf(v, dpp_f32<0xB1>(v));
  if constexpr (L >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));
  if constexpr (L >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (L >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  if constexpr (L >= 32) v = fmaxf(v, dpp_f32<0x142, 0xA>(v));
  if constexpr (L >= 64) v = fmaxf(v, dpp_f32<0x143, 0xC>(v));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<64>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = group_max<64>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// DPP move of a binary64 value (both 32-bit halves take the same pattern).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFFll), CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// group_sum<L> in binary64: the same lanes hold the result, same fixed
// pattern (lanes outside a row mask read +0, which adds exactly nothing).
template <int L>
__device__ __forceinline__ double group_sum_f64(double v) {
  if constexpr (L >= 2) v += dpp_f64<0xB1>(v);
  if constexpr (L >= 4) v += dpp_f64<0x4E>(v);
  if constexpr (L >= 8) v += dpp_f64<0x141>(v);
  if constexpr (L >= 16) v += dpp_f64<0x140>(v);
  if constexpr (L >= 32) v += dpp_f64<0x142, 0xA>(v);
  if constexpr (L >= 64) v += dpp_f64<0x143, 0xC>(v);
  return v;
}

// Sum over the wave in binary64 (DPP steps, then lane 63 broadcast).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = group_sum_f64<64>(v);
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// ---------------------------------------------------------------------------
// Containers.  A "chunk" is the 16 bytes of packed weights one lane loads at
// a time: 16 int8 codes (half a Q8_0 block), 32 int4 codes (one block) or
// 64 int2 codes (two blocks).
// ---------------------------------------------------------------------------
template <int BITS> struct Q;
template <> struct Q<8> { static constexpr int kElems = 16, kBlocks = 1, kShift = 0; };
template <> struct Q<4> { static constexpr int kElems = 32, kBlocks = 1, kShift = 4; };
template <> struct Q<2> { static constexpr int kElems = 64, kBlocks = 2, kShift = 6; };

// Activation ordering inside a Q8_0 block, chosen per weight container so a
// lane can feed shifted-and-masked weight words straight into dot4:
//   int8: natural order;
//   int4: per 8 values [0,2,4,6,1,3,5,7] (low nibbles, then high nibbles);
//   int2: per 16 values [0,4,8,12, 1,5,9,13, 2,6,10,14, 3,7,11,15].
// perm_src<BITS>(s) is the natural index stored at position s of the group.
template <int BITS>
__host__ __device__ __forceinline__ int perm_src(int s) {
  if constexpr (BITS == 4) {
    const int g = s & ~7, r = s & 7;
    return g + (r < 4 ? 2 * r : 2 * (r - 4) + 1);
  } else if constexpr (BITS == 2) {
    const int g = s & ~15, r = s & 15;
    return g + 4 * (r & 3) + (r >> 2);
  } else {
    return s;
  }
}

template <int BITS>
__host__ __device__ __forceinline__ int perm_dst(int n) {  // inverse of perm_src
  if constexpr (BITS == 4) {
    const int g = n & ~7, r = n & 7;
    return g + ((r & 1) ? 4 + (r >> 1) : (r >> 1));
  } else if constexpr (BITS == 2) {
    const int g = n & ~15, r = n & 15;
    return g + 4 * (r & 3) + (r >> 2);
  } else {
    return n;
  }
}

__device__ __forceinline__ int dot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Integer products of one 16-byte weight chunk with the matching activation
// codes (in the container's ordering).  Results are exact int32 block sums
// (the shift undoes the x16 / x64 of the in-place sign extension, exactly,
// since every product is a multiple of it).
//   int8: act = 16 codes (4 words), returns the partial sum of half a block;
//   int4: act = 32 codes (8 words), returns one block sum;
//   int2: act = 64 codes (16 words), returns two block sums.
__device__ __forceinline__ int chunk_dot_q8(const uint4 w, const int *a) {
  int acc = 0;
  acc = dot4((int)w.x, a[0], acc);
  acc = dot4((int)w.y, a[1], acc);
  acc = dot4((int)w.z, a[2], acc);
  acc = dot4((int)w.w, a[3], acc);
  return acc;
}

__device__ __forceinline__ int chunk_dot_q4(const uint4 w, const int *a) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  int acc = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int lo = (int)((ws[m] << 4) & 0xF0F0F0F0u);  // elements 8m+0,2,4,6 (x16)
    const int hi = (int)(ws[m] & 0xF0F0F0F0u);         // elements 8m+1,3,5,7 (x16)
    acc = dot4(lo, a[2 * m], acc);
    acc = dot4(hi, a[2 * m + 1], acc);
  }
  return acc >> 4;
}

__device__ __forceinline__ void chunk_dot_q2(const uint4 w, const int *a, int &b0, int &b1) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  int acc[2] = {0, 0};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    int s = acc[m >> 1];
    s = dot4((int)((ws[m] << 6) & 0xC0C0C0C0u), a[4 * m + 0], s);  // elements 16m+0,4,8,12 (x64)
    s = dot4((int)((ws[m] << 4) & 0xC0C0C0C0u), a[4 * m + 1], s);
    s = dot4((int)((ws[m] << 2) & 0xC0C0C0C0u), a[4 * m + 2], s);
    s = dot4((int)(ws[m] & 0xC0C0C0C0u), a[4 * m + 3], s);
    acc[m >> 1] = s;
  }
  b0 = acc[0] >> 6;
  b1 = acc[1] >> 6;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load for weights that are read once.
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace coli
