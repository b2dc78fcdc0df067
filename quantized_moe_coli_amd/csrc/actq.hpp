// actq.hpp -- Q8_0-style quantisation of one block of 32 activations
// (colibrì README, "Implemented features": integer dot products against
// Q8_0-style int8 activations).  d = amax/127 (IEEE binary32 division);
// q = clamp(round_half_even(x/d), -127, 127); d = 0 gives q = 0.  The 32 codes
// are stored in the ordering the weight container BITS consumes (perm_src).
#pragma once

#include "device.hpp"

namespace coli {

template <int BITS>
__device__ __forceinline__ void act_quant_block(const float *__restrict__ xb, int8_t *__restrict__ qb,
                                                float *__restrict__ db) {
  const float4 *x4 = reinterpret_cast<const float4 *>(xb);
  float v[32];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float4 f = x4[m];
    v[4 * m] = f.x; v[4 * m + 1] = f.y; v[4 * m + 2] = f.z; v[4 * m + 3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) amax = fmaxf(amax, fabsf(v[m]));
  const float d = amax / 127.f;
  *db = d;
  uint32_t words[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) words[m] = 0;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    float c = 0.f;
    if (d != 0.f) c = fminf(fmaxf(rintf(v[perm_src<BITS>(s)] / d), -127.f), 127.f);
    words[s >> 2] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (s & 3));
  }
  uint4 *out = reinterpret_cast<uint4 *>(qb);
  out[0] = make_uint4(words[0], words[1], words[2], words[3]);
  out[1] = make_uint4(words[4], words[5], words[6], words[7]);
}

// The same quantisation of a whole row of n values (n % 32 == 0, at most
// 8192) by the first NT threads of a workgroup, eight lanes per block of 32
// (four values each, one 16-byte load), writing the codes in the container
// ordering and one scale per block.  load() issues every load of the thread; quantize() then uses
// them, so other loads can be issued in between.  The block's amax is a max
// over its lanes (exact in any order), so codes and scales equal
// act_quant_block's.
template <int BITS, int NT>
struct ActRow {
  static constexpr int kPasses = 2048 / NT;  // blocks per group of eight threads, at most
  float4 v[kPasses];

  __device__ __forceinline__ void load(const float *__restrict__ x, int n) {
    const int tid = threadIdx.x, part = tid & 7, nb = n / 32;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int blk = p * (NT / 8) + tid / 8;
      v[p] = blk < nb ? reinterpret_cast<const float4 *>(x + (size_t)blk * 32)[part]
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void quantize(int n, int8_t *__restrict__ q, float *__restrict__ d) {
    const int tid = threadIdx.x, part = tid & 7, nb = n / 32;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int blk = p * (NT / 8) + tid / 8;
      if (p * (NT / 8) >= nb) break;  // uniform
      float m = fmaxf(fmaxf(fabsf(v[p].x), fabsf(v[p].y)), fmaxf(fabsf(v[p].z), fabsf(v[p].w)));
      m = group_max<8>(m);  // every lane of the eight holds the block's amax
      const float dd = m / 127.f;
      if (blk < nb) {
        if (part == 0) d[blk] = dd;
        const float e[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float c = 0.f;
          if (dd != 0.f) c = fminf(fmaxf(rintf(e[j] / dd), -127.f), 127.f);
          q[(size_t)blk * 32 + perm_dst<BITS>(4 * part + j)] = (int8_t)c;
        }
      }
    }
  }
};

}  // namespace coli
