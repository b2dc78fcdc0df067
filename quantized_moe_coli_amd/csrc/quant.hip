// quant.hip -- weight quantisation + packing and Q8_0 activation
// quantisation for gfx950.
//
// Weight containers: colibrì README, "Implemented features" (int8 / packed
// int4 / packed int2 kernels, one scale per row, dequantised on use; packing
// bit-identical to the int8 container).  Activations: same section (integer
// dot products against Q8_0-style int8 activations).  Both follow the
// symmetric-absmax reading with a correctly rounded binary32 division and
// round-half-even, so the codes and scales are bit-identical to any IEEE
// implementation of the same rule.
#include "actq.hpp"
#include "kernels.hpp"

namespace coli {

// One wave per row.  Each lane produces whole 32-bit words of packed output
// (4 int8, 8 int4 or 16 int2 codes) from the matching run of fp32 inputs.
template <int BITS>
__global__ __launch_bounds__(256) void k_quant_pack(const float *__restrict__ w, int64_t rows,
                                                    int64_t cols, uint32_t *__restrict__ q,
                                                    float *__restrict__ scale) {
  constexpr int kPer = 32 / BITS;                 // codes per output word
  constexpr float kQmax = BITS == 8 ? 127.f : (BITS == 4 ? 7.f : 1.f);
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float *wr = w + row * cols;

  float amax = 0.f;
  for (int64_t c = lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(wr[c]));
  amax = wave_max(amax);
  const float s = amax / kQmax;  // IEEE binary32 division
  if (lane == 0) scale[row] = s;

  const int64_t words = cols / kPer;
  uint32_t *qr = q + row * words;
  for (int64_t j = lane; j < words; j += 64) {
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      float v = 0.f;
      if (s != 0.f) v = fminf(fmaxf(rintf(wr[j * kPer + m] / s), -kQmax), kQmax);
      word |= ((uint32_t)(int32_t)v & kMask) << (BITS * m);
    }
    qr[j] = word;
  }
}

// One thread per Q8_0 block of 32 values (act_quant_block, actq.hpp).
template <int BITS>
__global__ __launch_bounds__(256) void k_act_quant(const float *__restrict__ x, int64_t T,
                                                   int64_t n, int8_t *__restrict__ q,
                                                   float *__restrict__ d) {
  const int64_t nb = n / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * nb) return;
  const int64_t t = i / nb, b = i % nb;
  act_quant_block<BITS>(x + t * n + b * 32, q + t * n + b * 32, d + i);
}

hipError_t launch_quant_pack(int bits, const float *w, int64_t rows, int64_t cols, uint8_t *q,
                             float *scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  uint32_t *qw = reinterpret_cast<uint32_t *>(q);
  switch (bits) {
    case 8: hipLaunchKernelGGL(k_quant_pack<8>, grid, block, 0, st, w, rows, cols, qw, scale); break;
    case 4: hipLaunchKernelGGL(k_quant_pack<4>, grid, block, 0, st, w, rows, cols, qw, scale); break;
    case 2: hipLaunchKernelGGL(k_quant_pack<2>, grid, block, 0, st, w, rows, cols, qw, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_act_quant(int layout_bits, const float *x, int64_t T, int64_t n, int8_t *q,
                            float *d, hipStream_t st, KEvents ev) {
  const int64_t blocks = T * (n / 32);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)((blocks + 255) / 256)), block(256);
  switch (layout_bits) {
    case 8: COLI_LAUNCH(ev, k_act_quant<8>, grid, block, 0, st, x, T, n, q, d); break;
    case 4: COLI_LAUNCH(ev, k_act_quant<4>, grid, block, 0, st, x, T, n, q, d); break;
    case 2: COLI_LAUNCH(ev, k_act_quant<2>, grid, block, 0, st, x, T, n, q, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
