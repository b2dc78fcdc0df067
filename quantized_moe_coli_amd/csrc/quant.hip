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

// FP8 checkpoint requantisation (colibrì README, "Implemented features": the
// offline FP8 -> int4 converter dequantises the checkpoint's 128x128
// block-scaled FP8 weights and requantises them into the engine's
// container).  The FP8 format is OCP E4M3 without infinities: bit 7 sign,
// bits 6..3 exponent (bias 7), bits 2..0 mantissa; exponent 0 is subnormal
// (m * 2^-9), exponent 15 with mantissa 7 is NaN.  Decoded here by placing
// the fields into a binary32 word, which is exact for every code.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// The same value for the 127 magnitudes that are not NaN, in two
// operations: the code's seven magnitude bits placed at the top of a
// binary32 mantissa/exponent give (1 + m/8) * 2^(e-127) (or the subnormal
// m/8 * 2^-126 for e = 0), which the exact product with 2^120 turns into
// the code's value; the sign bit is copied.  The NaN codes give 480.
__device__ __forceinline__ float e4m3_fast(uint32_t c) {
  return __uint_as_float(((c & 0x7Fu) << 20) | ((c & 0x80u) << 24)) * 0x1p120f;
}

// The 16 dequantised values of one 16-byte chunk of codes: each code's value
// times its block's scale, one correctly rounded binary32 product.
__device__ __forceinline__ void fp8_chunk(const uint4 c, float s, float (&v)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = e4m3_fast((w[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s;
}

// Quantises and packs the 16 values of one chunk (same rule as
// k_quant_pack; s != 0, r = fl32(1/s)) and stores them as one 4-, 8- or
// 16-byte group, so that consecutive lanes write consecutive bytes.
// round_half_even(fl32(v / s)) comes from a multiplication by r:
// y = fl32(v * r) is within 3 * 2^-24 * |v/s| of fl32(v/s) (one rounding in
// r, one in y; |v/s| <= qmax + 1, so within 2^-15), so wherever y lies more
// than 2^-15 from every half-integer both round to the same integer.  A
// chunk with a value closer than that (or a non-finite y) in any lane of the
// wave is redone with the correctly rounded division, in a branch the whole
// wave takes together.  The codes equal k_quant_pack's.
template <int BITS>
__device__ __forceinline__ void fp8_store_chunk(const float (&v)[16], float s, float r, uint32_t *dst,
                                                int64_t j) {
  constexpr float kQmax = BITS == 8 ? 127.f : (BITS == 4 ? 7.f : 1.f);
  constexpr int kPer = 32 / BITS;  // codes per 32-bit output word
  constexpr int kWords = 16 / kPer;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  float c[16];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = v[i] * r;
    c[i] = rintf(y);
    // more than 2^-15 from every half-integer <=> within 0.5 - 2^-15 of the
    // nearest integer (y - rint(y) is exact: the operands are within a
    // factor of two of each other, or rint(y) is zero); NaN and infinities
    // fail the test
    near |= !(fabsf(y - c[i]) < 0.5f - 0x1p-15f);
  }
  if (__ballot(near)) {
    if (near) {
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = rintf(v[i] / s);
    }
  }
  uint32_t word[kWords];
#pragma unroll
  for (int k = 0; k < kWords; ++k) word[k] = 0;
  if (s != 0.f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float q = __builtin_amdgcn_fmed3f(c[i], -kQmax, kQmax);
      word[i / kPer] |= ((uint32_t)(int32_t)q & kMask) << (BITS * (i % kPer));
    }
  }
  if constexpr (kWords == 4)
    reinterpret_cast<uint4 *>(dst)[j] = make_uint4(word[0], word[1], word[2], word[3]);
  else if constexpr (kWords == 2)
    reinterpret_cast<uint2 *>(dst)[j] = make_uint2(word[0], word[1]);
  else
    dst[j] = word[0];
}

// TPR threads (one to four waves) per row, 256 / TPR rows per workgroup; a
// thread handles 16-byte chunks of 16 codes, chunk j lying in block column
// j/8.  NC > 0: the row has at most TPR*NC chunks, and each thread loads
// all of its chunks at once and keeps them in registers (one read of the
// row, every load in flight together); the row's absmax (wave DPP maxima,
// then across the row's waves in LDS) and the codes are computed from the
// registers.  NC = 0: longer rows, read twice (the second time from cache).
template <int BITS, int TPR, int NC>
__global__ __launch_bounds__(256) void k_quant_pack_fp8(const uint8_t *__restrict__ w8,
                                                        const float *__restrict__ bscale,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t *__restrict__ q,
                                                        float *__restrict__ scale) {
  constexpr float kQmax = BITS == 8 ? 127.f : (BITS == 4 ? 7.f : 1.f);
  constexpr int kWpr = TPR / 64;  // waves per row
  __shared__ float wmax[4];
  const int tr = threadIdx.x % TPR, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const bool active = row < rows;  // uniform per wave
  const int64_t chunks = cols / 16;
  const int64_t rr = active ? row : 0;
  const uint4 *src = reinterpret_cast<const uint4 *>(w8 + rr * cols);
  const float *bs = bscale + (rr / 128) * ((cols + 127) / 128);
  uint32_t *dst = reinterpret_cast<uint32_t *>(q + rr * (cols * BITS / 8));

  // the row's absmax: each wave's maximum, then the row's waves' maxima
  auto row_max = [&](float m) {
    m = wave_max(m);
    if constexpr (kWpr > 1) {
      if (lane == 0) wmax[wave] = m;
      __syncthreads();
      const int w0 = wave - wave % kWpr;
#pragma unroll
      for (int i = 0; i < kWpr; ++i) m = fmaxf(m, wmax[w0 + i]);
    }
    return m;
  };

  if constexpr (NC > 0) {
    uint4 c[NC];
    float sc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t j = tr + (int64_t)TPR * i;
      const bool ok = active && j < chunks;
      c[i] = ok ? src[j] : make_uint4(0, 0, 0, 0);
      sc[i] = ok ? bs[j >> 3] : 0.f;
    }
    // E4M3 magnitudes grow with the low seven bits of the code and binary32
    // rounding is monotonic, so a chunk's largest |value * scale| is that of
    // its largest seven-bit magnitude: one decode per chunk
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint32_t w[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      uint32_t m = 0;
#pragma unroll
      for (int b = 0; b < 16; ++b) m = max(m, (w[b >> 2] >> (8 * (b & 3))) & 0x7Fu);
      amax = fmaxf(amax, fabsf(e4m3_value(m) * sc[i]));
    }
    amax = row_max(amax);
    if (!active) return;
    const float s = amax / kQmax;  // IEEE binary32 division
    const float r = 1.f / s;
    if (tr == 0) scale[row] = s;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t j = tr + (int64_t)TPR * i;
      if (j < chunks) {
        float v[16];
        fp8_chunk(c[i], sc[i], v);
        fp8_store_chunk<BITS>(v, s, r, dst, j);
      }
    }
  } else {
    float amax = 0.f;
    for (int64_t j = tr; active && j < chunks; j += TPR) {
      float v[16];
      fp8_chunk(src[j], bs[j >> 3], v);
#pragma unroll
      for (int m = 0; m < 16; ++m) amax = fmaxf(amax, fabsf(v[m]));
    }
    amax = row_max(amax);
    if (!active) return;
    const float s = amax / kQmax;
    const float r = 1.f / s;
    if (tr == 0) scale[row] = s;
    for (int64_t j = tr; j < chunks; j += TPR) {
      float v[16];
      fp8_chunk(src[j], bs[j >> 3], v);
      fp8_store_chunk<BITS>(v, s, r, dst, j);
    }
  }
}

// One thread per Q8_0 block of 32 values (act_quant_block, actq.hpp); with
// d64, each block scale also in binary64 (row stride xd64_ld(n)).
template <int BITS>
__global__ __launch_bounds__(256) void k_act_quant(const float *__restrict__ x, int64_t T,
                                                   int64_t n, int8_t *__restrict__ q,
                                                   float *__restrict__ d, double *__restrict__ d64) {
  const int64_t nb = n / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * nb) return;
  const int64_t t = i / nb, b = i % nb;
  act_quant_block<BITS>(x + t * n + b * 32, q + t * n + b * 32, d + i);
  if (d64) d64[t * xd64_ld(n) + b] = (double)d[i];
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

// f32-activation variant of the quantised product (colibrì README,
// "Implemented features": for a single row the int4 kernel keeps its
// activations in f32, measured faster than the integer path there):
// y[r] = s_r * sum_c code[r][c] * x[c] for one token.  The codes are taken
// in offset binary, u = code + B (B = 2^(BITS-1)): flipping each field's
// sign bit turns a two's complement field into u, masking spreads a word's
// fields over the bytes of NS words (byte b of group s: field s + NS*b of
// the word), and v_cvt_f32_ubyte converts each byte; so a weight costs a
// byte conversion, an FMA and a fraction of an integer op.  The sum of
// u * x then loses B * sum(x), one correction per row (sum(x) is the same
// for every row).  x is staged in LDS once per workgroup in the order the
// bytes consume it, the float4 groups of a chunk rotated by the chunk
// index so the lanes of a wave (one chunk each) read different banks.  A
// wave owns RW rows; a lane takes chunks lane, lane + 64, ... of each, all
// loaded at once.  fp32 sums, wave-reduced with DPP.
template <int BITS>
struct F32Act {
  static constexpr int NS = BITS == 8 ? 1 : BITS == 4 ? 2 : 4;  // byte groups per word
  static constexpr int G = 4 * NS;                               // float4 groups per chunk
  static constexpr int FPW = 32 / BITS;                          // fields per word
  static constexpr uint32_t FLIP = BITS == 8 ? 0x80808080u : BITS == 4 ? 0x88888888u : 0xAAAAAAAAu;
  static constexpr uint32_t MASK = BITS == 8 ? 0xFFFFFFFFu : BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
  static constexpr float BIAS = (float)(1 << (BITS - 1));
  // element (within the chunk) of byte b of group s of word w
  __host__ __device__ static int elem(int w, int s, int b) { return w * FPW + s + NS * b; }
};

template <int BITS, int CPL, int RW>
__global__ __launch_bounds__(256) void k_gemv_f32act(const uint8_t *__restrict__ W,
                                                     const float *__restrict__ scale, int64_t rows,
                                                     int64_t cols, const float *__restrict__ x,
                                                     float *__restrict__ y) {
  using F = F32Act<BITS>;
  constexpr int kElems = 128 / BITS;
  extern __shared__ __align__(16) float xs[];
  __shared__ float xsum_w[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nchunks = cols * BITS / 128;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RW;
  const size_t row_bytes = (size_t)cols * BITS / 8;
  uint4 wv[RW][CPL];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int64_t row = min(row0 + rr, rows - 1);
    const uint4 *wr = reinterpret_cast<const uint4 *>(W + row * row_bytes);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t c = lane + 64 * i;
      wv[rr][i] = c < nchunks ? ld_nt(wr + c) : make_uint4(F::FLIP, F::FLIP, F::FLIP, F::FLIP);
    }
  }
  // x into LDS, read as float4 and each value written to its place (byte b
  // of group g = NS * w + s of chunk c at float4 c*G + (g + c) % G), and
  // sum(x): each thread's values in order, then the waves' in order
  float part = 0.f;
  for (int64_t q = threadIdx.x; q < nchunks * (kElems / 4); q += 256) {
    const float4 v = reinterpret_cast<const float4 *>(x)[q];
    const int64_t c = q / (kElems / 4);
    const int e0 = (int)(q - c * (kElems / 4)) * 4;  // first element (within the chunk)
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = e0 + m, w = e / F::FPW, j = e % F::FPW, s = j % F::NS, b = j / F::NS;
      const int g = F::NS * w + s;
      xs[(c * F::G + (g + c) % F::G) * 4 + b] = vv[m];
    }
    part += ((v.x + v.y) + (v.z + v.w));
  }
  part = wave_sum(part);
  if (lane == 0) xsum_w[wave] = part;
  __syncthreads();
  const float xsum = (xsum_w[0] + xsum_w[1]) + (xsum_w[2] + xsum_w[3]);
  float acc[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) acc[rr] = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int64_t c = lane + 64 * i;
    if (c < nchunks) {
      const float4 *xc = reinterpret_cast<const float4 *>(xs) + c * F::G;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int s = 0; s < F::NS; ++s) {
          const int g = F::NS * w + s;
          const float4 v = xc[(g + c) % F::G];
#pragma unroll
          for (int rr = 0; rr < RW; ++rr) {
            const uint32_t word = w == 0 ? wv[rr][i].x : w == 1 ? wv[rr][i].y : w == 2 ? wv[rr][i].z : wv[rr][i].w;
            uint32_t u = ((word ^ F::FLIP) >> (BITS * s)) & F::MASK;
            // keep the masked word whole, so each byte converts straight
            // from it (v_cvt_f32_ubyte0..3) instead of a field extract first
            asm volatile("" : "+v"(u));
            acc[rr] = fmaf((float)(u & 0xFFu), v.x, acc[rr]);
            acc[rr] = fmaf((float)((u >> 8) & 0xFFu), v.y, acc[rr]);
            acc[rr] = fmaf((float)((u >> 16) & 0xFFu), v.z, acc[rr]);
            acc[rr] = fmaf((float)(u >> 24), v.w, acc[rr]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const float sum = wave_sum(acc[rr]);
    if (lane == 0 && row0 + rr < rows) y[row0 + rr] = scale[row0 + rr] * fmaf(-F::BIAS, xsum, sum);
  }
}

template <int BITS, int CPL, int RW>
static hipError_t launch_gemv_f32act_t(const uint8_t *W, const float *scale, int64_t rows,
                                       int64_t cols, const float *x, float *y, hipStream_t st) {
  const dim3 grid((unsigned)((rows + 4 * RW - 1) / (4 * RW))), block(256);
  hipLaunchKernelGGL((k_gemv_f32act<BITS, CPL, RW>), grid, block, (size_t)cols * 4, st, W, scale,
                     rows, cols, x, y);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_gemv_f32act_bits(const uint8_t *W, const float *scale, int64_t rows,
                                          int64_t cols, const float *x, float *y, hipStream_t st) {
  const int64_t per = (cols * BITS / 128 + 63) / 64;  // chunks per lane
  if (per <= 1) return launch_gemv_f32act_t<BITS, 1, 4>(W, scale, rows, cols, x, y, st);
  if (per <= 2) return launch_gemv_f32act_t<BITS, 2, 4>(W, scale, rows, cols, x, y, st);
  if (per <= 3) return launch_gemv_f32act_t<BITS, 3, 2>(W, scale, rows, cols, x, y, st);
  if (per <= 4) return launch_gemv_f32act_t<BITS, 4, 2>(W, scale, rows, cols, x, y, st);
  if (per <= 6) return launch_gemv_f32act_t<BITS, 6, 1>(W, scale, rows, cols, x, y, st);
  if (per <= 8) return launch_gemv_f32act_t<BITS, 8, 1>(W, scale, rows, cols, x, y, st);
  return hipErrorNotSupported;
}

hipError_t launch_gemv_f32act(int bits, const uint8_t *W, const float *scale, int64_t rows,
                              int64_t cols, const float *x, float *y, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 8: return launch_gemv_f32act_bits<8>(W, scale, rows, cols, x, y, st);
    case 4: return launch_gemv_f32act_bits<4>(W, scale, rows, cols, x, y, st);
    case 2: return launch_gemv_f32act_bits<2>(W, scale, rows, cols, x, y, st);
    default: return hipErrorInvalidValue;
  }
}

// Threads per row: one wave for rows of up to 256 chunks (4096 columns),
// four waves for longer rows, so a matrix of a few thousand rows still gives
// every SIMD several waves while short rows skip the cross-wave reduction.
template <int BITS, int TPR>
static hipError_t launch_fp8_tpr(const uint8_t *w8, const float *bscale, int64_t rows,
                                 int64_t cols, uint8_t *q, float *scale, hipStream_t st) {
  constexpr int RPW = 256 / TPR;
  const dim3 grid((unsigned)((rows + RPW - 1) / RPW)), block(256);
  const int64_t per = (cols / 16 + TPR - 1) / TPR;  // chunks per thread
  if (per <= 1)
    hipLaunchKernelGGL((k_quant_pack_fp8<BITS, TPR, 1>), grid, block, 0, st, w8, bscale, rows, cols, q, scale);
  else if (per <= 2)
    hipLaunchKernelGGL((k_quant_pack_fp8<BITS, TPR, 2>), grid, block, 0, st, w8, bscale, rows, cols, q, scale);
  else if (per <= 4)
    hipLaunchKernelGGL((k_quant_pack_fp8<BITS, TPR, 4>), grid, block, 0, st, w8, bscale, rows, cols, q, scale);
  else
    hipLaunchKernelGGL((k_quant_pack_fp8<BITS, TPR, 0>), grid, block, 0, st, w8, bscale, rows, cols, q, scale);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_fp8_bits(const uint8_t *w8, const float *bscale, int64_t rows,
                                  int64_t cols, uint8_t *q, float *scale, hipStream_t st) {
  const int64_t chunks = cols / 16;
  if (chunks > 256) return launch_fp8_tpr<BITS, 256>(w8, bscale, rows, cols, q, scale, st);
  return launch_fp8_tpr<BITS, 64>(w8, bscale, rows, cols, q, scale, st);
}

hipError_t launch_quant_pack_fp8(int bits, const uint8_t *w8, const float *bscale, int64_t rows,
                                 int64_t cols, uint8_t *q, float *scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 8: return launch_fp8_bits<8>(w8, bscale, rows, cols, q, scale, st);
    case 4: return launch_fp8_bits<4>(w8, bscale, rows, cols, q, scale, st);
    case 2: return launch_fp8_bits<2>(w8, bscale, rows, cols, q, scale, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_act_quant(int layout_bits, const float *x, int64_t T, int64_t n, int8_t *q,
                            float *d, hipStream_t st, KEvents ev, double *d64) {
  const int64_t blocks = T * (n / 32);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)((blocks + 255) / 256)), block(256);
  switch (layout_bits) {
    case 8: COLI_LAUNCH(ev, k_act_quant<8>, grid, block, 0, st, x, T, n, q, d, d64); break;
    case 4: COLI_LAUNCH(ev, k_act_quant<4>, grid, block, 0, st, x, T, n, q, d, d64); break;
    case 2: COLI_LAUNCH(ev, k_act_quant<2>, grid, block, 0, st, x, T, n, q, d, d64); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace coli
