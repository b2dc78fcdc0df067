// stream.hip -- a plain streaming read of a device buffer: the practical
// HBM ceiling for a kernel that reads the same bytes as a decode step with
// no routing and no dependencies, measured on the same GPU.
#include <algorithm>

#include "kernels.hpp"

namespace coli {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane

// Workgroup b reads 16-byte pieces b*256*U + ..., grid-strided, all U loads
// of a round issued before any is used; the xor of everything read is kept
// per workgroup so the loads are not dead.
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const uint4 *__restrict__ p,
                                                                size_t n16,
                                                                uint32_t *__restrict__ out) {
  uint32_t acc = 0;
  const size_t step = (size_t)gridDim.x * kStreamThreads * kStreamUnroll;
  for (size_t base = (size_t)blockIdx.x * kStreamThreads * kStreamUnroll + threadIdx.x; base < n16;
       base += step) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads;
      v[u] = i < n16 ? ld_nt(p + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  acc = (uint32_t)__builtin_amdgcn_readfirstlane((int)acc) ^ acc;  // cheap, keeps acc live
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, int *grid_out,
                              hipStream_t st, KEvents ev) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  const size_t n16 = bytes / 16;
  const size_t per_wg = (size_t)kStreamThreads * kStreamUnroll;
  const int grid = (int)std::max<size_t>(1, std::min<size_t>((size_t)n_cu * 8, (n16 + per_wg - 1) / per_wg));
  if (grid_out) *grid_out = grid;
  COLI_LAUNCH(ev, k_stream_read, dim3(grid), dim3(kStreamThreads), 0, st,
              static_cast<const uint4 *>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace coli
