// Streaming-read floor: a kernel that only reads a buffer from HBM, with
// 16-byte loads, U of them in flight per thread before any is consumed. It
// frames the decode kernels' bandwidth: at a given byte count, no kernel that
// must read those bytes can be faster than the fastest plain read of them
// (which includes the fixed cost of a launch). The loaded words are folded
// into one value per thread that is written only if it equals a value the
// caller passes (a value the data does not produce), so the loads cannot be
// dropped and the kernel writes nothing in practice.
#include "qlinear_kernels.hpp"

namespace qlinear {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_floor_kernel(const u32x4* __restrict__ buf, int64_t n16, uint32_t key,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = buf[i < n16 ? i : n16 - 1];   // clamped: a repeated read of the last piece
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == key) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_floor(const void* buf, size_t bytes, int loads, int grid, uint32_t key, uint32_t* sink,
                             hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const u32x4* b = reinterpret_cast<const u32x4*>(buf);
  switch (loads) {
    case 4: hipLaunchKernelGGL(read_floor_kernel<4>, dim3(grid), dim3(256), 0, stream, b, n16, key, sink); break;
    case 8: hipLaunchKernelGGL(read_floor_kernel<8>, dim3(grid), dim3(256), 0, stream, b, n16, key, sink); break;
    default: hipLaunchKernelGGL(read_floor_kernel<16>, dim3(grid), dim3(256), 0, stream, b, n16, key, sink); break;
  }
  return hipGetLastError();
}

}  // namespace qlinear
