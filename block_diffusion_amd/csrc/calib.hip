// Practical streaming-read ceiling of the device, for the measurement of the
// memory-bound kernels against both the nominal and a measured peak.
// Every thread reads 16-byte chunks, four at a time, grid-stride over the
// buffer; the XOR of everything read goes to one word per workgroup so
// that no load can be dropped.
#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

__global__ __launch_bounds__(512) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  __shared__ uint32_t s_x[8];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0u;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) y ^= s_x[w];
    sink[blockIdx.x] = y;
  }
}

hipError_t stream_read_launch(const void* data, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t st) {
  stream_read_kernel<<<grid, 512, 0, st>>>(static_cast<const u32x4*>(data), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace dbd
