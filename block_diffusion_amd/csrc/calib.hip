// Practical ceilings of the device, for the measurement of the kernels
// against both the nominal and a measured peak.
//
// stream_read_kernel: every thread reads 16-byte chunks, four at a time,
// grid-stride over the buffer; the XOR of everything read goes to one word
// per workgroup so that no load can be dropped.
//
// mfma_peak_kernel: a register-resident loop of v_mfma_f32_32x32x16_bf16.
// Each wave loads eight A and eight B operand fragments of one of 64
// operand sets once, then runs eight independent accumulator chains (more
// than the instruction's latency in issue slots), the operand pair of each
// chain rotating every step so that the multipliers see changing data as
// in a real GEMM (the chip's power limit depends on it).  Each thread
// writes the sum of its accumulators so that no product can be dropped.
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

__global__ __launch_bounds__(256) void mfma_peak_kernel(const bf16x8* __restrict__ src, int iters,
                                                       float* sink) {
  const int lane = threadIdx.x & 63;
  const int set = (blockIdx.x * 4 + (threadIdx.x >> 6)) % kMfmaPeakSets;
  const bf16x8* p = src + (size_t)set * 16 * 64 + lane;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = p[i * 64];
    b[i] = p[(8 + i) * 64];
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + r) & 7], b[(3 * c + r) & 7], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t mfma_peak_launch(const void* operands, int iters, float* sink, hipStream_t st) {
  mfma_peak_kernel<<<kMfmaPeakGrid, 256, 0, st>>>(static_cast<const bf16x8*>(operands), iters, sink);
  return hipGetLastError();
}

}  // namespace dbd
