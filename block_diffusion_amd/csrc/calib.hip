// Practical ceilings of the device, for the measurement of the kernels
// against both the nominal and a measured peak.
//
// stream_read_kernel: the fastest plain read found on the device.  Each
// workgroup reads whole contiguous 32 KB chunks (eight 16-byte non-temporal
// loads in flight per thread, consecutive threads on consecutive 16 bytes),
// chunks dealt round robin; a tail shorter than a chunk is read grid-stride.
// The XOR of everything read goes to one word per workgroup so that no load
// can be dropped.  Non-temporal loads stream past the caches: on MI355X they
// read at 7.0 TB/s where plain loads of the same shape read at 6.3 TB/s.
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

constexpr int kReadThreads = 256, kReadInflight = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                   uint32_t* sink) {
  constexpr size_t per = (size_t)kReadThreads * kReadInflight;   // 16-byte units per chunk
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t nfull = n16 / per;
  for (size_t c = blockIdx.x; c < nfull; c += gridDim.x) {
    const u32x4* q = p + c * per + threadIdx.x;
    u32x4 v[kReadInflight];
#pragma unroll
    for (int k = 0; k < kReadInflight; ++k) v[k] = __builtin_nontemporal_load(q + k * kReadThreads);
#pragma unroll
    for (int k = 0; k < kReadInflight; ++k) acc ^= v[k];
  }
  for (size_t i = nfull * per + (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kReadThreads)
    acc ^= p[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  __shared__ uint32_t s_x[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0u;
    for (int w = 0; w < kReadThreads / 64; ++w) y ^= s_x[w];
    sink[blockIdx.x] = y;
  }
}

hipError_t stream_read_launch(const void* data, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t st) {
  stream_read_kernel<<<grid, kReadThreads, 0, st>>>(static_cast<const u32x4*>(data), bytes / 16, sink);
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
