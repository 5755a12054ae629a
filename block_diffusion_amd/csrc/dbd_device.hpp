// Device-side helpers shared by the gfx950 kernels of libdbd: vector types,
// 16-byte loads, bf16 conversion and wave-level shuffles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// 16-byte global load (8 bf16) reinterpreted as an MFMA operand.
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ld_u32x4(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// two floats -> a bf16 pair (lo in bits 0-15), each rounded to nearest
// even as f2bf: one v_cvt_pk_bf16_f32 instead of two conversions and a pack
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// 2^x via the hardware exponential (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) {
  return __shfl_xor(v, m, kWave);
}
__device__ __forceinline__ int shfl_xor_i(int v, int m) {
  return __shfl_xor(v, m, kWave);
}

// Reductions over the lane pairs (l, l^16) and (l, l^32) with the gfx950
// permlane swaps (VALU; no LDS round trip as ds_bpermute takes).  Swapping
// a register with itself, v_permlane16_swap returns, in each lane, the
// values of its own and its xor-16 partner in its two results (16-lane
// groups 0,1 / 2,3 exchanged), and v_permlane32_swap those of it and its
// xor-32 partner; either order, so max and sum are exact.
// The maximum is one v_max_f32: fmaxf would first quiet each swapped value
// (a v_max of the value with itself, two per call), since the compiler
// cannot tell that a lane exchange leaves the bits of a quiet NaN as they
// were.  v_max_f32 returns the other operand for a quiet NaN, as fmaxf does.
__device__ __forceinline__ float vmax_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Compiler-level ordering of LDS traffic among the lanes of one wave.  A
// wave's LDS instructions execute in issue order, so a write by one lane is
// seen by a later read of another lane of the same wave once the compiler
// keeps the order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace dbd
