// hca_device.h -- small device helpers for the gfx950 HCA kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace hca {

typedef unsigned short bf16raw;  // bfloat16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wave issue priority around a block of matrix instructions: while it is
// raised, the SIMD's arbiter picks this wave ahead of waves that are issuing
// copies, softmax or address arithmetic, so the matrix unit stays fed while
// the other waves of the CU do that work.  It orders issue only.
__device__ __forceinline__ void mfma_phase_begin() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_phase_end() { __builtin_amdgcn_s_setprio(0); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint4 lds_load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ bf16x8 pack8(const float *x) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)x[t];
  return r;
}

__device__ __forceinline__ float bf2f(bf16raw v) {
  return __uint_as_float(((unsigned)v) << 16);
}

__device__ __forceinline__ bf16raw f2bf(float f) {
  return __builtin_bit_cast(bf16raw, (__bf16)f);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform read of a table the kernel never writes, through the scalar
// cache (counted by lgkmcnt, so waiting for it does not also wait for the
// vector-memory tile loads in flight).
__device__ __forceinline__ uint32_t uniform_load(const uint32_t *p, int i) {
  return ((const __attribute__((address_space(4))) uint32_t *)p)[i];
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

// Launch-order remap: workgroups are handed to the 8 XCDs round-robin, so
// consecutive block ids land on different L2s.  This bijection on [0, n)
// gives each XCD runs of G consecutive list entries (neighbouring query tiles
// share key tiles), while the list order (heaviest first) is kept across runs.
__device__ __forceinline__ int xcd_remap(int x, int n, int G = 4) {
  constexpr int X = 8;
  const int full = n / (X * G) * (X * G);
  if (x >= full) return x;
  const int r = x / X;
  return (r / G) * (X * G) + (x % X) * G + (r % G);
}

}  // namespace hca
