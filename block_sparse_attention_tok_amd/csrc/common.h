// Shared device definitions for the gfx950 Sol-Attn kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));
typedef unsigned int uint2v __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;     // KV / query block size (Sol-Attn paper §4.1: fixed 64x64 physical blocks)
constexpr int kDim = 128;      // head dimension fixed by the README's tensor contract
constexpr int kAnchor = 32;    // Sol-Attn2 query anchor size (draft, Method)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (gfx950 lowers this to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Value of lane (l ^ 32) combined with this lane's via v_permlane32_swap.
__device__ __forceinline__ float max_with_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Map a hardware workgroup id to a logical work item so that each of the 8
// XCDs (which receive workgroups round-robin) walks a contiguous range of the
// logical order; keeps a head's pooled keys and nearby KV blocks in one L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int nx = 8;
  int per = total / nx, rem = total % nx;
  int x = wg % nx, idx = wg / nx;
  return x * per + (x < rem ? x : rem) + idx;
}

}  // namespace solattn
