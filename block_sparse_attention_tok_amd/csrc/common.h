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

// Counting sort by descending count for one workgroup of 256 threads: qc[0 .. nb) in LDS holds
// counts in [0, nb]; out[rank] receives each index, larger counts first (equal counts in any
// order: the orders built with it only schedule work).  slot (nb + 1 ints) and part (256 ints)
// are LDS scratch.  A histogram of the counts, its exclusive scan from the largest count down
// (each thread scans a contiguous run of bins, one thread scans the 256 run totals), then one
// slot per index taken with an LDS atomic.
__device__ __forceinline__ void sort_desc_counts(const unsigned short* qc, int* slot, int* part, int nb, int* out) {
  const int tid = threadIdx.x;
  for (int v = tid; v <= nb; v += 256) slot[v] = 0;
  __syncthreads();
  for (int i = tid; i < nb; i += 256) atomicAdd(&slot[qc[i]], 1);
  __syncthreads();
  const int per = (nb + 1 + 255) / 256;
  const int u0 = tid * per, u1 = min(nb + 1, (tid + 1) * per);
  int local = 0;
  for (int u = u0; u < u1; ++u) local += slot[nb - u];
  part[tid] = local;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int t = 0; t < 256; ++t) {
      const int x = part[t];
      part[t] = acc;
      acc += x;
    }
  }
  __syncthreads();
  int acc = part[tid];
  for (int u = u0; u < u1; ++u) {
    const int x = slot[nb - u];
    slot[nb - u] = acc;
    acc += x;
  }
  __syncthreads();
  for (int i = tid; i < nb; i += 256) out[atomicAdd(&slot[qc[i]], 1)] = i;
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

namespace solattn {

// s_waitcnt immediates for the gfx9 encoding (vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4, lgkmcnt in 11:8); the counters not named are left at max.
constexpr int kWaitVm0 = 0x0F70;      // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;    // lgkmcnt(0)

// Workgroup barrier for LDS hand-offs that must not wait for in-flight global
// loads (unlike __syncthreads, whose fence drains vmcnt): completes this
// wave's LDS reads, then s_barrier; the signal fences keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void wait_vm0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): loads past the end return zeros
// instead of faulting (gfx9 word 3: default data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from rsrc + soffset + voffset to
// lds_base + 16 lane (lds_base wave-uniform).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset,
                                          unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_base, 16, voffset, soffset, 0, 0);
}

// buffer_load_dword ... lds: 4 bytes per lane from rsrc + soffset + voffset to
// lds_base + 4 lane (lds_base wave-uniform); lanes outside the buffer store zeros.
__device__ __forceinline__ void dma4_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset,
                                         unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_base, 4, voffset, soffset, 0, 0);
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4)
// of the 8-byte rows addressed by lanes 4 e + i / 4, e = 0..3.
__device__ __forceinline__ uint2v lds_read_tr16(const unsigned char* p) {
  shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(__attribute__((address_space(3))) unsigned char*)p);
  return __builtin_bit_cast(uint2v, r);
}

}  // namespace solattn
