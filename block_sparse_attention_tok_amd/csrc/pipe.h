// Tile pipeline pieces shared by the fused Sol-Attn and Sol-Attn2 kernels on gfx950:
// swizzled 64-row tiles moved HBM -> LDS by buffer DMA, and the PV product read
// back through ds_read_b64_tr_b16.
#pragma once
#include "common.h"

namespace solattn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool B> struct BoolTag { static constexpr bool value = B; };

// 16-byte slot swizzles of the 64 x 256-byte K and V tiles (row r, logical chunk
// lc lives in physical slot lc ^ swz(r)), chosen conflict-free for both 32- and
// 64-bank LDS: K spreads 16 consecutive rows of a b128 read over distinct slots;
// V spreads the 4 rows x 4 chunks touched by 32 lanes of a transposed read.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return (0xEA40 >> (4 * (r & 3))) & 15; }   // 0, 4, 10, 14

// DMA of a 64 x 128 bf16 tile into LDS (16 KB, two waves x 8 instructions)
// through a buffer resource.  Wave w, instruction n fills the 1 KB segment
// 8 w + n, i.e. rows r = 32 w + 4 n + lane / 16; lane's 16 bytes go to slot
// lane % 16 of row r, which holds logical chunk (lane % 16) ^ swz(r).  The
// per-lane byte offset depends on n only through swz_k(r) = 4 (n % 4) + lane / 16
// (four K variants, one V variant).  The whole offset (tile, 4 n rows, lane) is
// in the VGPR operand, the one the buffer range check covers, so rows past the
// end of the tensor read as zeros.
struct DmaOffsets {
  uint32_t k[4], v;
};

__device__ __forceinline__ DmaOffsets dma_offsets(uint32_t row_bytes, int w, int lane) {
  const uint32_t row = 32 * w + (lane >> 4);
  DmaOffsets d;
#pragma unroll
  for (int n = 0; n < 4; ++n) d.k[n] = row * row_bytes + (((lane & 15) ^ swz_k(row + 4 * n)) << 4);
  d.v = row * row_bytes + (((lane & 15) ^ swz_v(row)) << 4);
  return d;
}

template <bool kIsV>
__device__ __forceinline__ void dma_tile(unsigned char* lds, __amdgpu_buffer_rsrc_t rsrc, uint32_t tile_off,
                                         uint32_t row_bytes, const DmaOffsets& off, int w) {
#pragma unroll
  for (int n = 0; n < 8; ++n)
    dma16_buf(rsrc, (kIsV ? off.v : off.k[n & 3]) + tile_off + (uint32_t)n * 4 * row_bytes, 0, lds + (w * 8 + n) * 1024);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  return (const void*)uniform64((uint64_t)p);
}

// Routing numerator Q-bar_i . K-bar_j for key block j (the proxy score of Sol-Attn paper
// §3.1 Eq. (4) before its 1/sqrt(d) scale): 128 fp32 FMAs over the dims in ascending order,
// from Q-bar_i as 32 float4 (in LDS) and the head's 4-dim-interleaved fp32 key-block means
// kt = [32][nbp] float4.  Every kernel that routes a pair uses this one FMA sequence, so
// kernels that need the same pair's decision take it bit for bit alike.
__device__ __forceinline__ float proxy_dot(const float4* qb, const float4* kt, int nbp, int j) {
  float acc = 0.f;
#pragma unroll 8
  for (int g = 0; g < 32; ++g) {
    const float4 kv = kt[(size_t)g * nbp + j];
    const float4 qv = qb[g];
    acc = __builtin_fmaf(qv.x, kv.x, acc);
    acc = __builtin_fmaf(qv.y, kv.y, acc);
    acc = __builtin_fmaf(qv.z, kv.z, acc);
    acc = __builtin_fmaf(qv.w, kv.w, acc);
  }
  return acc;
}

// The exact-set word of 64-block chunk c (c < nbp / 64, so the chunk holds at least one
// block below nb) from the ballot of s_ij > tau_i: the sink's blocks [sink_b0, sink_b1]
// forced exact, the padding blocks cleared.
__device__ __forceinline__ uint64_t exact_word(uint64_t ballot, int c, int nb, int sink_b0, int sink_b1) {
  const int nvalid = nb - 64 * c;
  const uint64_t validm = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
  const int s0 = max(sink_b0, 64 * c), s1 = min(sink_b1, 64 * c + 63);
  if (s0 <= s1) ballot |= (~0ull >> (63 - (s1 - s0))) << (s0 - 64 * c);
  return ballot & validm;
}

// Sum of the 8 bf16 values of a packed P fragment into acc (v_dot2c_f32_bf16 with ones).
// The pairs are taken with shufflevector: extracting them from a bit_cast to
// 4 x uint32 lowers, with the ROCm 7.2 compiler, to four reads of the first pair.
__device__ __forceinline__ float add_bf16x8(bf16x8 x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
  return acc;
}

// V^T A-operand offsets of the transposed read (v_mfma_f32_32x32x16_bf16): lane group
// G = lane / 16, i' = lane % 16 addresses key 4 kg + i'/4 (+ 16 st + 8 half; the
// swizzle depends on key & 3 only), dims 32 mt + 16 (G % 2) + 4 (i' % 4) = logical
// chunk 4 mt + 2 (G % 2) + (i' % 4) / 2.
__device__ __forceinline__ void v_operand_offsets(int lane, int (&voff)[4]) {
  const int ip = lane & 15, gm = (lane >> 4) & 1, kg = lane >> 5;
  const int key = 4 * kg + (ip >> 2);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int lc = 4 * mt + 2 * gm + ((ip & 3) >> 1);
    voff[mt] = key * 256 + 16 * (lc ^ swz_v(key)) + (ip & 1) * 8;
  }
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmem = 0x010, kSchedDsRead = 0x100;
// The V^T operand of each PV product is read this many products ahead, so that the LDS
// latency overlaps the products before it (the scheduler otherwise places each read just
// before its MFMA under the register limit of two waves per SIMD).
constexpr int kPvAhead = 4;

// O^T += V^T P^T for one 64-key tile: pa[st] holds keys 16 st + 8 (e / 4) + 4 kg + e % 4
// (e = 0..7) of the lane's query column, the same key order as the transposed V read.
__device__ __forceinline__ void pv_tile(floatx16 (&o)[4], const unsigned char* Vl, const int (&voff)[4],
                                        const bf16x8 (&pa)[4]) {
  uint4v av[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mt = i >> 2, st = i & 3;
    const int vo = voff[mt] + st * 16 * 256;
    const uint2v lo = lds_read_tr16(Vl + vo);
    const uint2v hi = lds_read_tr16(Vl + vo + 8 * 256);
    av[i] = uint4v{lo[0], lo[1], hi[0], hi[1]};
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mt = i >> 2, st = i & 3;
    o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]), pa[st], o[mt], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPvAhead, 0);
#pragma unroll
  for (int i = 0; i < 16 - kPvAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPvAhead, 0);
}

// DMA instructions placed after each product when a tile's DMA is spread over a product chain.
constexpr int kDmaPerProduct = 1;

// pv_tile with the 8 DMA instructions that `dma` issues (the next tile's K) spread over the
// first products, kDmaPerProduct after each, so the wave reaches its first MFMA without first
// waiting for the issue of the whole DMA burst.
template <class Dma>
__device__ __forceinline__ void pv_tile_dma(floatx16 (&o)[4], const unsigned char* Vl, const int (&voff)[4],
                                            const bf16x8 (&pa)[4], Dma&& dma) {
  uint4v av[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mt = i >> 2, st = i & 3;
    const int vo = voff[mt] + st * 16 * 256;
    const uint2v lo = lds_read_tr16(Vl + vo);
    const uint2v hi = lds_read_tr16(Vl + vo + 8 * 256);
    av[i] = uint4v{lo[0], lo[1], hi[0], hi[1]};
  }
  dma();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mt = i >> 2, st = i & 3;
    o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]), pa[st], o[mt], 0, 0, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kPvAhead, 0);
#pragma unroll
  for (int i = 0; i < 16 - kPvAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    if (i < 8 / kDmaPerProduct) __builtin_amdgcn_sched_group_barrier(kSchedVmem, kDmaPerProduct, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPvAhead, 0);
}

}  // namespace solattn
