// Tile building blocks shared by the Sol-Attn and Sol-Attn2 fused kernels:
// LDS staging of a 64-key V tile (transposed) and the online-softmax + PV update
// of one 64-key tile against a wave's 32 query rows.
//
// Register layout (v_mfma_f32_32x32x16_bf16, lane l, l32 = l % 32, kg = l / 32):
//   S^T accumulators s0 / s1 (keys 0..31 / 32..63): element idx holds key
//   8 (idx/4) + 4 kg + idx%4 of its half, query l32.
//   O^T accumulators o[mt]: element idx holds dim 32 mt + 8 (idx/4) + 4 kg + idx%4,
//   query l32.  The online-softmax state (running max in log2 units, partial
//   row sum over this lane's keys) is per lane; lanes l and l ^ 32 share a query.
#pragma once
#include "common.h"

namespace solattn {

constexpr int kVtStride = 136;   // bytes per V^T row (one dim, 64 keys): 128 + 8 pad

// Stage a 64-key V tile into LDS transposed (V^T[dim][key]).  Rows r >= valid
// are zero-filled.  128 threads; `stride` = elements between consecutive keys.
__device__ __forceinline__ void load_v_transposed(unsigned char* Vt, const uint16_t* vb, size_t stride,
                                                  int valid, int tid) {
  const int r4 = 4 * (tid & 15);                  // keys r4 .. r4 + 3
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c8 = (tid >> 4) + 8 * p;            // dims 8 c8 .. 8 c8 + 7
    uint4v R[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      R[rr] = uint4v{0u, 0u, 0u, 0u};
      if (r4 + rr < valid) R[rr] = *(const uint4v*)(vb + (size_t)(r4 + rr) * stride + c8 * 8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint2v lo, hi;                              // dims 2m (low halves) and 2m + 1 (high halves)
      lo[0] = (R[0][m] & 0xffffu) | (R[1][m] << 16);
      lo[1] = (R[2][m] & 0xffffu) | (R[3][m] << 16);
      hi[0] = (R[0][m] >> 16) | (R[1][m] & 0xffff0000u);
      hi[1] = (R[2][m] >> 16) | (R[3][m] & 0xffff0000u);
      *(uint2v*)(Vt + (8 * c8 + 2 * m) * kVtStride + r4 * 2) = lo;
      *(uint2v*)(Vt + (8 * c8 + 2 * m + 1) * kVtStride + r4 * 2) = hi;
    }
  }
}

// Online softmax over one tile of logits (log2 units, masked keys = -inf) and
// O^T += V^T P^T.  P is rounded to bf16 for the MFMA; the row sum uses fp32 P.
__device__ __forceinline__ void softmax_pv(floatx16& s0, floatx16& s1, const unsigned char* Vt,
                                           floatx16 (&o)[4], float& m_run, float& l_run, int l32, int kg) {
  float mx = kNegInf;
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) mx = fmaxf(mx, fmaxf(s0[idx], s1[idx]));
  mx = max_with_partner(mx);
  const float m_new = fmaxf(m_run, mx);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  float psum = 0.f;
  bf16x8 pa[4];
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) {
    const float p0 = __builtin_amdgcn_exp2f(s0[idx] - m_use);
    const float p1 = __builtin_amdgcn_exp2f(s1[idx] - m_use);
    psum += p0 + p1;
    // k-step st covers keys 16 st .. 16 st + 15: tile st / 2, elements 8 (st % 2) .. + 7
    pa[(idx >> 3)][idx & 7] = (__bf16)p0;
    pa[2 + (idx >> 3)][idx & 7] = (__bf16)p1;
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) o[mt][idx] *= alpha;
  // logical k position (kg, e) of k-step st is key 16 st + 8 (e/4) + 4 kg + e%4 on both operands
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const unsigned char* vrow = Vt + (32 * mt + l32) * kVtStride + kg * 8;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint2v lo = *(const uint2v*)(vrow + st * 32);
      const uint2v hi = *(const uint2v*)(vrow + st * 32 + 16);
      const uint4v av = {lo[0], lo[1], hi[0], hi[1]};
      o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pa[st], o[mt], 0, 0, 0);
    }
  }
}

// fp32 routing dot products for one chunk of 64 pooled keys: s_ij = Q-bar_i . K-bar_j / sqrt(d)
// (Sol-Attn paper §3.2, Eq. (6)); wave w sums dims 64 w .. 64 w + 63, partials meet in LDS.
// Returns this lane's proxy score for key block j = 64 c + lane (after the barrier).
__device__ __forceinline__ float routing_scores(const float4* kt, int nbp, int c, const float* qb_s,
                                                float (*part)[64], int w, int lane) {
  const int j = c * 64 + lane;
  float acc = 0.f;
#pragma unroll 4
  for (int d4 = 16 * w; d4 < 16 * w + 16; ++d4) {
    const float4 kk = kt[(size_t)d4 * nbp + j];
    acc += qb_s[4 * d4] * kk.x + qb_s[4 * d4 + 1] * kk.y + qb_s[4 * d4 + 2] * kk.z + qb_s[4 * d4 + 3] * kk.w;
  }
  part[w][lane] = acc;
  __syncthreads();
  return (part[0][lane] + part[1][lane]) * 0.08838834764831845f;
}

}  // namespace solattn
