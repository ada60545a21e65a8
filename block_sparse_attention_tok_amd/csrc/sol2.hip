// Sol-Attn2 forward for gfx950: FP8 Q/K, routing on dequantized block means,
// complementary tail with 32-token query anchors and first-order mass
// correction, one shared denominator.
//
// "Sol-Attn2: Sparse Attention with Complementary Approximation" (draft):
//   Method, "Routing and complementary approximation", Eqs. (1)-(3);
//   output table ("How the outputs are combined", Sol-Attn2 row);
//   "FP8 quantization and ExpCast" (per-64-token-block E4M3 scales for Q and K).
// Readings where the draft is open (documented with the oracle): the
// mean-query direction is the per-(batch, head) mean of the dequantized
// queries; a key block splits at its mean projection onto that direction,
// ties joining the upper group; an empty block uses scale 1.  V is bf16 in the
// default path; the FP8-PV path ("FP8 quantization and ExpCast") stores V once
// per head as E4M3 with one scale and feeds the exact blocks' probabilities as
// ExpCast bytes c(u) = clip(RNE(8 u + 55.65), 0, 120) taken against the running
// per-row pivot, so the same decoded weights enter the PV product and the
// denominator.
#include "common.h"
#include "kernels.h"
#include "pipe.h"

namespace solattn {

constexpr float kScale2 = 0.08838834764831845f;       // 1/sqrt(128)
constexpr int kK8Stride = 144;                          // bytes per fp8 K row in LDS: 128 + 16 pad

// gfx950 converts with OCP E4M3FN semantics, round-to-nearest-even.
__device__ __forceinline__ uint32_t fp8x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

// x / s for an E4M3 scale s = RN(max|X| / 448), from one reciprocal r = RN(1 / s): q = x r,
// then Markstein's correction q + (x - q s) r, both steps fused multiply-adds (P. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990).  For s >= 2^-60, every bf16 x with |x| <= 448 s and either quotient at
// least 2^-12 it gives the IEEE quotient bit for bit (tests/host/div_by_scale.c checks every
// bf16 max and every x); below 2^-12 both quotients round to the E4M3 code 0.  Smaller scales
// take the IEEE division.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q = x * r;
  return fmaf(fmaf(-q, s, x), r, q);
}
constexpr float kMinReciprocalScale = 0x1p-60f;

// ---------------------------------------------------------------------------
// Stage 1a: quantization (draft "FP8 quantization": s = max|X| / 448, X8 = E4M3(X / s))
// and block / anchor means of the dequantized values.  One workgroup per
// (64-token block j < nbp, batch * head); thread (c = tid % 16, r = tid / 16)
// owns dims 8c..8c+7 of tokens r, r + 16, r + 32, r + 48.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_summary_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int N, int H, int nb, int nbp, int tp,
    uint8_t* __restrict__ q8, uint8_t* __restrict__ k8, float* __restrict__ qscale, float* __restrict__ kscale,
    float* __restrict__ qbar, float* __restrict__ kbar_t, float* __restrict__ qanc) {
  __shared__ float red[16][3][kDim];
  __shared__ float wmax[2][4];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / H, h = bh % H;
  const int c = tid & 15, r = tid >> 4;
  const int t0 = j * kBlock;
  const int n = j < nb ? min(kBlock, N - t0) : 0;
  const size_t rs = (size_t)H * kDim;
  const size_t src0 = ((size_t)b * N + t0) * rs + (size_t)h * kDim + c * 8;

  float xq[4][8], xk[4][8];
  float aq = 0.f, ak = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int t = r + 16 * p;
    uint4v a = {0u, 0u, 0u, 0u}, bb = {0u, 0u, 0u, 0u};
    if (t < n) {
      a = *(const uint4v*)(q + src0 + (size_t)t * rs);
      bb = *(const uint4v*)(k + src0 + (size_t)t * rs);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      xq[p][2 * m] = bf16_lo(a[m]);  xq[p][2 * m + 1] = bf16_hi(a[m]);
      xk[p][2 * m] = bf16_lo(bb[m]); xk[p][2 * m + 1] = bf16_hi(bb[m]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) { aq = fmaxf(aq, fabsf(xq[p][e])); ak = fmaxf(ak, fabsf(xk[p][e])); }
  }
  aq = wave_max(aq);
  ak = wave_max(ak);
  if ((tid & 63) == 0) { wmax[0][tid >> 6] = aq; wmax[1][tid >> 6] = ak; }
  __syncthreads();
  aq = fmaxf(fmaxf(wmax[0][0], wmax[0][1]), fmaxf(wmax[0][2], wmax[0][3]));
  ak = fmaxf(fmaxf(wmax[1][0], wmax[1][1]), fmaxf(wmax[1][2], wmax[1][3]));
  const float sq = aq > 0.f ? __fdiv_rn(aq, 448.0f) : 1.0f;
  const float sk = ak > 0.f ? __fdiv_rn(ak, 448.0f) : 1.0f;
  const float rq = __fdiv_rn(1.0f, sq), rk = __fdiv_rn(1.0f, sk);

  // E4M3 codes; rows t >= n hold zeros and encode to code 0
  uint2v cq[4], ck[4];
  auto encode = [&](auto recip_tag) {
    constexpr bool kRecip = decltype(recip_tag)::value;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float yq[4], yk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = xq[p][4 * m + e], x1 = xk[p][4 * m + e];
          yq[e] = fminf(fmaxf(kRecip ? div_by_scale(x0, sq, rq) : __fdiv_rn(x0, sq), -448.f), 448.f);
          yk[e] = fminf(fmaxf(kRecip ? div_by_scale(x1, sk, rk) : __fdiv_rn(x1, sk), -448.f), 448.f);
        }
        cq[p][m] = fp8x2(yq[0], yq[1]) | (fp8x2(yq[2], yq[3]) << 16);
        ck[p][m] = fp8x2(yk[0], yk[1]) | (fp8x2(yk[2], yk[3]) << 16);
      }
    }
  };
  if (sq >= kMinReciprocalScale && sk >= kMinReciprocalScale) encode(BoolTag<true>{});   // uniform branch
  else encode(BoolTag<false>{});

  float sumq0[8], sumq1[8], sumk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sumq0[e] = sumq1[e] = sumk[e] = 0.f;
  const size_t dst0 = ((size_t)bh * tp + t0) * kDim + c * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int t = r + 16 * p;
    // sums of the decoded codes (exact in fp32: multiples of 2^-9 below 2^15)
    float dq[8], dk[8];
    fp8x4_to_f32(cq[p][0], dq); fp8x4_to_f32(cq[p][1], dq + 4);
    fp8x4_to_f32(ck[p][0], dk); fp8x4_to_f32(ck[p][1], dk + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (p < 2) sumq0[e] += dq[e]; else sumq1[e] += dq[e];
      sumk[e] += dk[e];
    }
    if (j < nb) {   // codes of rows t >= n inside the last block are written as zeros
      *(uint2v*)(q8 + dst0 + (size_t)t * kDim) = cq[p];
      *(uint2v*)(k8 + dst0 + (size_t)t * kDim) = ck[p];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[r][0][c * 8 + e] = sumq0[e];
    red[r][1][c * 8 + e] = sumq1[e];
    red[r][2][c * 8 + e] = sumk[e];
  }
  __syncthreads();
  if (tid < kDim) {
    float a0 = 0.f, a1 = 0.f, kk = 0.f;
    for (int rr = 0; rr < 16; ++rr) { a0 += red[rr][0][tid]; a1 += red[rr][1][tid]; kk += red[rr][2][tid]; }
    const int n0 = min(n, 32), n1 = max(n - 32, 0);
    const size_t row = (size_t)bh * nbp + j;
    qbar[row * kDim + tid] = n > 0 ? sq * (a0 + a1) / (float)n : 0.f;
    qanc[(row * 2) * kDim + tid] = n0 > 0 ? sq * a0 / (float)n0 : 0.f;
    qanc[(row * 2 + 1) * kDim + tid] = n1 > 0 ? sq * a1 / (float)n1 : 0.f;
    kbar_t[(((size_t)bh * 32 + (tid >> 2)) * nbp + j) * 4 + (tid & 3)] = n > 0 ? sk * kk / (float)n : 0.f;
    if (tid == 0) { qscale[row] = sq; kscale[row] = sk; }
  }
}

hipError_t launch_quant_summary(const uint16_t* q, const uint16_t* k, const uint16_t*, Shape s,
                                const Workspace& ws, hipStream_t stream) {
  hipLaunchKernelGGL(quant_summary_kernel, dim3(ws.nbp, s.B * s.H), dim3(256), 0, stream, q, k, s.N, s.H, ws.nb,
                     ws.nbp, ws.nbp * kBlock, ws.q8, ws.k8, ws.qscale, ws.kscale, ws.qbar, ws.kbar_t, ws.qanc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 1c: mean-query direction q-hat = mean of the dequantized queries of the (b, h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void qhat_kernel(const float* __restrict__ qbar, int N, int nb, int nbp,
                                                    float* __restrict__ qhat) {
  // thread (d, slice): dim d of the blocks slice, slice + 8, ...; the 8 slices meet in LDS
  __shared__ float part[8][kDim];
  const int bh = blockIdx.x, d = threadIdx.x & (kDim - 1), slice = threadIdx.x >> 7;
  float acc = 0.f;
  int i = slice;
  for (; i + 24 < nb - 1; i += 32) {                     // four loads in flight (before the last block)
    const float x0 = qbar[((size_t)bh * nbp + i) * kDim + d];
    const float x1 = qbar[((size_t)bh * nbp + i + 8) * kDim + d];
    const float x2 = qbar[((size_t)bh * nbp + i + 16) * kDim + d];
    const float x3 = qbar[((size_t)bh * nbp + i + 24) * kDim + d];
    acc += 64.f * ((x0 + x1) + (x2 + x3));               // full blocks
  }
  for (; i < nb; i += 8) acc += (float)min(kBlock, N - i * kBlock) * qbar[((size_t)bh * nbp + i) * kDim + d];
  part[slice][d] = acc;
  __syncthreads();
  if (slice == 0) {
    float t = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) t += part[s8][d];
    qhat[(size_t)bh * kDim + d] = t / (float)N;
  }
}

hipError_t launch_qhat(Shape s, const Workspace& ws, hipStream_t stream) {
  hipLaunchKernelGGL(qhat_kernel, dim3(s.B * s.H), dim3(1024), 0, stream, ws.qbar, s.N, ws.nb, ws.nbp, ws.qhat);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 1d: two content groups per key block (draft, Method): projection of each
// dequantized key onto q-hat, split at the block's mean projection (ties to G_hi);
// n_g, mean key k-bar_g (dequantized) and mean value v-bar_g.  One wave per
// (b, h, block j < nbp); padding blocks get empty groups.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void groups_kernel(const uint16_t* __restrict__ v, const uint8_t* __restrict__ k8,
                                                     const float* __restrict__ kscale, const float* __restrict__ qhat,
                                                     int N, int H, int nb, int nbp, int tp, int total,
                                                     uint16_t* __restrict__ gk, uint16_t* __restrict__ gv,
                                                     float* __restrict__ glogn, uint64_t* __restrict__ ghi,
                                                     float* __restrict__ vbmax) {
  __shared__ float qh_s[4][kDim];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + wv;
  if (item >= total) return;                            // whole wave exits; no block barrier below
  const int j = item % nbp, bh = item / nbp;
  const int b = bh / H, h = bh % H;
  const size_t row = (size_t)bh * nbp + j;
  qh_s[wv][lane] = qhat[(size_t)bh * kDim + lane];
  qh_s[wv][lane + 64] = qhat[(size_t)bh * kDim + lane + 64];
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const int t0 = j * kBlock;
  const int n = j < nb ? min(kBlock, N - t0) : 0;
  const float sk = j < nb ? kscale[row] : 1.f;
  // projection of token `lane` (scale-free: sk > 0 is common to the block)
  float p = 0.f;
  if (lane < n) {
    const uint4v* kr = (const uint4v*)(k8 + ((size_t)bh * tp + t0 + lane) * kDim);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint4v w4 = kr[cc];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float f[4];
        fp8x4_to_f32(w4[m], f);
#pragma unroll
        for (int e = 0; e < 4; ++e) p += f[e] * qh_s[wv][16 * cc + 4 * m + e];
      }
    }
    p *= sk;
  }
  const float pbar = n > 0 ? wave_sum(lane < n ? p : 0.f) / (float)n : 0.f;
  const uint64_t hi = __ballot(lane < n && p >= pbar);
  // group sums: lane owns dims 2 lane, 2 lane + 1
  float kh[2] = {0.f, 0.f}, kl[2] = {0.f, 0.f}, vh[2] = {0.f, 0.f}, vl[2] = {0.f, 0.f};
  const size_t rs = (size_t)H * kDim;
  const uint16_t* vb = v + ((size_t)b * N + t0) * rs + (size_t)h * kDim + 2 * lane;
  const uint8_t* kb = k8 + ((size_t)bh * tp + t0) * kDim + 2 * lane;
  float vmax = 0.f;
  for (int u0 = 0; u0 < n; u0 += 16) {                    // 16 tokens' loads in flight together
    uint32_t vw[16], kw[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int u = u0 + e;
      vw[e] = u < n ? *(const uint32_t*)(vb + (size_t)u * rs) : 0u;
      kw[e] = u < n ? (uint32_t)*(const uint16_t*)(kb + (size_t)u * kDim) : 0u;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int u = u0 + e;
      if (u < n) {
        const auto kf = __builtin_amdgcn_cvt_pk_f32_fp8(kw[e], false);
        const float v0 = bf16_lo(vw[e]), v1 = bf16_hi(vw[e]);
        vmax = fmaxf(vmax, fmaxf(fabsf(v0), fabsf(v1)));
        if ((hi >> u) & 1) { kh[0] += kf[0]; kh[1] += kf[1]; vh[0] += v0; vh[1] += v1; }
        else               { kl[0] += kf[0]; kl[1] += kf[1]; vl[0] += v0; vl[1] += v1; }
      }
    }
  }
  const int nh = __popcll(hi), nl = n - nh;
  const float ih = nh > 0 ? 1.f / (float)nh : 0.f, il = nl > 0 ? 1.f / (float)nl : 0.f;
  uint32_t* gko = (uint32_t*)(gk + row * 2 * kDim);
  uint32_t* gvo = (uint32_t*)(gv + row * 2 * kDim);
  gko[lane] = pack_bf16x2(sk * kh[0] * ih, sk * kh[1] * ih);
  gko[64 + lane] = pack_bf16x2(sk * kl[0] * il, sk * kl[1] * il);
  gvo[lane] = pack_bf16x2(vh[0] * ih, vh[1] * ih);
  gvo[64 + lane] = pack_bf16x2(vl[0] * il, vl[1] * il);
  vmax = wave_max(vmax);
  if (lane == 0) {
    glogn[row * 2] = nh > 0 ? __logf((float)nh) : kNegInf;
    glogn[row * 2 + 1] = nl > 0 ? __logf((float)nl) : kNegInf;
    ghi[row] = hi;
    if (vbmax) vbmax[row] = vmax;
  }
}

hipError_t launch_groups(const uint16_t* v, Shape s, const Workspace& ws, hipStream_t stream) {
  const int total = s.B * s.H * ws.nbp;
  hipLaunchKernelGGL(groups_kernel, dim3((total + 3) / 4), dim3(256), 0, stream, v, ws.k8, ws.kscale, ws.qhat, s.N,
                     s.H, ws.nb, ws.nbp, ws.nbp * kBlock, total, ws.gk, ws.gv, ws.glogn, ws.ghi, ws.vbmax);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 1e (FP8 PV only): per-head V scale s_V = max |V| / 448 (draft "FP8
// quantization": V with one scale per head) and the E4M3 codes of V / s_V, written
// dim-major with each 64-token block in the FP8 PV operand order: token
// 32 h + 8 q + 4 g + r at position 32 g + 16 h + 4 q + r (g is the MFMA k-half a
// lane of the score tile holds; h, q, r index its accumulator registers).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vscale_kernel(const float* __restrict__ vbmax, int nbp,
                                                     float* __restrict__ vscale) {
  __shared__ float red[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  float m = 0.f;
  for (int j = tid; j < nbp; j += 256) m = fmaxf(m, vbmax[(size_t)bh * nbp + j]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    vscale[bh] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  }
}

__device__ __forceinline__ int pv_token(int p) {         // inverse of the operand-order permutation
  const int g = p >> 5, e = p & 31;
  return 32 * (e >> 4) + 8 * ((e >> 2) & 3) + 4 * g + (e & 3);
}

__global__ __launch_bounds__(256) void v8t_kernel(const uint16_t* __restrict__ v, const float* __restrict__ vscale,
                                                  int N, int H, int tp, uint8_t* __restrict__ v8t) {
  __shared__ uint16_t vs[64][kDim + 8];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / H, h = bh % H;
  const int t0 = j * kBlock, n = max(0, min(kBlock, N - t0));
  const size_t rs = (size_t)H * kDim;
  for (int e = tid; e < 64 * 16; e += 256) {
    const int r = e >> 4, c = e & 15;
    uint4v x = {0u, 0u, 0u, 0u};
    if (r < n) x = *(const uint4v*)(v + ((size_t)b * N + t0 + r) * rs + (size_t)h * kDim + 8 * c);
    *(uint4v*)(&vs[r][8 * c]) = x;
  }
  __syncthreads();
  const float s = vscale[bh];
  const float rinv = __fdiv_rn(1.0f, s);
  const int d = tid >> 1, p0 = 32 * (tid & 1);
  uint32_t w[8];
  auto encode = [&](auto recip_tag) {
    constexpr bool kRecip = decltype(recip_tag)::value;
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = bf16_bits_to_f32(vs[pv_token(p0 + 4 * q4 + e)][d]);
        y[e] = fminf(fmaxf(kRecip ? div_by_scale(x, s, rinv) : __fdiv_rn(x, s), -448.f), 448.f);
      }
      w[q4] = fp8x2(y[0], y[1]) | (fp8x2(y[2], y[3]) << 16);
    }
  };
  if (s >= kMinReciprocalScale) encode(BoolTag<true>{});   // uniform branch
  else encode(BoolTag<false>{});
  uint4v* dst = (uint4v*)(v8t + ((size_t)bh * kDim + d) * tp + (size_t)j * kBlock + p0);
  dst[0] = uint4v{w[0], w[1], w[2], w[3]};
  dst[1] = uint4v{w[4], w[5], w[6], w[7]};
}

hipError_t launch_vquant(const uint16_t* v, Shape s, const Workspace& ws, hipStream_t stream) {
  if (!ws.v8t || !ws.vbmax || !ws.vscale) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vscale_kernel, dim3(s.B * s.H), dim3(256), 0, stream, ws.vbmax, ws.nbp, ws.vscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v8t_kernel, dim3(ws.nbp, s.B * s.H), dim3(256), 0, stream, v, ws.vscale, s.N, s.H,
                     ws.nbp * kBlock, ws.v8t);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 2a: the complementary tail of every anchor (draft, Method, Eq. (1)).  One
// workgroup (two waves) per (b, h, 32 consecutive query blocks); wave w's lane column
// n = lane % 32 is anchor n of query blocks i0 + 16 w .. i0 + 16 w + 15 (query block
// i0 + 16 w + n / 2, half n % 2).  Tiles of 16 key blocks (32 groups) stream through
// LDS two tiles ahead, each row a group's bf16 mean key then mean value, with ln n_g of
// the tile's groups; the routing words of the workgroup's query blocks are decided on
// chip first (below):
//   scores   l_ga = ln n_g + q-bar_a . k-bar_g / sqrt(d) on v_mfma_f32_32x32x16_bf16
//            (A = the group rows, B = the anchors), masked to groups of blocks the
//            anchor's query block did not select; online log-sum-exp per anchor;
//   means    [mu_a; nu_a]^T += [Gk | Gv]^T W^T on the same MFMA (A = the group rows
//            through ds_read_b64_tr_b16, B = the bf16 weights).
// The anchor results (mu_a, nu_a, log2 Z_a - log2(e) q-bar_a . mu_a / sqrt(d)) go to
// the workspace; the exact pass adds delta_t and combines (Eqs. (2), (3)).
// ---------------------------------------------------------------------------
// 16-byte slot swizzle of the 32 x 256-byte group tiles of the tail pass: 16 consecutive
// rows at one logical slot (the scores' row reads) and 4 consecutive rows x 4 slots (the
// means' transposed reads) both land on 16 distinct slots.
__device__ __forceinline__ int swz_g(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct Tail2Args {
  int B, N, H, nb, nbp, nbw;
  const float* qanc;
  const uint16_t* gk; const uint16_t* gv; const float* glogn;
  const float* qbar; const float* kbar_t; const float* tau_i;   // routing inputs (fp32 block means)
  int sink_b0, sink_b1;
  float* tmu; float* tnu; float* tlz;
};

constexpr int kTailBufs = 3;               // tiles in flight: the one computed and two more
constexpr int kTailDmaPerTile = 9;         // buffer loads per wave per tile

// The tail pass's tile DMA is issued from asm.  Its three tile buffers are one LDS array,
// so for a DMA the compiler issues itself it cannot tell the buffer being filled from the
// one being read and waits for the newest DMA before the tile's first LDS read, which
// undoes the two-tile lead.  The compiler does not track these loads: every read of a
// buffer they fill is ordered by the loop's own vmcnt wait and barrier.  Hazard padding as
// in the asm: s_nop 4 after the v_readfirstlane writes of the resource and the LDS base,
// s_nop 0 between the M0 write and the load.
typedef int tail_intx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ tail_intx4 tail_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return tail_intx4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p),
                    (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu),
                    (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane to lds + 16 lane.
__device__ __forceinline__ void tail_dma16(tail_intx4 rsrc, uint32_t voffset, unsigned char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %0, 0 offen lds"
               ::"s"(rsrc), "s"(base), "v"(voffset)
               : "memory", "m0");
}

// buffer_load_dword ... lds: 4 bytes per lane to lds + 4 lane; lanes outside the buffer store zeros.
__device__ __forceinline__ void tail_dma4(tail_intx4 rsrc, uint32_t voffset, unsigned char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %0, 0 offen lds"
               ::"s"(rsrc), "s"(base), "v"(voffset)
               : "memory", "m0");
}

__global__ __launch_bounds__(128) void sol2_tail_kernel(Tail2Args a) {
  // Per buffer, filled by buffer DMA: the 32 group mean keys and mean values (32 rows x
  // 256 B each, 16-byte slots swizzled by swz_g so that both the row reads of the scores
  // and the transposed reads of the means are conflict-free); ln n_g of the tile's groups
  // (wave w brings groups 16 w .. 16 w + 15 into gl_s[.][w]); lanes past that range read
  // outside the buffer and store zeros in the unused tail of each row.  The routing words
  // of the workgroup's 32 query blocks (every chunk) are decided in the prologue and kept
  // in wsel (dynamic LDS, 32 x nbw words).
  __shared__ __attribute__((aligned(1024))) unsigned char Gk_s[kTailBufs][32 * 256];
  __shared__ __attribute__((aligned(1024))) unsigned char Gv_s[kTailBufs][32 * 256];
  __shared__ __attribute__((aligned(256))) float gl_s[kTailBufs][2][64];
  __shared__ int redo_s[2];
  extern __shared__ uint64_t wsel[];

  const int bh = blockIdx.y, i0 = blockIdx.x * 32;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;

  // Anchor means as the bf16 B operand: qa[ks] = dims 16 ks + 8 kg .. + 7 of anchor l32.
  const int qr = 16 * w + (l32 >> 1);                    // local query block of the anchor
  const int qi = i0 + qr;                                 // < nbp always (nbp is a multiple of 64)
  const size_t arow = ((size_t)bh * a.nbp + qi) * 2 + (l32 & 1);
  bf16x8 qa[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const float4 x0 = ((const float4*)(a.qanc + arow * kDim))[4 * ks + 2 * kg];
    const float4 x1 = ((const float4*)(a.qanc + arow * kDim))[4 * ks + 2 * kg + 1];
    qa[ks] = bf16x8{(__bf16)x0.x, (__bf16)x0.y, (__bf16)x0.z, (__bf16)x0.w,
                    (__bf16)x1.x, (__bf16)x1.y, (__bf16)x1.z, (__bf16)x1.w};
  }
  // Transposed-read offsets of the group rows (the V^T pattern of the Sol-Attn pass over 32
  // rows): row 4 kg + i'/4 (+ 8 for the upper half, + 16 per k-step), logical chunk
  // 4 mt + 2 (G % 2) + (i' % 4) / 2 of the 16-chunk row.
  int toff[4][2];
  {
    const int ip = lane & 15, gm = (lane >> 4) & 1;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 4 * kg + (ip >> 2) + 8 * half;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        toff[mt][half] = row * 256 + 16 * ((4 * mt + 2 * gm + ((ip & 3) >> 1)) ^ swz_g(row)) + 8 * (ip & 1);
    }
  }
  // scores A operand: group row l32, logical chunk 2 ks + kg
  int goff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) goff[ks] = l32 * 256 + 16 * ((2 * ks + kg) ^ swz_g(l32));

  // Routing of the workgroup's 32 query blocks i0 .. i0 + 31 against every key block, on
  // chip (Sol-Attn paper §3.1 Eq. (4) with the sink forced): the FMA sequence of
  // proxy_dot, the one the exact pass uses for its own query block, so both passes take
  // every decision alike.  Wave w takes chunks w, w + 2, w + 4, ... two at a time (c and
  // c + 2), lane l key blocks 64 c + l and 64 (c + 2) + l, each with 32 accumulators; the
  // Q-bar values are wave-uniform and come through scalar loads, each feeding 8 FMAs.
  {
    // the 32 Q-bar rows (rows i0 + q < nbp: in memory) are wave-uniform and read-only
    // here: read them through the constant address space, i.e. with scalar loads
    typedef const __attribute__((address_space(4))) float const_float;
    const const_float* qs = (const const_float*)(a.qbar + ((size_t)bh * a.nbp + i0) * kDim);
    const float4* kt = (const float4*)a.kbar_t + (size_t)bh * 32 * a.nbp;
    for (int c = w; c < a.nbw; c += 4) {                 // chunks c and c + 2 together
      const bool two = c + 2 < a.nbw;                    // uniform
      const int j0 = 64 * c + lane, j1 = two ? 64 * (c + 2) + lane : j0;
      float acc0[32], acc1[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) acc0[q] = acc1[q] = 0.f;
      for (int g = 0; g < 32; ++g) {
        const float4 kv0 = kt[(size_t)g * a.nbp + j0];
        const float4 kv1 = kt[(size_t)g * a.nbp + j1];
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const float4 qv = make_float4(qs[128 * q + 4 * g], qs[128 * q + 4 * g + 1], qs[128 * q + 4 * g + 2],
                                        qs[128 * q + 4 * g + 3]);
          acc0[q] = __builtin_fmaf(qv.x, kv0.x, acc0[q]);
          acc0[q] = __builtin_fmaf(qv.y, kv0.y, acc0[q]);
          acc0[q] = __builtin_fmaf(qv.z, kv0.z, acc0[q]);
          acc0[q] = __builtin_fmaf(qv.w, kv0.w, acc0[q]);
          acc1[q] = __builtin_fmaf(qv.x, kv1.x, acc1[q]);
          acc1[q] = __builtin_fmaf(qv.y, kv1.y, acc1[q]);
          acc1[q] = __builtin_fmaf(qv.z, kv1.z, acc1[q]);
          acc1[q] = __builtin_fmaf(qv.w, kv1.w, acc1[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const int qi = i0 + q;
        const float tau = a.tau_i[(size_t)bh * a.nbp + qi];
        const uint64_t w0 = exact_word(__ballot(acc0[q] * kScale2 > tau), c, a.nb, a.sink_b0, a.sink_b1);
        if (lane == 0) wsel[q * a.nbw + c] = qi < a.nb ? w0 : 0ull;
        if (two) {
          const uint64_t w1 = exact_word(__ballot(acc1[q] * kScale2 > tau), c + 2, a.nb, a.sink_b0, a.sink_b1);
          if (lane == 0) wsel[q * a.nbw + c + 2] = qi < a.nb ? w1 : 0ull;
        }
      }
    }
    __syncthreads();                                      // words complete; staging buffer free
  }

  // DMA of tile t (key blocks 16 t .. 16 t + 15) into buffer `buf`: wave w, instruction n
  // fills 1 KB segment 4 w + n of each group array (rows r = 16 w + 4 n + lane / 16; slot
  // lane % 16 holds logical chunk (lane % 16) ^ swz_g(r)), then one dword per lane of
  // ln n_g.
  const uint32_t grow = (uint32_t)(16 * w + (lane >> 4));
  uint32_t gdma[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) gdma[n] = (grow + 4 * n) * 256 + 16 * ((lane & 15) ^ swz_g(grow + 4 * n));
  constexpr uint32_t kPastEnd = 0x80000000u;             // beyond every buffer's range: reads zero
  const uint32_t gldma = lane < 16 ? (uint32_t)(16 * w + lane) * 4 : kPastEnd;
  const int ntiles = a.nbp / 16;
  auto issue_tile = [&](int t, int buf) {
    const uint32_t gbytes = (uint32_t)a.nbp * 2 * 256;
    const tail_intx4 rk = tail_rsrc(a.gk + (size_t)bh * a.nbp * 2 * kDim, gbytes);
    const tail_intx4 rv = tail_rsrc(a.gv + (size_t)bh * a.nbp * 2 * kDim, gbytes);
    const tail_intx4 rl = tail_rsrc(a.glogn + (size_t)bh * a.nbp * 2, (uint32_t)a.nbp * 2 * 4);
    const uint32_t toff_g = (uint32_t)t * 32 * 256;          // 32 group rows per tile
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      tail_dma16(rk, toff_g + gdma[n], Gk_s[buf] + 1024 * (4 * w + n));
      tail_dma16(rv, toff_g + gdma[n], Gv_s[buf] + 1024 * (4 * w + n));
    }
    tail_dma4(rl, lane < 16 ? (uint32_t)t * 32 * 4 + gldma : kPastEnd, (unsigned char*)gl_s[buf][w]);
  };

  floatx16 num[8];                                        // rows: dims (0..127 mu, 128..255 nu); cols: anchors
  float m_run = kNegInf, z_run = 0.f;
  // One pass over the tiles.  kSafe = false: the anchor's first tile with a tail group
  // fixes the reference m (its largest tail logit) and every weight is 2^(l - m) with no
  // rescaling of the 128 accumulators; kSafe = true: running maximum with the rescale.
  auto run_tiles = [&](auto safe_tag) {
    constexpr bool kSafe = decltype(safe_tag)::value;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) num[mt] = floatx16{};
    m_run = kNegInf;
    z_run = 0.f;
    issue_tile(0, 0);
    if (ntiles > 1) issue_tile(1, 1);
    for (int t = 0; t < ntiles; ++t) {
      const int j0 = 16 * t, buf = t % kTailBufs;
      if (t + 1 < ntiles) wait_vm<kTailDmaPerTile>();     // tile t landed (tile t + 1 may be in flight)
      else wait_vm0();
      lds_barrier();                                      // every wave's part of tile t; buffer of t - 1 free
      if (t + 2 < ntiles) issue_tile(t + 2, (t + 2) % kTailBufs);
      // ---- tail scores of the tile's 32 groups against the wave's 32 anchors
      floatx16 s = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(Gk_s[buf] + goff[ks]), qa[ks], s, 0, 0, 0);
      // routing bits of the anchor's query block for the tile's 16 key blocks
      const uint32_t mine = (uint32_t)(wsel[qr * a.nbw + (t >> 2)] >> (16 * (t & 3))) & 0xffffu;
      // ln n_g of the lane's 16 groups: rows 8 q4 + 4 kg .. + 3, four 16-byte LDS reads taken
      // up front (read under the tail condition, each would be a branch with its own wait)
      float4 lng4[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int g0 = 8 * q4 + 4 * kg;
        lng4[q4] = *(const float4*)&gl_s[buf][g0 >> 4][g0 & 15];
      }
      float mx = kNegInf;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int g = 8 * (idx >> 2) + 4 * kg + (idx & 3);  // group row of the tile
        const bool tail = !((mine >> (g >> 1)) & 1) && j0 + (g >> 1) < a.nb;
        const float4 l4 = lng4[idx >> 2];
        const float lng = (idx & 3) == 0 ? l4.x : (idx & 3) == 1 ? l4.y : (idx & 3) == 2 ? l4.z : l4.w;
        s[idx] = tail ? (s[idx] * kScale2 + lng) * kLog2e : kNegInf;
        mx = fmaxf(mx, s[idx]);
      }
      mx = max_with_partner(mx);
      float m_use;
      if constexpr (kSafe) {
        const float m_new = fmaxf(m_run, mx);
        m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        z_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) num[mt][idx] *= alpha;
        m_run = m_new;
      } else {
        m_run = m_run == kNegInf ? mx : m_run;
        m_use = m_run == kNegInf ? 0.f : m_run;
      }
      bf16x8 pa[2];
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) pa[idx >> 3][idx & 7] = (__bf16)__builtin_amdgcn_exp2f(s[idx] - m_use);
      z_run = add_bf16x8(pa[1], add_bf16x8(pa[0], z_run));  // the bf16 weights of the numerators
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const unsigned char* gt = mt < 4 ? Gk_s[buf] : Gv_s[buf];   // m-tiles 0..3: mu dims, 4..7: nu
          const uint2v lo = lds_read_tr16(gt + toff[mt & 3][0] + st * 16 * 256);
          const uint2v hi = lds_read_tr16(gt + toff[mt & 3][1] + st * 16 * 256);
          const uint4v av = {lo[0], lo[1], hi[0], hi[1]};
          num[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pa[st], num[mt], 0, 0, 0);
        }
    }
  };
  run_tiles(BoolTag<false>{});
  {
    // A weight or sum that overflowed the fixed reference (a tail logit more than ~2^127
    // above it): redo the workgroup's tiles with the running maximum.
    float chk = z_run * 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) chk = __builtin_fmaf(num[mt][idx], 0.f, chk);
    const bool bad = __ballot(!(chk == 0.f)) != 0;
    if (lane == 0) redo_s[w] = bad;
    __syncthreads();                                      // also: every wave is past its last tile
    if (redo_s[0] | redo_s[1]) run_tiles(BoolTag<true>{});
  }

  // ---- anchor results: mu_a, nu_a and log2 Z_a - log2(e) q-bar_a . mu_a / sqrt(d)
  const float z = sum_with_partner(z_run);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  if (qi < a.nb) {
    float qmu = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * (mt & 3) + 8 * gq + 4 * kg;   // dims d .. d + 3 of mu (mt < 4) or nu
        float4 r4 = make_float4(num[mt][4 * gq] * inv, num[mt][4 * gq + 1] * inv, num[mt][4 * gq + 2] * inv,
                                num[mt][4 * gq + 3] * inv);
        if (mt < 4) {
          *(float4*)(a.tmu + arow * kDim + d) = r4;
          const float4 q4 = *(const float4*)(a.qanc + arow * kDim + d);
          qmu += q4.x * r4.x + q4.y * r4.y + q4.z * r4.z + q4.w * r4.w;
        } else {
          *(float4*)(a.tnu + arow * kDim + d) = r4;
        }
      }
    qmu = sum_with_partner(qmu);
    if (kg == 0) a.tlz[arow] = z > 0.f ? m_run + __log2f(z) - qmu * kScale2 * kLog2e : kNegInf;
  }
}

hipError_t launch_tail2(Shape s, const Workspace& ws, int sink_b0, int sink_b1, hipStream_t stream) {
  Tail2Args a;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = ws.nbp / 64;
  a.qanc = ws.qanc;
  a.gk = ws.gk; a.gv = ws.gv; a.glogn = ws.glogn;
  a.qbar = ws.qbar; a.kbar_t = ws.kbar_t; a.tau_i = ws.tau_i;
  a.sink_b0 = sink_b0; a.sink_b1 = sink_b1;
  a.tmu = ws.tmu; a.tnu = ws.tnu; a.tlz = ws.tlz;
  const size_t words_lds = (size_t)32 * a.nbw * sizeof(uint64_t);   // <= 32 KB (nbw <= 128)
  hipLaunchKernelGGL(sol2_tail_kernel, dim3((ws.nb + 31) / 32, s.B * s.H), dim3(128), words_lds, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 2b: exact FP8 attention over the selected blocks, combined with the tail.
// One workgroup per (b, h, query block i), two wave64s; wave w owns query rows
// 32 w .. 32 w + 31, which are exactly anchor a = (i, w).
//   * Routing on chip: the query block's words, decided with the tail pass's arithmetic.
//   * The selected blocks stream through LDS: the
//     FP8 K tile (64 x 128 B) and the bf16 V tile (64 x 256 B) by buffer DMA
//     (buffer_load ... lds), V of tile t overlapping S_t, K of tile t + 1
//     overlapping PV_t.
//   * S^T = K8 Q8^T on v_mfma_f32_32x32x64_f8f6f4 (OCP E4M3; issued through the
//     scaled form with unit scales), times s_q s_k / sqrt(d); online softmax; O^T +=
//     V^T P^T in bf16 exactly as in the Sol-Attn pass.  The FP8-PV instance instead
//     streams the per-head E4M3 V^T tile (128 x 64 B), turns each score into its
//     ExpCast byte against the running row maximum, and runs PV and the row sums
//     (an all-ones B operand) on the same FP8 MFMA, so the denominator is the sum
//     of exactly the decoded weights that multiply V.
//   * Epilogue: delta_t = (q'_t - q-bar_a) . mu_a / sqrt(d) from the dequantized query
//     codes, lambda_t = ln Z_a + delta_t, and Eq. (3) with the exact state.
// ---------------------------------------------------------------------------
constexpr int kMaxChunks2 = 128;
constexpr int kThreeWaveChunks = 8;   // 32768 tokens

struct Fused2Args {
  const uint16_t* v; uint16_t* out;
  int B, N, H, nb, nbp, nbw, tp;
  const uint8_t* q8; const uint8_t* k8; const float* qscale; const float* kscale;
  const float* qbar; const float* kbar_t; const float* tau_i;   // routing inputs (fp32 block means)
  int sink_b0, sink_b1;
  uint64_t* mask_out;                        // routing words out (training / test export; NULL = none)
  const float* tmu; const float* tnu; const float* tlz;
  const uint8_t* v8t; const float* vscale;   // FP8 PV only
  unsigned long long* pairs;                 // += selected token pairs n_i n_j (NULL = none)
  float* lse;                                // [B][H][tp] base-2 log of each row's denominator (NULL = none)
  float* ofp;                                // [B][H][tp][128] fp32 output rows (training; NULL = none)
};

// 16-byte slot swizzle of the 128 x 64-byte FP8 V^T tile (rows = dims): 16 consecutive
// rows reading one logical chunk cover all 16 bank groups of a 64-bank LDS.
__device__ __forceinline__ int swz8v(int r) { return (r >> 2) & 3; }

// 16-byte slot swizzle of the 64 x 128-byte FP8 K tile: 16 consecutive rows reading one
// logical chunk land on 16 distinct (row parity, slot) bank groups with 64 banks, and
// 8 consecutive rows on 8 distinct slots with 32 banks.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// kWaves: waves per SIMD the register budget is cut for.  Both instances come in two forms:
// three waves (bf16 V: 163 VGPRs; FP8 PV: 168 with a few spilled) for sequences of up to
// kThreeWaveChunks routing chunks, where the extra occupancy hides more of the memory waits,
// and two beyond, where more workgroups in flight cost more in L2 misses than they hide.
template <bool kPv8, int kWaves>
__global__ __launch_bounds__(128, kWaves) void sol2_fused_kernel(Fused2Args a) {
  __shared__ __attribute__((aligned(1024))) unsigned char K8l[64 * 128];
  __shared__ __attribute__((aligned(1024))) unsigned char Vl[64 * 256];
  __shared__ uint64_t sel_s[kMaxChunks2];
  __shared__ float4 qbar_s[kDim / 4];                        // Q-bar_i (fp32), read by every lane
  __shared__ __attribute__((aligned(16))) float mu_s[2][kDim];
  __shared__ __attribute__((aligned(16))) float nu_s[2][kDim];
  __shared__ int redo2_s[2];

  const int total = a.B * a.H * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  const int i = __builtin_amdgcn_readfirstlane(item % a.nb);
  const int bh = __builtin_amdgcn_readfirstlane(item / a.nb);
  const int h = __builtin_amdgcn_readfirstlane(bh % a.H), b = __builtin_amdgcn_readfirstlane(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)a.H * kDim;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;
  const size_t qrow_blk = (size_t)bh * a.nbp + i;

  if (tid < kDim / 4) qbar_s[tid] = ((const float4*)(a.qbar + qrow_blk * kDim))[tid];
  const size_t arow = qrow_blk * 2 + w;
  if (lane < 32) {
    ((float4*)mu_s[w])[lane] = ((const float4*)(a.tmu + arow * kDim))[lane];
    ((float4*)nu_s[w])[lane] = ((const float4*)(a.tnu + arow * kDim))[lane];
  }
  const float tlz = a.tlz[arow];
  const float sq = a.qscale[qrow_blk];

  const int qrow = i * kBlock + w * 32 + l32;           // < tp always; rows >= N hold zero codes
  intx8 qf[2];
  {
    const intx8* src = (const intx8*)(a.q8 + ((size_t)bh * a.tp + qrow) * kDim);
    qf[0] = src[kg];          // dims 32 kg .. 32 kg + 31
    qf[1] = src[2 + kg];      // dims 64 + 32 kg .. + 31
  }
  __syncthreads();
  // Routing on chip (Sol-Attn paper §3.1 Eq. (4), sink forced): wave w scores chunks w,
  // w + 2, ..., lane l key block 64 c + l, with proxy_dot -- the FMA sequence the tail pass
  // uses for the same pairs -- and one ballot per chunk; the words stay in LDS.
  {
    const float tau = a.tau_i[qrow_blk];
    const float4* kt = (const float4*)a.kbar_t + (size_t)bh * 32 * a.nbp;
    for (int c = w; c < a.nbw; c += 2) {
      const float acc = proxy_dot(qbar_s, kt, a.nbp, 64 * c + lane);
      const uint64_t word = exact_word(__ballot(acc * kScale2 > tau), c, a.nb, a.sink_b0, a.sink_b1);
      if (lane == 0) {
        sel_s[c] = word;
        if (a.mask_out != nullptr) a.mask_out[((size_t)bh * a.nb + i) * a.nbw + c] = word;
      }
    }
  }
  __syncthreads();
  if (a.pairs != nullptr && tid == 0) {
    // selected token pairs of this query block: n_i times the valid tokens of its exact blocks
    unsigned long long cols = 0;
    for (int c = 0; c < a.nbw; ++c) cols += 64ull * (unsigned)__builtin_popcountll(sel_s[c]);
    const int last = a.nb - 1;
    if ((sel_s[last / 64] >> (last & 63)) & 1) cols -= (unsigned long long)(kBlock - (a.N - last * kBlock));
    atomicAdd(a.pairs, cols * (unsigned long long)min(kBlock, a.N - i * kBlock));
  }

  // K8 operand reads: row 32 mt + l32, logical chunks 4 ks + 2 kg (+1); swz8 depends on l32 only.
  const int sz = swz8(l32);
  int k8off[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) k8off[ks][hf] = l32 * 128 + 16 * ((4 * ks + 2 * kg + hf) ^ sz);
  int voff[4];
  v_operand_offsets(lane, voff);
  // K8 DMA, wave w instruction n: 1 KB segment 4 w + n = rows 8 (4 w + n) + lane / 8, slot
  // lane % 8 holding logical chunk (lane % 8) ^ swz8(row); swz8(row) = lane / 8 ^ (n & 1).
  uint32_t k8dma[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) k8dma[par] = (lane >> 3) * 128 + 16 * ((lane & 7) ^ (lane >> 3) ^ par);
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const uint32_t span_in = (uint32_t)(((size_t)a.N - 1) * rs + kDim) * 2;
  const DmaOffsets doff = dma_offsets(row_bytes, w, lane);
  const uint8_t* k8_head = a.k8 + (size_t)bh * a.tp * kDim;
  const uint32_t span_k8 = (uint32_t)a.tp * kDim;
  auto issue_k = [&](int jb) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(uniform_ptr(k8_head), span_k8);
    const uint32_t tile_off = (uint32_t)jb * 64 * 128;
#pragma unroll
    for (int n = 0; n < 4; ++n)
      dma16_buf(rsrc, tile_off + 1024 * (4 * w + n) + k8dma[n & 1], 0, K8l + 1024 * (4 * w + n));
  };
  // FP8 V^T tile DMA, wave w instruction n: 1 KB segment 4 w + n = dims 16 (4 w + n) + lane / 4,
  // slot lane % 4 holding logical chunk (lane % 4) ^ swz8v(dim) (swz8v depends on lane / 4 only).
  const uint32_t v8dma = (uint32_t)(lane >> 2) * a.tp + 16 * ((lane & 3) ^ swz8v(lane >> 2));
  const uint8_t* v8_head = a.v8t + (size_t)bh * kDim * a.tp;
  auto issue_v = [&](int jb) {
    if constexpr (kPv8) {
      const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(uniform_ptr(v8_head), (uint32_t)kDim * a.tp);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        dma16_buf(rsrc, (uint32_t)(16 * (4 * w + n)) * a.tp + (uint32_t)jb * 64 + v8dma, 0, Vl + 1024 * (4 * w + n));
    } else {
      dma_tile<true>(Vl, make_rsrc(uniform_ptr(a.v + head_off), span_in), (uint32_t)jb * 64 * row_bytes, row_bytes,
                     doff, w);
    }
  };
  // FP8 V^T operand reads: row (dim) 32 mt + l32, logical chunks 2 kg, 2 kg + 1.
  int v8off[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) v8off[hf] = l32 * 64 + 16 * ((2 * kg + hf) ^ swz8v(l32));
  floatx16 ol = {};                                        // FP8 PV: sum of the decoded P bytes (all rows)
  // Selected blocks in order.
  int c_it = 0;
  uint64_t bits = 0;
  auto next_sel = [&]() -> int {
    while (!bits) {
      if (c_it >= a.nbw) return -1;
      bits = uniform64(sel_s[c_it++]);
    }
    const int jb = (c_it - 1) * 64 + __builtin_ctzll(bits);
    bits &= bits - 1;
    return __builtin_amdgcn_readfirstlane(jb);
  };

  floatx16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  const float qs = sq * kScale2 * kLog2e;
  const int last_partial = a.N % kBlock ? a.nb - 1 : -1;   // the only block with masked rows
  // One selected block: scores, reference, P (bf16 or ExpCast bytes), PV.  kPartial masks
  // the rows past the end of the sequence (only the last block, which comes last in the
  // ascending order); full blocks take the logits straight from the raw scores.  The
  // ExpCast bytes are defined against the running maximum, so the FP8 PV path always keeps
  // it (kSafe); the bf16 path takes its reference from the first exact block of the row
  // (kSafe = false: no rescaling of O and l) and is redone with the running maximum if a sum
  // overflows.
  auto tile = [&](auto partial_tag, auto safe_tag, int cur, int nxt) {
    constexpr bool kPartial = decltype(partial_tag)::value;
    constexpr bool kSafe = kPv8 || decltype(safe_tag)::value;
    floatx16 s0 = {}, s1 = {};
    // This block's V DMA is issued here, its instructions spread over the score products
    // (two per product for the bf16 tile, one for the FP8 one) instead of as one burst.
    issue_v(cur);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4v a0l = *(const uint4v*)(K8l + k8off[ks][0]), a0h = *(const uint4v*)(K8l + k8off[ks][1]);
      const uint4v a1l = *(const uint4v*)(K8l + 32 * 128 + k8off[ks][0]);
      const uint4v a1h = *(const uint4v*)(K8l + 32 * 128 + k8off[ks][1]);
      const intx8 a0 = {(int)a0l[0], (int)a0l[1], (int)a0l[2], (int)a0l[3], (int)a0h[0], (int)a0h[1], (int)a0h[2], (int)a0h[3]};
      const intx8 a1 = {(int)a1l[0], (int)a1l[1], (int)a1l[2], (int)a1l[3], (int)a1h[0], (int)a1h[1], (int)a1h[2], (int)a1h[3]};
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[ks], s0, 0, 0, 0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[ks], s1, 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmem, kPv8 ? 1 : 2, 0);
      }
    }
    // logits in log2 units are f * s (f = s_q s_k log2(e) / sqrt(d) > 0, so the max of the
    // raw scores gives the max of the logits)
    const float f = qs * a.kscale[(size_t)bh * a.nbp + cur];
    if constexpr (kPartial) {
      const int valid = a.N - cur * kBlock;
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
        s0[idx] = key0 < valid ? s0[idx] : kNegInf;
        s1[idx] = key0 + 32 < valid ? s1[idx] : kNegInf;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int idx = 1; idx < 16; ++idx) mx = fmaxf(mx, fmaxf(s0[idx], s1[idx]));
    mx = max_with_partner(mx) * f;
    float m_use, alpha = 1.f;
    if constexpr (kSafe) {
      const float m_new = fmaxf(m_run, mx);
      m_use = m_new == kNegInf ? 0.f : m_new;
      // Unconditional rescale (skipping it behind a wave-uniform branch made results
      // timing-dependent with two waves per SIMD).
      alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) o[mt][idx] *= alpha;
      m_run = m_new;
    } else {
      m_run = m_run == kNegInf ? mx : m_run;               // the row's first exact block
      m_use = m_run == kNegInf ? 0.f : m_run;
    }
    if constexpr (kPv8) {
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) ol[idx] *= alpha;
      // ExpCast bytes c = RNE(8 (x - m) + 55.65) (<= 56 since x <= m; v_cvt_pk_u8_f32
      // rounds to nearest even and saturates below at 0, which is the clip; masked rows
      // are -inf and give 0), in the PV operand order: byte e = idx of s0, 16 + idx of s1.
      const float c0 = 55.65f - 8.f * m_use;
      const float f8 = 8.f * f;
      uint32_t pw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        pw[idx >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s0[idx], f8, c0), idx & 3, pw[idx >> 2]);
        pw[4 + (idx >> 2)] =
            __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(s1[idx], f8, c0), idx & 3, pw[4 + (idx >> 2)]);
      }
      const intx8 pc = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
      const intx8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,   // E4M3 1.0
                          0x38383838, 0x38383838, 0x38383838, 0x38383838};
      wait_vm0();
      lds_barrier();                                       // V(cur) landed; K buffer free
      // the next block's K DMA (after the last block, this block's again, so that every
      // block has the same shape), one instruction per PV product
      issue_k(nxt >= 0 ? nxt : cur);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint4v lo = *(const uint4v*)(Vl + mt * 32 * 64 + v8off[0]);
        const uint4v hi = *(const uint4v*)(Vl + mt * 32 * 64 + v8off[1]);
        const intx8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        o[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pc, o[mt], 0, 0, 0, 0, 0, 0);
      }
      ol = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pc, ol, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmem, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    } else {
      const float neg_m = -m_use;
      bf16x8 pa[4];
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        pa[idx >> 3][idx & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[idx], f, neg_m));   // keys 16 st ..
        pa[2 + (idx >> 3)][idx & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s1[idx], f, neg_m));
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) l_run = add_bf16x8(pa[st], l_run);
      wait_vm0();
      lds_barrier();                                       // V(cur) landed; K buffer free
      if (nxt >= 0) issue_k(nxt);
      pv_tile(o, Vl, voff, pa);
    }
  };
  auto run_tiles = [&](auto safe_tag) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
    m_run = kNegInf;
    l_run = 0.f;
    c_it = 0;
    bits = 0;
    int cur = next_sel();
    if (cur >= 0) issue_k(cur);
    while (cur >= 0) {
      const int nxt = next_sel();
      wait_vm0();
      lds_barrier();                                       // K8(cur) landed; V buffer free
      if (cur == last_partial) tile(BoolTag<true>{}, safe_tag, cur, nxt);
      else tile(BoolTag<false>{}, safe_tag, cur, nxt);
      cur = nxt;
    }
    wait_vm0();                                            // FP8 PV: the last block's repeated K DMA
  };
  if constexpr (kPv8) {
    run_tiles(BoolTag<true>{});
  } else {
    run_tiles(BoolTag<false>{});
    // A sum that overflowed the row's reference (a logit more than ~2^127 above it): redo
    // the workgroup's blocks with the running maximum.
    float chk = l_run * 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) chk = __builtin_fmaf(o[mt][idx], 0.f, chk);
    const bool bad = __ballot(!(chk == 0.f)) != 0;
    if (lane == 0) redo2_s[w] = bad;
    __syncthreads();                                       // also: both waves are past their last block
    if (redo2_s[0] | redo2_s[1]) run_tiles(BoolTag<true>{});
  }

  // ---- epilogue: tail logit lambda_t = log2 Z_a + log2(e) q'_t . mu_a / sqrt(d) (the
  // q-bar_a term is in tlz), then Eq. (3) with one shared denominator.
  float qmu = 0.f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float f4[4];
      fp8x4_to_f32((uint32_t)qf[ks][m], f4);
#pragma unroll
      for (int e = 0; e < 4; ++e) qmu += f4[e] * mu_s[w][64 * ks + 32 * kg + 4 * m + e];
    }
  qmu = sum_with_partner(qmu) * sq;
  const float lam2 = tlz == kNegInf ? kNegInf : tlz + qmu * kScale2 * kLog2e;
  const float m_fin = fmaxf(m_run, lam2);
  const float m_use = m_fin == kNegInf ? 0.f : m_fin;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  const float wt = __builtin_amdgcn_exp2f(lam2 - m_use);
  // FP8 PV: the exact sums come from the MFMA (already over both k-halves) and the
  // numerator carries the per-head V scale.
  const float l_ex = kPv8 ? ol[0] : sum_with_partner(l_run);
  const float vs = kPv8 ? a.vscale[bh] : 1.f;
  const float l_tot = l_ex * alpha + wt;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (a.lse != nullptr && kg == 0 && qrow < a.N)     // training forward: the row's log2-sum-exp
    a.lse[(size_t)bh * a.tp + qrow] = l_tot > 0.f ? m_use + __log2f(l_tot) : kNegInf;
  if (qrow < a.N && a.out != nullptr) {
    uint16_t* dst = a.out + head_off + (size_t)qrow * rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * kg;
        float r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = (o[mt][4 * g + e] * (alpha * vs) + wt * nu_s[w][d0 + e]) * inv;
        if (a.ofp != nullptr) *(floatx4*)(a.ofp + ((size_t)bh * a.tp + qrow) * kDim + d0) = floatx4{r4[0], r4[1], r4[2], r4[3]};
        uint2v pk;
        pk[0] = pack_bf16x2(r4[0], r4[1]);
        pk[1] = pack_bf16x2(r4[2], r4[3]);
        *(uint2v*)(dst + d0) = pk;
      }
  }
}

__global__ void zero_counter2_kernel(unsigned long long* p) { *p = 0ull; }

hipError_t launch_fused2(const uint16_t* v, uint16_t* out, Shape s, const Workspace& ws, bool pv8,
                         unsigned long long* pairs, int sink_b0, int sink_b1, uint64_t* mask_out,
                         hipStream_t stream) {
  if (ws.nbp / 64 > kMaxChunks2 || (pv8 && (!ws.v8t || !ws.vscale))) return hipErrorInvalidValue;
  Fused2Args a;
  a.v = v; a.out = out;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = ws.nbp / 64; a.tp = ws.nbp * kBlock;
  a.q8 = ws.q8; a.k8 = ws.k8; a.qscale = ws.qscale; a.kscale = ws.kscale;
  a.qbar = ws.qbar; a.kbar_t = ws.kbar_t; a.tau_i = ws.tau_i;
  a.sink_b0 = sink_b0; a.sink_b1 = sink_b1; a.mask_out = mask_out;
  a.tmu = ws.tmu; a.tnu = ws.tnu; a.tlz = ws.tlz;
  a.v8t = ws.v8t; a.vscale = ws.vscale;
  a.pairs = pairs;
  a.lse = pv8 ? nullptr : ws.lse;            // set for the Sol-Attn2 training layout only
  a.ofp = pv8 ? nullptr : ws.ofp;
  if (pairs != nullptr) {   // the counter is cleared on the stream by a kernel (graph-safe)
    hipLaunchKernelGGL(zero_counter2_kernel, dim3(1), dim3(1), 0, stream, pairs);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  const int total = s.B * s.H * ws.nb;
  const bool three = ws.nbp / 64 <= kThreeWaveChunks;
  if (pv8) {
    if (three) hipLaunchKernelGGL((sol2_fused_kernel<true, 3>), dim3(total), dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((sol2_fused_kernel<true, 2>), dim3(total), dim3(128), 0, stream, a);
  } else {
    if (three) hipLaunchKernelGGL((sol2_fused_kernel<false, 3>), dim3(total), dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((sol2_fused_kernel<false, 2>), dim3(total), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace solattn
