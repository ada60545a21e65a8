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
// ties joining the upper group; V stays bf16; an empty block uses scale 1.
#include "common.h"
#include "kernels.h"
#include "tile.h"

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

  float sumq0[8], sumq1[8], sumk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sumq0[e] = sumq1[e] = sumk[e] = 0.f;
  const size_t dst0 = ((size_t)bh * tp + t0) * kDim + c * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int t = r + 16 * p;
    uint2v cq = {0u, 0u}, ck = {0u, 0u};
    if (t < n) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float yq[4], yk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          yq[e] = fminf(fmaxf(__fdiv_rn(xq[p][4 * m + e], sq), -448.f), 448.f);
          yk[e] = fminf(fmaxf(__fdiv_rn(xk[p][4 * m + e], sk), -448.f), 448.f);
        }
        cq[m] = fp8x2(yq[0], yq[1]) | (fp8x2(yq[2], yq[3]) << 16);
        ck[m] = fp8x2(yk[0], yk[1]) | (fp8x2(yk[2], yk[3]) << 16);
      }
      // sums of the decoded codes (exact in fp32: multiples of 2^-9 below 2^15)
      float dq[8], dk[8];
      fp8x4_to_f32(cq[0], dq); fp8x4_to_f32(cq[1], dq + 4);
      fp8x4_to_f32(ck[0], dk); fp8x4_to_f32(ck[1], dk + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (p < 2) sumq0[e] += dq[e]; else sumq1[e] += dq[e];
        sumk[e] += dk[e];
      }
    }
    if (j < nb) {   // codes of rows t >= n inside the last block are written as zeros
      *(uint2v*)(q8 + dst0 + (size_t)t * kDim) = cq;
      *(uint2v*)(k8 + dst0 + (size_t)t * kDim) = ck;
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
__global__ __launch_bounds__(128) void qhat_kernel(const float* __restrict__ qbar, int N, int nb, int nbp,
                                                   float* __restrict__ qhat) {
  const int bh = blockIdx.x, d = threadIdx.x;
  float acc = 0.f;
  for (int i = 0; i < nb; ++i) acc += (float)min(kBlock, N - i * kBlock) * qbar[((size_t)bh * nbp + i) * kDim + d];
  qhat[(size_t)bh * kDim + d] = acc / (float)N;
}

hipError_t launch_qhat(Shape s, const Workspace& ws, hipStream_t stream) {
  hipLaunchKernelGGL(qhat_kernel, dim3(s.B * s.H), dim3(kDim), 0, stream, ws.qbar, s.N, ws.nb, ws.nbp, ws.qhat);
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
                                                     float* __restrict__ glogn, uint64_t* __restrict__ ghi) {
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
  for (int u = 0; u < n; ++u) {
    const uint32_t vw = *(const uint32_t*)(vb + (size_t)u * rs);
    const uint32_t kw = *(const uint16_t*)(kb + (size_t)u * kDim);
    const auto kf = __builtin_amdgcn_cvt_pk_f32_fp8(kw, false);
    const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
    if ((hi >> u) & 1) { kh[0] += kf[0]; kh[1] += kf[1]; vh[0] += v0; vh[1] += v1; }
    else               { kl[0] += kf[0]; kl[1] += kf[1]; vl[0] += v0; vl[1] += v1; }
  }
  const int nh = __popcll(hi), nl = n - nh;
  const float ih = nh > 0 ? 1.f / (float)nh : 0.f, il = nl > 0 ? 1.f / (float)nl : 0.f;
  uint32_t* gko = (uint32_t*)(gk + row * 2 * kDim);
  uint32_t* gvo = (uint32_t*)(gv + row * 2 * kDim);
  gko[lane] = pack_bf16x2(sk * kh[0] * ih, sk * kh[1] * ih);
  gko[64 + lane] = pack_bf16x2(sk * kl[0] * il, sk * kl[1] * il);
  gvo[lane] = pack_bf16x2(vh[0] * ih, vh[1] * ih);
  gvo[64 + lane] = pack_bf16x2(vl[0] * il, vl[1] * il);
  if (lane == 0) {
    glogn[row * 2] = nh > 0 ? __logf((float)nh) : kNegInf;
    glogn[row * 2 + 1] = nl > 0 ? __logf((float)nl) : kNegInf;
    ghi[row] = hi;
  }
}

hipError_t launch_groups(const uint16_t* v, Shape s, const Workspace& ws, hipStream_t stream) {
  const int total = s.B * s.H * ws.nbp;
  hipLaunchKernelGGL(groups_kernel, dim3((total + 3) / 4), dim3(256), 0, stream, v, ws.k8, ws.kscale, ws.qhat, s.N,
                     s.H, ws.nb, ws.nbp, ws.nbp * kBlock, total, ws.gk, ws.gv, ws.glogn, ws.ghi);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 2: fused FP8 exact attention + complementary tail.
// One workgroup per (b, h, query block i); wave w owns query rows 32 w .. 32 w + 31,
// which are exactly anchor a = (i, w).
//   exact: S^T = K8 Q8^T on v_mfma_f32_32x32x64_f8f6f4 (OCP E4M3), times s_q s_k;
//          online softmax and O^T += V^T P^T in bf16 as in Sol-Attn.
//   tail:  per chunk, lane jj scores the two groups of block 64 c + jj against the
//          anchor mean (Eq. (1), online log-sum-exp in log2 units) and the wave
//          accumulates sum w (k-bar_g, v-bar_g) with lane-owned dims.
//   end:   mu_a, nu_a, ln Z_a; delta_t (Eq. (2)); Eq. (3) with the exact state.
// ---------------------------------------------------------------------------
struct Fused2Args {
  const uint16_t* v; uint16_t* out;
  int B, N, H, nb, nbp, nbw, tp;
  const uint8_t* q8; const uint8_t* k8; const float* qscale; const float* kscale;
  const float* qbar; const float* kbar_t; const float* tau_i; const float* qanc;
  const uint16_t* gk; const uint16_t* gv; const float* glogn;
  int sink_b0, sink_b1;
  uint64_t* mask_out;
};

__global__ __launch_bounds__(128) void sol2_fused_kernel(Fused2Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char K8s[64 * kK8Stride];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[128 * kVtStride];
  __shared__ __attribute__((aligned(16))) float qb_s[kDim];
  __shared__ float part[2][64];
  __shared__ __attribute__((aligned(16))) float qa_s[2][kDim];
  __shared__ float w_s[2][128];
  __shared__ __attribute__((aligned(16))) float mu_s[2][kDim];
  __shared__ __attribute__((aligned(16))) float nu_s[2][kDim];

  const int total = a.B * a.H * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  const int i = item % a.nb;
  const int bh = item / a.nb;
  const int h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const size_t rs = (size_t)a.H * kDim;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;
  const size_t qrow_blk = (size_t)bh * a.nbp + i;

  if (tid < 32) ((float4*)qb_s)[tid] = ((const float4*)(a.qbar + qrow_blk * kDim))[tid];
  if (lane < 32) ((float4*)qa_s[w])[lane] = ((const float4*)(a.qanc + (qrow_blk * 2 + w) * kDim))[lane];
  const float tau_i = a.tau_i[qrow_blk];
  const float sq = a.qscale[qrow_blk];

  const int qrow = i * kBlock + w * 32 + l32;           // < tp always; rows >= N hold zero codes
  intx8 qf[2];
  {
    const intx8* src = (const intx8*)(a.q8 + ((size_t)bh * a.tp + qrow) * kDim);
    qf[0] = src[kg];          // dims 32 kg .. 32 kg + 31
    qf[1] = src[2 + kg];      // dims 64 + 32 kg .. + 31
  }
  floatx16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  // tail state (log2 units), lane owns dims 2 lane, 2 lane + 1
  float m_t = kNegInf, z_t = 0.f, tk0 = 0.f, tk1 = 0.f, tv0 = 0.f, tv1 = 0.f;
  __syncthreads();

  const float4* kt = (const float4*)a.kbar_t + (size_t)bh * 32 * a.nbp;
  const int nchunks = a.nbp / 64;
  for (int c = 0; c < nchunks; ++c) {
    const int j = c * 64 + lane;
    const float s_hat = routing_scores(kt, a.nbp, c, qb_s, part, w, lane);
    const bool valid = j < a.nb;
    const bool sel = valid && (s_hat > tau_i || (j >= a.sink_b0 && j <= a.sink_b1));
    uint64_t selm = __ballot(sel);
    const uint64_t tailm = __ballot(valid) & ~selm;
    if (a.mask_out && tid == 0) a.mask_out[((size_t)bh * a.nb + i) * a.nbw + c] = selm;

    // ---- tail: groups of the unselected blocks of this chunk, against anchor w
    if (tailm) {
      float l0 = kNegInf, l1 = kNegInf;
      const size_t grow = ((size_t)bh * a.nbp + j) * 2;
      if ((tailm >> lane) & 1) {
        const uint4v* g0 = (const uint4v*)(a.gk + grow * kDim);
        float d0 = 0.f, d1 = 0.f;
#pragma unroll 4
        for (int cc = 0; cc < 16; ++cc) {
          const uint4v x0 = g0[cc], x1 = g0[16 + cc];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float q0 = qa_s[w][8 * cc + 2 * m], q1 = qa_s[w][8 * cc + 2 * m + 1];
            d0 += bf16_lo(x0[m]) * q0 + bf16_hi(x0[m]) * q1;
            d1 += bf16_lo(x1[m]) * q0 + bf16_hi(x1[m]) * q1;
          }
        }
        const float gl0 = a.glogn[grow], gl1 = a.glogn[grow + 1];
        l0 = gl0 == kNegInf ? kNegInf : (gl0 + d0 * kScale2) * kLog2e;
        l1 = gl1 == kNegInf ? kNegInf : (gl1 + d1 * kScale2) * kLog2e;
      }
      const float mc = wave_max(fmaxf(l0, l1));
      if (mc != kNegInf) {
        const float m_new = fmaxf(m_t, mc);
        const float sc = __builtin_amdgcn_exp2f(m_t - m_new);
        const float w0 = __builtin_amdgcn_exp2f(l0 - m_new), w1 = __builtin_amdgcn_exp2f(l1 - m_new);
        w_s[w][2 * lane] = w0;
        w_s[w][2 * lane + 1] = w1;
        z_t = z_t * sc + wave_sum(w0 + w1);
        m_t = m_new;
        tk0 *= sc; tk1 *= sc; tv0 *= sc; tv1 *= sc;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const uint32_t* gkc = (const uint32_t*)(a.gk + ((size_t)bh * a.nbp + c * 64) * 2 * kDim) + lane;
        const uint32_t* gvc = (const uint32_t*)(a.gv + ((size_t)bh * a.nbp + c * 64) * 2 * kDim) + lane;
        uint64_t tm = tailm;
        while (tm) {
          const int jj = __builtin_ctzll(tm);
          tm &= tm - 1;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const float wg = w_s[w][2 * jj + g];
            if (wg == 0.f) continue;
            const uint32_t kw = gkc[(2 * jj + g) * 64], vw = gvc[(2 * jj + g) * 64];
            tk0 += wg * bf16_lo(kw); tk1 += wg * bf16_hi(kw);
            tv0 += wg * bf16_lo(vw); tv1 += wg * bf16_hi(vw);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();

    // ---- exact blocks of this chunk: FP8 S^T, bf16 PV
    while (selm) {
      const int jb = c * 64 + __builtin_ctzll(selm);
      selm &= selm - 1;
      const int t0 = jb * kBlock;
      const int valid_rows = min(kBlock, a.N - t0);
      {
        // K8 tile: 64 rows x 128 B (rows >= N hold zero codes), 8 x 16 B per row
        const uint8_t* src = a.k8 + ((size_t)bh * a.tp + t0) * kDim;
        const int cc = tid & 7, r0 = tid >> 3;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = r0 + 16 * p;
          *(uint4v*)(K8s + r * kK8Stride + cc * 16) = *(const uint4v*)(src + (size_t)r * kDim + cc * 16);
        }
      }
      load_v_transposed(Vt, a.v + head_off + (size_t)t0 * rs, rs, valid_rows, tid);
      __syncthreads();
      const float f = sq * a.kscale[(size_t)bh * a.nbp + jb] * kScale2 * kLog2e;
      floatx16 s0 = {}, s1 = {};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const intx8 a0 = *(const intx8*)(K8s + l32 * kK8Stride + 64 * ks + 32 * kg);
        const intx8 a1 = *(const intx8*)(K8s + (32 + l32) * kK8Stride + 64 * ks + 32 * kg);
        s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[ks], s0, 0, 0, 0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[ks], s1, 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
        s0[idx] = key0 < valid_rows ? s0[idx] * f : kNegInf;
        s1[idx] = key0 + 32 < valid_rows ? s1[idx] * f : kNegInf;
      }
      softmax_pv(s0, s1, Vt, o, m_run, l_run, l32, kg);
      __syncthreads();
    }
  }

  // ---- tail finalisation: mu_a, nu_a, ln Z_a (log2), delta_t, Eq. (3)
  const float inv_z = z_t > 0.f ? 1.f / z_t : 0.f;
  mu_s[w][2 * lane] = tk0 * inv_z;
  mu_s[w][2 * lane + 1] = tk1 * inv_z;
  nu_s[w][2 * lane] = tv0 * inv_z;
  nu_s[w][2 * lane + 1] = tv1 * inv_z;
  const float qa_mu = wave_sum(qa_s[w][2 * lane] * tk0 * inv_z + qa_s[w][2 * lane + 1] * tk1 * inv_z);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const float lnz2 = z_t > 0.f ? m_t + __log2f(z_t) : kNegInf;
  // q'_t . mu over this lane's 64 dims (32 kg .. +31 and 64 + 32 kg .. +31), then with the partner
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
  const float lam2 = lnz2 == kNegInf ? kNegInf : lnz2 + (qmu - qa_mu) * kScale2 * kLog2e;
  const float m_fin = fmaxf(m_run, lam2);
  const float m_use = m_fin == kNegInf ? 0.f : m_fin;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  const float wt = __builtin_amdgcn_exp2f(lam2 - m_use);
  const float l_tot = sum_with_partner(l_run) * alpha + wt;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < a.N && a.out != nullptr) {
    uint16_t* dst = a.out + head_off + (size_t)qrow * rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * kg;
        float r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = (o[mt][4 * g + e] * alpha + wt * nu_s[w][d0 + e]) * inv;
        uint2v pk;
        pk[0] = pack_bf16x2(r4[0], r4[1]);
        pk[1] = pack_bf16x2(r4[2], r4[3]);
        *(uint2v*)(dst + d0) = pk;
      }
  }
}

hipError_t launch_fused2(const uint16_t* v, uint16_t* out, Shape s, const Workspace& ws, int sink_b0, int sink_b1,
                         uint64_t* mask_out, hipStream_t stream) {
  Fused2Args a;
  a.v = v; a.out = out;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = (ws.nb + 63) / 64; a.tp = ws.nbp * kBlock;
  a.q8 = ws.q8; a.k8 = ws.k8; a.qscale = ws.qscale; a.kscale = ws.kscale;
  a.qbar = ws.qbar; a.kbar_t = ws.kbar_t; a.tau_i = ws.tau_i; a.qanc = ws.qanc;
  a.gk = ws.gk; a.gv = ws.gv; a.glogn = ws.glogn;
  a.sink_b0 = sink_b0; a.sink_b1 = sink_b1; a.mask_out = mask_out;
  const int total = s.B * s.H * ws.nb;
  hipLaunchKernelGGL(sol2_fused_kernel, dim3(total), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace solattn
