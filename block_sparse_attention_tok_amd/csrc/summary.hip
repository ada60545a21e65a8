// Block summaries and the per-query-block threshold (Sol-Attn stage 1).
//
// Sol-Attn paper (arXiv 2607.24027) §3.2 "Hardware-Aligned Implementation":
// the fused kernel streams pooled keys KC[j] = K-bar_j (block means) and
// summed values VC[j] = V-hat_j; §2 Eq. (3) pools queries the same way.  §3.1
// Eqs. (4)-(5) and the appendix "Diagonal threshold estimator" give
// tau_i = mu_i + beta sigma_i from statistics of the pooled keys; §4.5 keeps
// only this threshold computation outside the attention kernel.
#include "common.h"
#include "kernels.h"

namespace solattn {

// Heads per workgroup of the summary pass: 4 heads (64 chunks, 4 token groups) put more
// workgroups in flight than one per block (measured 4 / 8 / 16 / 32: 291 / 297 / 307 / 305 us
// for prepare at 32768 tokens x 32 heads).
constexpr int kSummaryHeads = 4;
constexpr float kScaleR = 0.08838834764831845f;       // 1/sqrt(128)

// One workgroup per (64-token block j < nbp, batch b, group of hpw heads).  In
// BTHD the group's part of each token row is one contiguous span of hpw * 256
// bytes, so the reads are coalesced 16-byte loads; each thread owns 8 dims of one
// head (a 16-byte column chunk) and sums a subset of the block's tokens in fp32,
// the subsets meeting in LDS.  The same loads feed the head-major copies of K
// and V.
__global__ __launch_bounds__(256) void summary_kernel(
    const uint4v* __restrict__ q, const uint4v* __restrict__ k, const uint4v* __restrict__ v,
    int N, int H, int nb, int nbp, float* __restrict__ qbar, float* __restrict__ kbar_t,
    uint4v* __restrict__ kbar_h, uint4v* __restrict__ vbar_h, uint4v* __restrict__ kh_out,
    uint4v* __restrict__ vh_out, int hpw) {
  extern __shared__ float red[];
  const int j = blockIdx.x, b = blockIdx.y, h0 = blockIdx.z * hpw, tid = threadIdx.x;
  const int C = 16 * hpw;                               // 16-byte chunks of the group per token
  const int Cv = 16 * min(hpw, H - h0);                 // of heads that exist
  const int R = C >= 256 ? 1 : 256 / C;                 // token groups per chunk
  const int t0 = j * kBlock;
  const int n = j < nb ? min(kBlock, N - t0) : 0;
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
  const size_t rowc = (size_t)16 * H;                   // chunks per token row
  const size_t base = ((size_t)b * N + t0) * rowc + 16 * (size_t)h0;

  for (int cbase = 0; cbase < C; cbase += (R == 1 ? 256 : C)) {
    const int r = R == 1 ? 0 : tid / C;
    const int c = R == 1 ? cbase + tid : tid % C;
    const bool active = c < Cv && (R == 1 || r < R);
    float qs[8], ks[8], vs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[e] = ks[e] = vs[e] = 0.f;
    if (active) {
#pragma unroll 4
      for (int t = r; t < n; t += R) {
        const size_t off = base + (size_t)t * rowc + c;
        uint4v a = q[off], bb = k[off], cc = v[off];
        if (kh_out != nullptr) {   // head-major copies: head c / 16, dims 8 (c % 16) ..
          const size_t dst = (((size_t)b * H + h0 + c / 16) * N + t0 + t) * 16 + (c & 15);
          kh_out[dst] = bb;
          vh_out[dst] = cc;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          qs[2 * m] += bf16_lo(a[m]);  qs[2 * m + 1] += bf16_hi(a[m]);
          ks[2 * m] += bf16_lo(bb[m]); ks[2 * m + 1] += bf16_hi(bb[m]);
          vs[2 * m] += bf16_lo(cc[m]); vs[2 * m + 1] += bf16_hi(cc[m]);
        }
      }
    }
    if (R > 1) {
      if (active) {
        float* p = red + ((size_t)r * C + c) * 24;
#pragma unroll
        for (int e = 0; e < 8; ++e) { p[e] = qs[e]; p[8 + e] = ks[e]; p[16 + e] = vs[e]; }
      }
      __syncthreads();
      if (r == 0 && active) {
        for (int rr = 1; rr < R; ++rr) {
          const float* p = red + ((size_t)rr * C + c) * 24;
#pragma unroll
          for (int e = 0; e < 8; ++e) { qs[e] += p[e]; ks[e] += p[8 + e]; vs[e] += p[16 + e]; }
        }
      }
    }
    if (active && r == 0) {
      const int h = h0 + c / 16, d8 = c % 16;
      const size_t bh = (size_t)b * H + h;
      float4* qo = (float4*)(qbar + (bh * nbp + j) * kDim + 8 * d8);
      qo[0] = make_float4(qs[0] * inv_n, qs[1] * inv_n, qs[2] * inv_n, qs[3] * inv_n);
      qo[1] = make_float4(qs[4] * inv_n, qs[5] * inv_n, qs[6] * inv_n, qs[7] * inv_n);
      float kb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kb[e] = ks[e] * inv_n;
      float4* kt = (float4*)kbar_t;
      kt[(bh * 32 + 2 * d8) * nbp + j] = make_float4(kb[0], kb[1], kb[2], kb[3]);
      kt[(bh * 32 + 2 * d8 + 1) * nbp + j] = make_float4(kb[4], kb[5], kb[6], kb[7]);
      uint4v kh, vh;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        kh[m] = pack_bf16x2(kb[2 * m], kb[2 * m + 1]);
        vh[m] = pack_bf16x2(vs[2 * m] * inv_n, vs[2 * m + 1] * inv_n);
      }
      const size_t prow = bh * nbp + j;                       // [B][H][nbp][128]
      kbar_h[prow * 16 + d8] = kh;
      vbar_h[prow * 16 + d8] = vh;
    }
  }
}

hipError_t launch_summary(const uint16_t* q, const uint16_t* k, const uint16_t* v, Shape s,
                          const Workspace& ws, hipStream_t stream) {
  const int hpw = s.H < kSummaryHeads ? s.H : kSummaryHeads;
  const int C = 16 * hpw;
  const int R = C >= 256 ? 1 : 256 / C;
  const size_t lds = R > 1 ? (size_t)R * C * 24 * sizeof(float) : 0;
  dim3 grid(ws.nbp, s.B, (s.H + hpw - 1) / hpw);
  hipLaunchKernelGGL(summary_kernel, grid, dim3(256), lds, stream, (const uint4v*)q, (const uint4v*)k,
                     (const uint4v*)v, s.N, s.H, ws.nb, ws.nbp, ws.qbar, ws.kbar_t, (uint4v*)ws.kbar_h,
                     (uint4v*)ws.vbar_h, (uint4v*)ws.kh, (uint4v*)ws.vh, hpw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Routing (Sol-Attn paper §3.1, Eq. (6); Sol-Attn2 draft, Method, Eq. (1) selection):
// s-hat_ij = Q-bar_i . K-bar_j / sqrt(d) from the fp32 block means (for Sol-Attn2 of the
// dequantized values), against tau_i, with the blocks of a sink range forced exact.  One wave per (b, h, 32 query blocks from i0, 64-block chunk c): the 32 x 64
// products on v_mfma_f32_32x32x2_f32 (fp32 operands and sums), A = the query-block means,
// B = the key-block means, with the contraction order chosen so that lane (m, kh) reads
// dims 64 kh .. 64 kh + 63 of its row contiguously (k-step s takes dim 64 kh + s).  The
// accumulator of row i holds key blocks 32 t + n in lane n (+ 32 for rows i + 4), so one
// ballot per row pair gives the routing bits of two query blocks.
// ---------------------------------------------------------------------------
struct RouteArgs {
  int nb, nbp, nbw;
  const float* qbar; const float* kbar_t; const float* tau_i;
  int sink_b0, sink_b1;
  uint64_t* sel;
};

__global__ __launch_bounds__(64) void route_kernel(RouteArgs a) {
  const int c = blockIdx.x, i0 = blockIdx.y * 32, bh = blockIdx.z;
  const int lane = threadIdx.x, m = lane & 31, kh = lane >> 5;
  // rows i0 + m < nbp and key blocks 64 c + 63 < nbp: padding rows / blocks are in memory
  const float4* qa = (const float4*)(a.qbar + ((size_t)bh * a.nbp + i0 + m) * kDim) + 16 * kh;
  const float4* kb = (const float4*)a.kbar_t + ((size_t)bh * 32 + 16 * kh) * a.nbp + 64 * c + m;
  floatx16 acc[2] = {floatx16{}, floatx16{}};               // key blocks 64 c + 32 t + n
#pragma unroll 4
  for (int cc = 0; cc < 16; ++cc) {
    const float4 x = qa[cc];
    const float4 y0 = kb[(size_t)cc * a.nbp];
    const float4 y1 = kb[(size_t)cc * a.nbp + 32];
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y0.x, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y1.x, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y0.y, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y1.y, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y0.z, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y1.z, acc[1], 0, 0, 0);
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y0.w, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y1.w, acc[1], 0, 0, 0);
  }
  const bool sink[2] = {64 * c + m >= a.sink_b0 && 64 * c + m <= a.sink_b1,
                        64 * c + 32 + m >= a.sink_b0 && 64 * c + 32 + m <= a.sink_b1};
  const bool kvalid[2] = {64 * c + m < a.nb, 64 * c + 32 + m < a.nb};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * kh + (r & 3);     // this lane's query block in row r
    const float tau = a.tau_i[(size_t)bh * a.nbp + i];
    uint64_t bits[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float s_hat = acc[t][r] * kScaleR;
      bits[t] = __ballot(i < a.nb && kvalid[t] && (s_hat > tau || sink[t]));
    }
    if (lane == 0) {
      const int ilo = i0 + 8 * (r >> 2) + (r & 3);          // rows ilo (lanes 0..31) and ilo + 4
      const uint64_t wlo = (bits[1] << 32) | (bits[0] & 0xffffffffull);
      const uint64_t whi = (bits[1] & 0xffffffff00000000ull) | (bits[0] >> 32);
      if (ilo < a.nb) a.sel[((size_t)bh * a.nb + ilo) * a.nbw + c] = wlo;
      if (ilo + 4 < a.nb) a.sel[((size_t)bh * a.nb + ilo + 4) * a.nbw + c] = whi;
    }
  }
}

hipError_t launch_route(Shape s, const Workspace& ws, int sink_b0, int sink_b1, uint64_t* sel,
                        hipStream_t stream) {
  RouteArgs r;
  r.nb = ws.nb; r.nbp = ws.nbp; r.nbw = ws.nbp / 64;
  r.qbar = ws.qbar; r.kbar_t = ws.kbar_t; r.tau_i = ws.tau_i;
  r.sink_b0 = sink_b0; r.sink_b1 = sink_b1;
  r.sel = sel;
  hipLaunchKernelGGL(route_kernel, dim3(ws.nbp / 64, (ws.nb + 31) / 32, s.B * s.H), dim3(64), 0, stream, r);
  return hipGetLastError();
}

// One workgroup per (batch, head).  mu_K and v_K are averages over the nb key
// blocks with weight 1/nb; v_K is accumulated in the centred two-pass form
// mean_j (K-bar_j - mu_K)^2, which equals the printed mean of squares minus the
// squared mean.  tau_i = mu_i + tau sigma_i in scaled-logit units (1/sqrt d).
// exact != 0 uses the full covariance (Eq. (5)): sigma_i^2 = Q-bar_i Cov Q-bar_i^T.
__global__ __launch_bounds__(256) void threshold_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar_t, int nb, int nbp, float tau,
    int exact, float* __restrict__ kstat, float* __restrict__ kcov, float* __restrict__ tau_i) {
  __shared__ float s_mu[kDim], s_var[kDim], s_part[256];
  __shared__ float s_chunk[32][kDim];                   // 32 centred key means, for the covariance
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int d = tid & 127, half = tid >> 7;
  const float* kt = kbar_t + (size_t)bh * 32 * nbp * 4;
  auto kval = [&](int jj, int dd) { return kt[((size_t)(dd >> 2) * nbp + jj) * 4 + (dd & 3)]; };

  float acc = 0.f;
  for (int jj = half; jj < nb; jj += 2) acc += kval(jj, d);
  s_part[tid] = acc;
  __syncthreads();
  if (tid < kDim) s_mu[tid] = (s_part[tid] + s_part[tid + 128]) / (float)nb;
  __syncthreads();
  const float mu = s_mu[d];
  acc = 0.f;
  for (int jj = half; jj < nb; jj += 2) { float x = kval(jj, d) - mu; acc += x * x; }
  s_part[tid] = acc;
  __syncthreads();
  if (tid < kDim) {
    s_var[tid] = (s_part[tid] + s_part[tid + 128]) / (float)nb;
    kstat[(size_t)bh * 256 + tid] = s_mu[tid];
    kstat[(size_t)bh * 256 + 128 + tid] = s_var[tid];
  }
  __syncthreads();

  float* cov = kcov + (size_t)bh * kDim * kDim;
  if (exact) {
    // thread owns row r = tid / 2 and 64 columns starting at 64 * (tid % 2)
    const int r = tid >> 1, c0 = (tid & 1) * 64;
    float cacc[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) cacc[e] = 0.f;
    for (int j0 = 0; j0 < nb; j0 += 32) {
      __syncthreads();
      for (int idx = tid; idx < 32 * kDim; idx += 256) {
        int jj = j0 + idx / kDim, dd = idx % kDim;
        s_chunk[idx / kDim][dd] = jj < nb ? kval(jj, dd) - s_mu[dd] : 0.f;
      }
      __syncthreads();
      for (int jj = 0; jj < 32; ++jj) {
        const float xr = s_chunk[jj][r];
#pragma unroll
        for (int e = 0; e < 64; ++e) cacc[e] += xr * s_chunk[jj][c0 + e];
      }
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) cov[(size_t)r * kDim + c0 + e] = cacc[e] / (float)nb;
    __threadfence_block();
    __syncthreads();
  }

  const float scale = 0.08838834764831845f;             // 1/sqrt(128)
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = wave; i < nb; i += 4) {
    const float* qi = qbar + ((size_t)bh * nbp + i) * kDim;
    const float q0 = qi[lane], q1 = qi[lane + 64];
    float m = q0 * s_mu[lane] + q1 * s_mu[lane + 64];
    float var;
    if (exact) {
      // (Cov q)[lane] and [lane + 64], then q . (Cov q)
      float c0 = 0.f, c1 = 0.f;
      for (int e = 0; e < kDim; ++e) {
        const float qe = qi[e];
        c0 += cov[(size_t)lane * kDim + e] * qe;
        c1 += cov[(size_t)(lane + 64) * kDim + e] * qe;
      }
      var = q0 * c0 + q1 * c1;
    } else {
      var = q0 * q0 * s_var[lane] + q1 * q1 * s_var[lane + 64];
    }
    m = wave_sum(m);
    var = wave_sum(var);
    if (lane == 0) {
      const float sigma = sqrtf(fmaxf(var, 0.f)) * scale;
      tau_i[(size_t)bh * nbp + i] = m * scale + tau * sigma;
    }
  }
}

// Diagonal threshold in two wide passes (the single-workgroup-per-head kernel
// above is latency-bound on long sequences).  Pass 1: per (b, h, slice of key
// blocks) the sums of K-bar_j and K-bar_j (.) K-bar_j in fp64.  Pass 2: mu_K and
// v_K = mean of squares - squared mean (the printed estimator, in fp64), then
// tau_i for 32 query blocks per workgroup.
constexpr int kStatSlices = 16;

__global__ __launch_bounds__(256) void kstat_partial_kernel(const float* __restrict__ kbar_t, int nb, int nbp,
                                                            double* __restrict__ part) {
  __shared__ double s_sum[2][kDim], s_sq[2][kDim];
  const int bh = blockIdx.x, sl = blockIdx.y, tid = threadIdx.x;
  const int d = tid & 127, half = tid >> 7;
  const int per = (nb + kStatSlices - 1) / kStatSlices;
  const int j0 = sl * per, j1 = min(nb, j0 + per);
  const float* kt = kbar_t + (size_t)bh * 32 * nbp * 4 + (size_t)(d >> 2) * nbp * 4 + (d & 3);
  double a = 0.0, q = 0.0;
  for (int jj = j0 + half; jj < j1; jj += 2) {
    const double x = kt[(size_t)jj * 4];
    a += x;
    q += x * x;
  }
  s_sum[half][d] = a;
  s_sq[half][d] = q;
  __syncthreads();
  if (tid < kDim) {
    double* o = part + ((size_t)bh * kStatSlices + sl) * 2 * kDim;
    o[tid] = s_sum[0][tid] + s_sum[1][tid];
    o[kDim + tid] = s_sq[0][tid] + s_sq[1][tid];
  }
}

__global__ __launch_bounds__(256) void tau_diag_kernel(const double* __restrict__ part, const float* __restrict__ qbar,
                                                       int nb, int nbp, float tau, float* __restrict__ kstat,
                                                       float* __restrict__ tau_i) {
  __shared__ float s_mu[kDim], s_var[kDim];
  const int bh = blockIdx.x, tid = threadIdx.x;
  if (tid < kDim) {
    double a = 0.0, q = 0.0;
    const double* p = part + (size_t)bh * kStatSlices * 2 * kDim;
    for (int sl = 0; sl < kStatSlices; ++sl) { a += p[sl * 2 * kDim + tid]; q += p[sl * 2 * kDim + kDim + tid]; }
    const double mu = a / nb;
    const float var = (float)(q / nb - mu * mu);
    s_mu[tid] = (float)mu;
    s_var[tid] = var;
    if (blockIdx.y == 0) {
      kstat[(size_t)bh * 256 + tid] = (float)mu;
      kstat[(size_t)bh * 256 + 128 + tid] = var;
    }
  }
  __syncthreads();
  const float scale = 0.08838834764831845f;             // 1/sqrt(128)
  const int wave = tid >> 6, lane = tid & 63;
  const int i0 = blockIdx.y * 32 + wave * 8;
  for (int i = i0; i < min(nb, i0 + 8); ++i) {
    const float* qi = qbar + ((size_t)bh * nbp + i) * kDim;
    const float q0 = qi[lane], q1 = qi[lane + 64];
    float m = q0 * s_mu[lane] + q1 * s_mu[lane + 64];
    float var = q0 * q0 * s_var[lane] + q1 * q1 * s_var[lane + 64];
    m = wave_sum(m);
    var = wave_sum(var);
    if (lane == 0) tau_i[(size_t)bh * nbp + i] = m * scale + tau * sqrtf(fmaxf(var, 0.f)) * scale;
  }
}

hipError_t launch_threshold(Shape s, const Workspace& ws, float tau, int exact, hipStream_t stream) {
  if (exact) {
    hipLaunchKernelGGL(threshold_kernel, dim3(s.B * s.H), dim3(256), 0, stream, ws.qbar, ws.kbar_t, ws.nb,
                       ws.nbp, tau, exact, ws.kstat, ws.kcov, ws.tau_i);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kstat_partial_kernel, dim3(s.B * s.H, kStatSlices), dim3(256), 0, stream, ws.kbar_t, ws.nb,
                     ws.nbp, ws.kpart);
  hipLaunchKernelGGL(tau_diag_kernel, dim3(s.B * s.H, (ws.nb + 31) / 32), dim3(256), 0, stream, ws.kpart, ws.qbar,
                     ws.nb, ws.nbp, tau, ws.kstat, ws.tau_i);
  return hipGetLastError();
}

}  // namespace solattn
