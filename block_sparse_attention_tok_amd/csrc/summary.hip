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

// Full-covariance threshold (§3.1 Eq. (5)): sigma_i^2 = Q-bar_i Cov Q-bar_i^T with
// Cov = mean_j (K-bar_j - mu_K)(K-bar_j - mu_K)^T, the centred form of the printed
// second moment minus the squared mean.  Three wide passes after the fp64 sums of pass 1:
//   cov_partial_kernel  per (b, h, slice of key blocks): the slice's centred outer
//                       products, one 8 x 8 tile of the 128 x 128 sum per thread;
//   cov_reduce_kernel   per (b, h, 8 rows): the slices summed, / nb, into kcov (and kstat);
//   tau_cov_kernel      per (b, h, 32 query blocks): Cov in LDS, y = Cov Q-bar_i^T with
//                       lanes reading Cov's rows contiguously (Cov is symmetric), then
//                       tau_i = mu_i + tau sigma_i.
constexpr int kCovSlices = 8;

// mu_K (fp32) of (b, h) from the fp64 slice sums of kstat_partial_kernel, for dim d.
__device__ __forceinline__ float mean_from_part(const double* __restrict__ part, size_t bh, int d, int nb) {
  double a = 0.0;
  const double* p = part + bh * kStatSlices * 2 * kDim;
  for (int sl = 0; sl < kStatSlices; ++sl) a += p[sl * 2 * kDim + d];
  return (float)(a / nb);
}

__global__ __launch_bounds__(256) void cov_partial_kernel(const float* __restrict__ kbar_t, const double* __restrict__ part,
                                                          int nb, int nbp, float* __restrict__ covp) {
  __shared__ float s_mu[kDim];
  __shared__ __attribute__((aligned(16))) float s_x[32][kDim + 4];
  const int bh = blockIdx.x, sl = blockIdx.y, tid = threadIdx.x;
  if (tid < kDim) s_mu[tid] = mean_from_part(part, bh, tid, nb);
  const int per = (nb + kCovSlices - 1) / kCovSlices;
  const int j0 = sl * per, j1 = min(nb, j0 + per);
  const int ti = tid >> 4, tj = tid & 15;                // rows 8 ti .., columns 8 tj ..
  const float* kt = kbar_t + (size_t)bh * 32 * nbp * 4;
  float acc[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  for (int c0 = j0; c0 < j1; c0 += 32) {
    __syncthreads();                                     // s_mu written; previous chunk consumed
    for (int e = tid; e < 32 * kDim; e += 256) {
      const int r = e >> 7, d = e & (kDim - 1), j = c0 + r;
      s_x[r][d] = j < j1 ? kt[((size_t)(d >> 2) * nbp + j) * 4 + (d & 3)] - s_mu[d] : 0.f;
    }
    __syncthreads();
    const int rows = min(32, j1 - c0);
    for (int r = 0; r < rows; ++r) {
      const float4 a0 = *(const float4*)&s_x[r][8 * ti], a1 = *(const float4*)&s_x[r][8 * ti + 4];
      const float4 b0 = *(const float4*)&s_x[r][8 * tj], b1 = *(const float4*)&s_x[r][8 * tj + 4];
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y) acc[x][y] = __builtin_fmaf(av[x], bv[y], acc[x][y]);
    }
  }
  float* dst = covp + ((size_t)bh * kCovSlices + sl) * kDim * kDim;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    float* row = dst + (size_t)(8 * ti + x) * kDim + 8 * tj;
    *(float4*)row = make_float4(acc[x][0], acc[x][1], acc[x][2], acc[x][3]);
    *(float4*)(row + 4) = make_float4(acc[x][4], acc[x][5], acc[x][6], acc[x][7]);
  }
}

__global__ __launch_bounds__(256) void cov_reduce_kernel(const float* __restrict__ covp, const double* __restrict__ part,
                                                         int nb, float* __restrict__ kcov, float* __restrict__ kstat) {
  const int bh = blockIdx.x, rb = blockIdx.y, tid = threadIdx.x;
  const size_t e = (size_t)rb * 8 * kDim + 4 * tid;      // 4 consecutive entries of rows 8 rb ..
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sl = 0; sl < kCovSlices; ++sl) {
    const float4 x = *(const float4*)(covp + ((size_t)bh * kCovSlices + sl) * kDim * kDim + e);
    s.x += x.x; s.y += x.y; s.z += x.z; s.w += x.w;
  }
  const float inv = 1.0f / (float)nb;
  s.x *= inv; s.y *= inv; s.z *= inv; s.w *= inv;
  *(float4*)(kcov + (size_t)bh * kDim * kDim + e) = s;
  // kstat: mu_K (first row block) and the diagonal of Cov
  if (rb == 0 && tid < kDim) kstat[(size_t)bh * 256 + tid] = mean_from_part(part, bh, tid, nb);
  const int r = (int)(e / kDim), c = (int)(e % kDim);
  if (c <= r && r < c + 4) kstat[(size_t)bh * 256 + kDim + r] = r == c ? s.x : r == c + 1 ? s.y : r == c + 2 ? s.z : s.w;
}

__global__ __launch_bounds__(256) void tau_cov_kernel(const float* __restrict__ kcov, const float* __restrict__ kstat,
                                                      const float* __restrict__ qbar, int nb, int nbp, float tau,
                                                      float* __restrict__ tau_i) {
  __shared__ __attribute__((aligned(16))) float s_c[kDim * kDim];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* cv = kcov + (size_t)bh * kDim * kDim;
  for (int e = 4 * tid; e < kDim * kDim; e += 1024) *(float4*)&s_c[e] = *(const float4*)(cv + e);
  __syncthreads();
  const float scale = 0.08838834764831845f;             // 1/sqrt(128)
  const int wave = tid >> 6, lane = tid & 63;
  const float mu0 = kstat[(size_t)bh * 256 + lane], mu1 = kstat[(size_t)bh * 256 + lane + 64];
  const int i0 = blockIdx.y * 32 + wave * 8;
  for (int i = i0; i < min(nb, i0 + 8); ++i) {
    const float* qi = qbar + ((size_t)bh * nbp + i) * kDim;
    const float q0 = qi[lane], q1 = qi[lane + 64];
    float y0 = 0.f, y1 = 0.f;                            // (Cov q)[lane], [lane + 64]
#pragma unroll 8
    for (int e = 0; e < kDim; ++e) {
      const float qe = qi[e];                            // uniform: one scalar load per dim
      y0 = __builtin_fmaf(s_c[e * kDim + lane], qe, y0);
      y1 = __builtin_fmaf(s_c[e * kDim + lane + 64], qe, y1);
    }
    const float m = wave_sum(q0 * mu0 + q1 * mu1);
    const float var = wave_sum(q0 * y0 + q1 * y1);
    if (lane == 0) tau_i[(size_t)bh * nbp + i] = m * scale + tau * sqrtf(fmaxf(var, 0.f)) * scale;
  }
}

hipError_t launch_threshold(Shape s, const Workspace& ws, float tau, int exact, hipStream_t stream) {
  hipLaunchKernelGGL(kstat_partial_kernel, dim3(s.B * s.H, kStatSlices), dim3(256), 0, stream, ws.kbar_t, ws.nb,
                     ws.nbp, ws.kpart);
  if (exact) {
    if (!ws.kcovp) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cov_partial_kernel, dim3(s.B * s.H, kCovSlices), dim3(256), 0, stream, ws.kbar_t, ws.kpart,
                       ws.nb, ws.nbp, ws.kcovp);
    hipLaunchKernelGGL(cov_reduce_kernel, dim3(s.B * s.H, kDim / 8), dim3(256), 0, stream, ws.kcovp, ws.kpart, ws.nb,
                       ws.kcov, ws.kstat);
    hipLaunchKernelGGL(tau_cov_kernel, dim3(s.B * s.H, (ws.nb + 31) / 32), dim3(256), 0, stream, ws.kcov, ws.kstat,
                       ws.qbar, ws.nb, ws.nbp, tau, ws.tau_i);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(tau_diag_kernel, dim3(s.B * s.H, (ws.nb + 31) / 32), dim3(256), 0, stream, ws.kpart, ws.qbar,
                     ws.nb, ws.nbp, tau, ws.kstat, ws.tau_i);
  return hipGetLastError();
}

}  // namespace solattn
