// Fused Sol-Attn forward kernel for gfx950 (Sol-Attn stage 2).
//
// Sol-Attn paper (arXiv 2607.24027) §3.2, Figure 4 and "Hardware-Aligned
// Implementation": each program keeps one query block and its threshold
// tau_i on chip and one online-softmax state in registers; an outer loop
// streams chunks of pooled keys / values, compares each block's proxy score
// s_ij = Q-bar_i . K-bar_j / sqrt(d) with tau_i (Eq. (4), Eq. (6)), folds every
// unselected block in through its proxy (token-to-block tile Q_i K-bar^T with
// weight n_j and the V sum V-hat_j), and an inner loop runs exact attention on
// the original K/V blocks of the selected indices.  No proxy or routing map is
// written to memory (only the optional test export below).
//
// gfx950 mapping (one workgroup = one (batch, head, 64-row query block),
// two wave64s of 32 query rows each):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K tile rows from LDS,
//     B = the wave's 32 query rows held in registers.  The accumulator puts
//     one query per lane (lane % 32) and 16 keys per lane, so the row max and
//     row sum are in-lane plus one v_permlane32_swap with the partner lane.
//   * O^T += V^T P^T on the same MFMA: A = V^T read from a transposed LDS
//     copy, B = P taken straight from the S^T accumulator (the k order inside
//     one MFMA is permuted consistently on both operands), so O^T also keeps
//     one query per lane and the softmax rescale is a per-lane multiply.
//   * A proxy chunk is the same tile computation with K-bar / V-bar (V-hat_j/n_j)
//     as keys / values and an additive log2(n_j) logit bias, selected and
//     padding columns masked to -inf: sum_u e^{q.K-bar} v_u style algebra,
//     n_j e^{q.K-bar_j} V-bar_j = e^{q.K-bar_j} V-hat_j, shares the softmax state.
//   * Routing dot products run in fp32 from fp32 block means (VALU), so the
//     selection does not depend on bf16 rounding of the pooled keys.
#include "common.h"
#include "kernels.h"
#include "tile.h"

namespace solattn {

constexpr int kKsStride = 272;   // bytes per K row in LDS: 256 + 16 pad (conflict-free b128 reads)
constexpr float kScale = 0.08838834764831845f;        // 1/sqrt(128)
constexpr float kScaleLog2 = kScale * kLog2e;

struct FusedArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; uint16_t* out;
  int B, N, H, nb, nbp, nbw;
  const float* qbar; const float* kbar_t; const uint16_t* kbar_h; const uint16_t* vbar_h;
  const float* tau_i;
  int sink_b0, sink_b1;
  uint64_t* mask_out;
};

// Stage a 64-row K tile (row-major) and V tile (transposed) into LDS.
// Rows r >= valid are zero-filled.  `stride` is the element distance between
// consecutive rows in global memory.
__device__ __forceinline__ void load_tile(unsigned char* Ks, unsigned char* Vt, const uint16_t* kb,
                                          const uint16_t* vb, size_t stride, int valid, int tid) {
  // K: thread owns 16-byte chunk cc of rows r0, r0 + 8, ...
  const int cc = tid & 15, r0 = tid >> 4;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = r0 + 8 * p;
    uint4v x = {0u, 0u, 0u, 0u};
    if (r < valid) x = *(const uint4v*)(kb + (size_t)r * stride + cc * 8);
    *(uint4v*)(Ks + r * kKsStride + cc * 16) = x;
  }
  load_v_transposed(Vt, vb, stride, valid, tid);
}

enum TileMode { kExactFull = 0, kExactPartial = 1, kProxy = 2 };

// One 64-key tile against the wave's 32 query rows: S^T, online softmax, O^T += V^T P^T.
// kProxy: key r carries bias log2(n_j) when bit r of `colmask` is set, else -inf.
// kExactPartial: keys r >= `valid` are masked.
template <int MODE>
__device__ __forceinline__ void process_tile(const unsigned char* Ks, const unsigned char* Vt,
                                             const bf16x8 (&qreg)[8], floatx16 (&o)[4], float& m_run,
                                             float& l_run, uint64_t colmask, int valid, float last_bias,
                                             int last_key, int l32, int kg) {
  floatx16 s0 = {}, s1 = {};
  const unsigned char* k0 = Ks + l32 * kKsStride + kg * 16;
  const unsigned char* k1 = Ks + (32 + l32) * kKsStride + kg * 16;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    bf16x8 a0 = *(const bf16x8*)(k0 + ks * 32);
    bf16x8 a1 = *(const bf16x8*)(k1 + ks * 32);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
  }
  // logits in log2 units; element idx of tile mt holds key 32 mt + 8 (idx/4) + 4 kg + idx%4
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) {
    const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
    float x0 = s0[idx] * kScaleLog2, x1 = s1[idx] * kScaleLog2;
    if (MODE == kProxy) {
      const float b0 = key0 == last_key ? last_bias : 6.0f;        // log2(64) for full blocks
      const float b1 = key0 + 32 == last_key ? last_bias : 6.0f;
      x0 = ((colmask >> key0) & 1) ? x0 + b0 : kNegInf;
      x1 = ((colmask >> (key0 + 32)) & 1) ? x1 + b1 : kNegInf;
    } else if (MODE == kExactPartial) {
      if (key0 >= valid) x0 = kNegInf;
      if (key0 + 32 >= valid) x1 = kNegInf;
    }
    s0[idx] = x0;
    s1[idx] = x1;
  }
  softmax_pv(s0, s1, Vt, o, m_run, l_run, l32, kg);
}

template <bool kExport>
__global__ __launch_bounds__(128) void sol_fused_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[64 * kKsStride];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[128 * kVtStride];
  __shared__ __attribute__((aligned(16))) float qb_s[kDim];
  __shared__ float part[2][64];

  const int total = a.B * a.H * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  const int i = item % a.nb;
  const int bh = item / a.nb;
  const int h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const size_t rs = (size_t)a.H * kDim;                      // elements between tokens (BTHD)
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;

  if (tid < 32) ((float4*)qb_s)[tid] = ((const float4*)(a.qbar + ((size_t)bh * a.nbp + i) * kDim))[tid];
  const float tau_i = a.tau_i[(size_t)bh * a.nbp + i];

  const int qrow = i * kBlock + w * 32 + l32;
  bf16x8 qreg[8];
  if (qrow < a.N) {
    const uint4v* src = (const uint4v*)(a.q + head_off + (size_t)qrow * rs);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, src[2 * ks + kg]);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, uint4v{0u, 0u, 0u, 0u});
  }

  floatx16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  const int last_n = a.N - (a.nb - 1) * kBlock;               // valid tokens of the last block
  const float last_bias = __log2f((float)last_n);
  __syncthreads();

  const float4* kt = (const float4*)a.kbar_t + (size_t)bh * 32 * a.nbp;
  const size_t pooled_off = (size_t)bh * a.nbp * kDim;
  const int nchunks = a.nbp / 64;
  for (int c = 0; c < nchunks; ++c) {
    // ---- routing: s_ij for the 64 pooled keys of this chunk (fp32)
    const int j = c * 64 + lane;
    const float s_hat = routing_scores(kt, a.nbp, c, qb_s, part, w, lane);
    const bool valid = j < a.nb;
    const bool sel = valid && (s_hat > tau_i || (j >= a.sink_b0 && j <= a.sink_b1));
    uint64_t selm = __ballot(sel);
    const uint64_t proxym = __ballot(valid) & ~selm;
    if (kExport && tid == 0) a.mask_out[((size_t)bh * a.nb + i) * a.nbw + c] = selm;

    // ---- proxy update for the unselected blocks of the chunk
    if (proxym) {
      load_tile(Ks, Vt, a.kbar_h + pooled_off + (size_t)c * 64 * kDim,
                a.vbar_h + pooled_off + (size_t)c * 64 * kDim, kDim, 64, tid);
      __syncthreads();
      process_tile<kProxy>(Ks, Vt, qreg, o, m_run, l_run, proxym, 64, last_bias, a.nb - 1 - c * 64,
                           l32, kg);
    }
    __syncthreads();

    // ---- exact update for the selected blocks of the chunk
    while (selm) {
      const int jb = c * 64 + __builtin_ctzll(selm);
      selm &= selm - 1;
      const int t0 = jb * kBlock;
      const int valid_rows = min(kBlock, a.N - t0);
      load_tile(Ks, Vt, a.k + head_off + (size_t)t0 * rs, a.v + head_off + (size_t)t0 * rs, rs,
                valid_rows, tid);
      __syncthreads();
      if (valid_rows == kBlock)
        process_tile<kExactFull>(Ks, Vt, qreg, o, m_run, l_run, 0, kBlock, 0.f, -1, l32, kg);
      else
        process_tile<kExactPartial>(Ks, Vt, qreg, o, m_run, l_run, 0, valid_rows, 0.f, -1, l32, kg);
      __syncthreads();
    }
  }

  // ---- epilogue: O / l, bf16 RNE, BTHD store
  const float l_tot = sum_with_partner(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < a.N && a.out != nullptr) {
    uint16_t* dst = a.out + head_off + (size_t)qrow * rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2v pk;
        pk[0] = pack_bf16x2(o[mt][4 * g] * inv, o[mt][4 * g + 1] * inv);
        pk[1] = pack_bf16x2(o[mt][4 * g + 2] * inv, o[mt][4 * g + 3] * inv);
        *(uint2v*)(dst + 32 * mt + 8 * g + 4 * kg) = pk;
      }
  }
}

hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                        Shape s, const Workspace& ws, int sink_b0, int sink_b1, uint64_t* mask_out,
                        hipStream_t stream) {
  FusedArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = (ws.nb + 63) / 64;
  a.qbar = ws.qbar; a.kbar_t = ws.kbar_t; a.kbar_h = ws.kbar_h; a.vbar_h = ws.vbar_h; a.tau_i = ws.tau_i;
  a.sink_b0 = sink_b0; a.sink_b1 = sink_b1; a.mask_out = mask_out;
  const int total = s.B * s.H * ws.nb;
  if (mask_out)
    hipLaunchKernelGGL(sol_fused_kernel<true>, dim3(total), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL(sol_fused_kernel<false>, dim3(total), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace solattn
