// Sol-Attn backward pass with the forward's routing held fixed, for gfx950.
//
// What is differentiated: the Sol-Attn output (paper arXiv 2607.24027, §3.2
// "Proxy-Score Reuse as Approximate Correction") with the block masks treated
// as constants, as the Sol-Attn2 draft (Method, Stage A1 passage) fixes for its
// training: gradients reach Q, K and V through the exact tokens, the pooled
// keys and the shared normalization.  With V-hat_j = n_j V-bar_j the forward is
// one softmax over an augmented key set -- the tokens of the exact blocks and
// one pooled key K-bar_j per unselected block with logit bias ln n_j and value
// V-bar_j -- so its backward is the softmax backward
//     P = 2^(x - lse),  dS = P (dO . value - D),  D = dO . O,
//     dq += dS key / sqrt(d),  dkey += dS^T q / sqrt(d),  dvalue += P^T dO,
// and the pooled keys / values pass 1/n_j of their gradient to every token of
// their block (they are block means).
//
// Kernels (one stream, in order):
//   bwd_init_kernel       D per query row next to the forward's lse, padding rows
//                         (lse = +inf), zeroed pooled-key gradients;
//   bwd_transpose_kernel  the routing bits by key block (which query blocks chose j);
//   bwd_kv_kernel<true>   pooled keys: one workgroup per (b, h, 64 pooled keys, query
//                         range) over the query blocks that did not select them;
//                         fp32 atomics into dkbar / dvbar;
//   bwd_kv_kernel<false>  exact keys: one workgroup per (b, h, key block j) over the
//                         query blocks that selected j; adds dkbar_j / n_j, dvbar_j / n_j;
//   bwd_dq_kernel         one workgroup per (b, h, query block) over the forward's tile
//                         stream (pooled tiles and exact blocks).
// Tiles move HBM -> LDS by buffer DMA into double buffers whose 16-byte slots use a
// swizzle that keeps both the row reads (b128) and the transposed reads
// (ds_read_b64_tr_b16) free of bank conflicts; every product is a 32x32x16 bf16 MFMA
// with fp32 accumulation, P and dS entering the MFMA as bf16 straight from the score
// accumulator (the same k-order trick as the forward's PV product).
#include "common.h"
#include "kernels.h"
#include "pipe.h"

namespace solattn {

namespace {

constexpr float kScaleB = 0.08838834764831845f;        // 1/sqrt(128)
constexpr float kScaleLog2B = kScaleB * kLog2e;
constexpr int kMaxChunksB = 128;
constexpr int kEndB = -0x7fffffff;
constexpr int kMaxRange = 512;                          // query blocks per pooled-key workgroup

struct BwdArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* out; const uint16_t* dout;
  uint16_t* dq; uint16_t* dk; uint16_t* dv;
  int B, N, H, nb, nbp, nbw, tp;
  const uint16_t* kbar_h; const uint16_t* vbar_h;   // [B][H][nbp][128]
  const uint16_t* kh; const uint16_t* vh;           // head-major copies of k and v ([B][H][N][128])
  const float* lse;
  const uint64_t* mrow; uint64_t* mcol;
  float* ld;
  float* dkbar; float* dvbar;
  int nrange, bpr;            // pooled-key kernel: query ranges per chunk, query blocks per range
};

// Slot swizzle of a 64 x 256-byte tile that is read both by rows (16 consecutive rows,
// one logical chunk: 16 distinct slots) and transposed (4 consecutive rows x 4 chunks:
// 16 distinct slots).
__device__ __forceinline__ int swz_d(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct DmaOffsetsD {
  uint32_t o[4];
};

// Wave w, instruction n fills rows 32 w + 4 n + lane / 16, slot lane % 16 (see dma_tile).
__device__ __forceinline__ DmaOffsetsD dma_offsets_d(uint32_t row_bytes, int w, int lane) {
  const int row = 32 * w + (lane >> 4);
  DmaOffsetsD d;
#pragma unroll
  for (int n = 0; n < 4; ++n) d.o[n] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_d(row + 4 * n)) << 4);
  return d;
}

__device__ __forceinline__ void dma_tile_d(unsigned char* lds, __amdgpu_buffer_rsrc_t rsrc, uint32_t tile_off,
                                           uint32_t row_bytes, const DmaOffsetsD& off, int w) {
#pragma unroll
  for (int n = 0; n < 8; ++n)
    dma16_buf(rsrc, off.o[n & 3] + tile_off + (uint32_t)n * 4 * row_bytes, 0, lds + (w * 8 + n) * 1024);
}

// Row-read offsets: A operand row 32 mt + l32 (mt adds 32 rows, same swizzle), k-step ks
// reads logical chunk 2 ks + kg.
__device__ __forceinline__ void row_offsets(int lane, int (&roff)[8]) {
  const int l32 = lane & 31, kg = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) roff[ks] = l32 * 256 + 16 * ((2 * ks + kg) ^ swz_d(l32));
}

// Transposed-read offsets (A operand = tile^T, 128 columns x 64 rows): as the forward's V^T
// read, lane group G = lane / 16, i' = lane % 16 addresses row 4 kg + i'/4 (+ 8 for the upper
// half, + 16 st per k-step) and logical chunk 4 mt + 2 (G % 2) + (i' % 4) / 2.
__device__ __forceinline__ void tr_offsets(int lane, int (&toff)[4][2]) {
  const int ip = lane & 15, gm = (lane >> 4) & 1, kg = lane >> 5;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 4 * kg + (ip >> 2) + 8 * half;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int lc = 4 * mt + 2 * gm + ((ip & 3) >> 1);
      toff[mt][half] = row * 256 + 16 * (lc ^ swz_d(row)) + (ip & 1) * 8;
    }
  }
}

// acc (tile^T x B): acc[mt] += tile^T[32 mt .. 32 mt + 31][rows] x B[rows][32 columns], the
// B fragments pb[st] holding rows 16 st + 8 (e / 4) + 4 kg + e % 4 of the lane's column.
__device__ __forceinline__ void tr_product(floatx16 (&acc)[4], const unsigned char* L, const int (&toff)[4][2],
                                           const bf16x8 (&pb)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint2v lo = lds_read_tr16(L + toff[mt][0] + st * 16 * 256);
      const uint2v hi = lds_read_tr16(L + toff[mt][1] + st * 16 * 256);
      const uint4v av = {lo[0], lo[1], hi[0], hi[1]};
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[st], acc[mt], 0, 0, 0);
    }
  }
}

// s0 / s1 = rows 0..31 / 32..63 of the tile at L times the register fragments breg (the
// lane's column): s[idx] is row 8 (idx / 4) + 4 kg + idx % 4 (+ 32 for s1).
__device__ __forceinline__ void row_product(const unsigned char* L, const int (&roff)[8], const bf16x8 (&breg)[8],
                                            floatx16& s0, floatx16& s1) {
  s0 = floatx16{};
  s1 = floatx16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 a0 = *(const bf16x8*)(L + roff[ks]);
    const bf16x8 a1 = *(const bf16x8*)(L + 32 * 256 + roff[ks]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, breg[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, breg[ks], s1, 0, 0, 0);
  }
}

__device__ __forceinline__ void load_row_frags(const uint16_t* row, bf16x8 (&r)[8], int kg) {
  const uint4v* src = (const uint4v*)row;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) r[ks] = __builtin_bit_cast(bf16x8, src[2 * ks + kg]);
}

// ---------------------------------------------------------------------------
// D_t = dO_t . O_t next to the forward's lse; 16 threads per (b, n, h) row, BTHD order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdArgs a) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rows = (size_t)a.B * a.N * a.H;
  const size_t row = t >> 4;
  float acc = 0.f;
  if (row < rows) {
    const uint4v x = ((const uint4v*)a.out)[t];
    const uint4v g = ((const uint4v*)a.dout)[t];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(x[e]) * bf16_lo(g[e]) + bf16_hi(x[e]) * bf16_hi(g[e]);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 16);
  if (row < rows && (t & 15) == 0) {
    const int h = (int)(row % a.H);
    const size_t n = (row / a.H) % a.N, b = row / ((size_t)a.H * a.N);
    const size_t r = (b * a.H + h) * a.tp + n;
    a.ld[2 * r] = a.lse[r];
    a.ld[2 * r + 1] = acc;
  }
}

// Padding rows N .. tp - 1 of every (b, h) get lse = +inf (P = 0) and D = 0; the pooled-key
// gradients start at zero.
__global__ __launch_bounds__(256) void bwd_init_kernel(BwdArgs a) {
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t bh_n = (size_t)a.B * a.H;
  const size_t pad = (size_t)(a.tp - a.N);
  for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < bh_n * pad; t += stride) {
    const size_t r = (t / pad) * a.tp + a.N + t % pad;
    a.ld[2 * r] = __builtin_inff();
    a.ld[2 * r + 1] = 0.f;
  }
  const size_t nz = bh_n * a.nbp * kDim;
  for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < nz; t += stride) {
    a.dkbar[t] = 0.f;
    a.dvbar[t] = 0.f;
  }
}

// mcol[bh][j][w] bit i % 64 (i = 64 w + bit) = mrow[bh][i][j / 64] bit j % 64.
__global__ __launch_bounds__(256) void bwd_transpose_kernel(BwdArgs a) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t per_bh = (size_t)a.nbw * a.nb;
  if (t >= (size_t)a.B * a.H * per_bh) return;
  const size_t bh = t / per_bh;
  const int wd = (int)((t % per_bh) / a.nb), j = (int)(t % a.nb);
  const uint64_t* src = a.mrow + bh * a.nb * a.nbw + (j >> 6);
  uint64_t word = 0;
  const int i_end = min(64, a.nb - 64 * wd);
  for (int ii = 0; ii < i_end; ++ii) word |= ((src[(size_t)(64 * wd + ii) * a.nbw] >> (j & 63)) & 1ull) << ii;
  a.mcol[(bh * a.nb + j) * a.nbw + wd] = word;
}

// ---------------------------------------------------------------------------
// dK / dV.  kPooled = false: one workgroup per (b, h, key block j), the query blocks that
// selected j.  kPooled = true: one workgroup per (b, h, chunk of 64 pooled keys, query
// range), the query blocks of the range, each pooled key j masked where i selected j.
// Two waves; wave w owns keys 32 w .. 32 w + 31 (one key column per lane): its K / V rows
// are the B operands of S = Q K^T and dP = dO V^T, and it accumulates dK^T and dV^T.
// ---------------------------------------------------------------------------
template <bool kPooled>
__global__ __launch_bounds__(128, 1) void bwd_kv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ql[2][16384];
  __shared__ __attribute__((aligned(16))) unsigned char Gl[2][16384];
  __shared__ __attribute__((aligned(16))) float St[2][256];     // (lse, D) pairs of 64 rows + copy
  __shared__ uint64_t mw_s[kPooled ? kMaxRange : 1];            // routing words of the range (pooled)

  const int nchunks = a.nbp / 64;
  const int total = kPooled ? a.B * a.H * nchunks * a.nrange : a.B * a.H * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  int bh, jb = 0, c = 0, r = 0;
  if constexpr (kPooled) {
    r = __builtin_amdgcn_readfirstlane(item % a.nrange);
    const int rest = __builtin_amdgcn_readfirstlane(item / a.nrange);
    c = __builtin_amdgcn_readfirstlane(rest % nchunks);
    bh = __builtin_amdgcn_readfirstlane(rest / nchunks);
  } else {
    jb = __builtin_amdgcn_readfirstlane(item % a.nb);
    bh = __builtin_amdgcn_readfirstlane(item / a.nb);
  }
  const int h = __builtin_amdgcn_readfirstlane(bh % a.H), b = __builtin_amdgcn_readfirstlane(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)a.H * kDim;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;
  const size_t pooled_head = (size_t)bh * a.nbp * kDim;

  // the lane's key column: token 64 jb + 32 w + l32, or pooled key 64 c + 32 w + l32
  const int key = (kPooled ? 64 * c : 64 * jb) + 32 * w + l32;
  const bool key_ok = kPooled ? key < a.nb : key < a.N;
  const int last_n = a.N - (a.nb - 1) * kBlock;
  const float bias = kPooled ? (key == a.nb - 1 ? __log2f((float)last_n) : 6.0f) : 0.f;
  bf16x8 kreg[8], vreg[8];
  if constexpr (kPooled) {
    load_row_frags(a.kbar_h + pooled_head + (size_t)key * kDim, kreg, kg);
    load_row_frags(a.vbar_h + pooled_head + (size_t)key * kDim, vreg, kg);
  } else {
    const int kr = key_ok ? key : a.N - 1;
    load_row_frags(a.k + head_off + (size_t)kr * rs, kreg, kg);
    load_row_frags(a.v + head_off + (size_t)kr * rs, vreg, kg);
  }

  // query-block iteration
  uint64_t valid_chunk = 0;
  if constexpr (kPooled) {
    const int nvalid = min(64, a.nb - 64 * c);
    valid_chunk = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
  }
  const uint64_t* mrow_bh = a.mrow + (size_t)bh * a.nb * a.nbw;
  const uint64_t* mcol_j = a.mcol + ((size_t)bh * a.nb + jb) * a.nbw;
  int it_i = kPooled ? r * a.bpr : 0;
  const int it_end = kPooled ? min(a.nb, (r + 1) * a.bpr) : a.nbw;
  if constexpr (kPooled) {
    // the chunk's routing word of every query block of the range, loaded once (bpr <= kMaxRange)
    for (int e = threadIdx.x; e < it_end - it_i; e += 128) mw_s[e] = mrow_bh[(size_t)(it_i + e) * a.nbw + c];
    __syncthreads();
  }
  const int range0 = it_i;
  uint64_t it_bits = 0;
  auto next_query = [&]() -> int {
    if constexpr (kPooled) {
      while (it_i < it_end) {
        const int i = it_i++;
        if (valid_chunk & ~uniform64(mw_s[i - range0])) return i;
      }
      return kEndB;
    } else {
      while (true) {
        if (it_bits) {
          const int i = (it_i - 1) * 64 + __builtin_ctzll(it_bits);
          it_bits &= it_bits - 1;
          return i;
        }
        if (it_i >= it_end) return kEndB;
        it_bits = uniform64(mcol_j[it_i++]);
      }
    }
  };

  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const uint32_t span_in = (uint32_t)((a.N - 1) * rs + kDim) * 2;
  const DmaOffsetsD doff = dma_offsets_d(row_bytes, w, lane);
  auto issue = [&](int i, int buf) {
    const uint32_t toff = (uint32_t)i * 64 * row_bytes;
    dma_tile_d(Ql[buf], make_rsrc(uniform_ptr(a.q + head_off), span_in), toff, row_bytes, doff, w);
    dma_tile_d(Gl[buf], make_rsrc(uniform_ptr(a.dout + head_off), span_in), toff, row_bytes, doff, w);
    if (w == 0)   // 64 (lse, D) pairs = 512 bytes; lanes 32..63 repeat lanes 0..31 into the copy half
      dma16_buf(make_rsrc(uniform_ptr(a.ld + (size_t)bh * a.tp * 2), (uint32_t)a.tp * 8),
                (uint32_t)i * 512 + (lane & 31) * 16, 0, (unsigned char*)St[buf]);
  };

  int roff[8];
  row_offsets(lane, roff);
  int toff[4][2];
  tr_offsets(lane, toff);

  floatx16 dkT[4], dvT[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    dkT[mt] = floatx16{};
    dvT[mt] = floatx16{};
  }
  int cur = next_query();
  int buf = 0;
  if (cur != kEndB) issue(cur, 0);
  while (cur != kEndB) {
    const int nxt = next_query();
    wait_vm0();
    lds_barrier();                                           // tile cur landed; other buffer free
    if (nxt != kEndB) issue(nxt, buf ^ 1);
    const unsigned char* Q = Ql[buf];
    const unsigned char* G = Gl[buf];
    bool ok = key_ok;
    if constexpr (kPooled) ok = ok && !((uniform64(mw_s[cur - range0]) >> (32 * w + l32)) & 1ull);
    floatx16 s0, s1, d0, d1;
    row_product(Q, roff, kreg, s0, s1);                      // S = Q K^T (rows = queries)
    row_product(G, roff, vreg, d0, d1);                      // dP = dO V^T
    bf16x8 pp[4], pd[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // rows 32 half + 8 q4 + 4 kg + 0..3: (lse, D) pairs, 32 bytes
        const float* st = St[buf] + 2 * (32 * half + 8 * q4 + 4 * kg);
        const floatx4 ld0 = *(const floatx4*)st;
        const floatx4 ld1 = *(const floatx4*)(st + 4);
        const float lse4[4] = {ld0[0], ld0[2], ld1[0], ld1[2]};
        const float dd4[4] = {ld0[1], ld0[3], ld1[1], ld1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * q4 + e;
          const float sv = half ? s1[idx] : s0[idx];
          const float dv = half ? d1[idx] : d0[idx];
          const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sv, kScaleLog2B, bias - lse4[e])) : 0.f;
          const float ds = p * (dv - dd4[e]);
          pp[2 * half + (idx >> 3)][idx & 7] = (__bf16)p;
          pd[2 * half + (idx >> 3)][idx & 7] = (__bf16)ds;
        }
      }
    }
    tr_product(dvT, G, toff, pp);                            // dV^T += dO^T P
    tr_product(dkT, Q, toff, pd);                            // dK^T += Q^T dS
    buf ^= 1;
    cur = nxt;
  }

  // epilogue: lane holds dims 32 mt + 8 g + 4 kg + 0..3 of its key
  if constexpr (kPooled) {
    if (key_ok) {
      float* gk = a.dkbar + ((size_t)bh * a.nbp + key) * kDim;
      float* gv = a.dvbar + ((size_t)bh * a.nbp + key) * kDim;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          const int dim = 32 * mt + 8 * (idx >> 2) + 4 * kg + (idx & 3);
          unsafeAtomicAdd(gk + dim, dkT[mt][idx] * kScaleB);
          unsafeAtomicAdd(gv + dim, dvT[mt][idx]);
        }
    }
  } else if (key_ok) {
    const float inv_n = 1.0f / (float)(jb == a.nb - 1 ? last_n : kBlock);
    const float* gk = a.dkbar + ((size_t)bh * a.nbp + jb) * kDim;
    const float* gv = a.dvbar + ((size_t)bh * a.nbp + jb) * kDim;
    uint16_t* dkr = a.dk + head_off + (size_t)key * rs;
    uint16_t* dvr = a.dv + head_off + (size_t)key * rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * kg;
        const floatx4 pk = *(const floatx4*)(gk + d0);
        const floatx4 pv = *(const floatx4*)(gv + d0);
        uint2v ok4, ov4;
        ok4[0] = pack_bf16x2(__builtin_fmaf(dkT[mt][4 * g], kScaleB, pk[0] * inv_n),
                             __builtin_fmaf(dkT[mt][4 * g + 1], kScaleB, pk[1] * inv_n));
        ok4[1] = pack_bf16x2(__builtin_fmaf(dkT[mt][4 * g + 2], kScaleB, pk[2] * inv_n),
                             __builtin_fmaf(dkT[mt][4 * g + 3], kScaleB, pk[3] * inv_n));
        ov4[0] = pack_bf16x2(dvT[mt][4 * g] + pv[0] * inv_n, dvT[mt][4 * g + 1] + pv[1] * inv_n);
        ov4[1] = pack_bf16x2(dvT[mt][4 * g + 2] + pv[2] * inv_n, dvT[mt][4 * g + 3] + pv[3] * inv_n);
        *(uint2v*)(dkr + d0) = ok4;
        *(uint2v*)(dvr + d0) = ov4;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, query block i), two waves of 32 query rows (one per lane
// column), over the forward's tiles: per routing chunk the pooled tile (K-bar / V-bar rows,
// bias log2 n_j, columns of unselected valid blocks) and the exact blocks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char Kl[2][16384];
  __shared__ __attribute__((aligned(16))) unsigned char Vl[2][16384];
  __shared__ uint64_t sel_s[kMaxChunksB], prox_s[kMaxChunksB];

  const int nchunks = a.nbp / 64;
  const int total = a.B * a.H * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  const int i = __builtin_amdgcn_readfirstlane(item % a.nb);
  const int bh = __builtin_amdgcn_readfirstlane(item / a.nb);
  const int h = __builtin_amdgcn_readfirstlane(bh % a.H), b = __builtin_amdgcn_readfirstlane(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)a.H * kDim;
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;
  const size_t pooled_head = (size_t)bh * a.nbp * kDim;

  for (int cc = tid; cc < nchunks; cc += 128) {
    const uint64_t selm = a.mrow[((size_t)bh * a.nb + i) * a.nbw + cc];
    const int nvalid = min(64, a.nb - 64 * cc);
    const uint64_t validm = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
    sel_s[cc] = selm & validm;
    prox_s[cc] = validm & ~selm;
  }
  const int qrow = i * kBlock + w * 32 + l32;
  const int qr = qrow < a.N ? qrow : a.N - 1;
  bf16x8 qreg[8], greg[8];
  load_row_frags(a.q + head_off + (size_t)qr * rs, qreg, kg);
  load_row_frags(a.dout + head_off + (size_t)qr * rs, greg, kg);
  const float lse = a.ld[((size_t)bh * a.tp + qrow) * 2];
  const float dd = a.ld[((size_t)bh * a.tp + qrow) * 2 + 1];
  __syncthreads();

  // K / V tiles from the head-major copies and the pooled K-bar / V-bar: 256-byte rows,
  // one head contiguous, rows past the end read as zeros
  const uint32_t row_bytes = kDim * 2;
  const uint32_t span_in = (uint32_t)a.N * row_bytes;
  const uint32_t span_pool = (uint32_t)a.nbp * row_bytes;
  const size_t kv_head = (size_t)bh * a.N * kDim;
  const DmaOffsetsD doff = dma_offsets_d(row_bytes, w, lane);
  auto issue = [&](int code, int buf) {
    if (code < 0) {
      const uint32_t toff = (uint32_t)(-code - 1) * 64 * row_bytes;
      dma_tile_d(Kl[buf], make_rsrc(uniform_ptr(a.kbar_h + pooled_head), span_pool), toff, row_bytes, doff, w);
      dma_tile_d(Vl[buf], make_rsrc(uniform_ptr(a.vbar_h + pooled_head), span_pool), toff, row_bytes, doff, w);
    } else {
      const uint32_t toff = (uint32_t)code * 64 * row_bytes;
      dma_tile_d(Kl[buf], make_rsrc(uniform_ptr(a.kh + kv_head), span_in), toff, row_bytes, doff, w);
      dma_tile_d(Vl[buf], make_rsrc(uniform_ptr(a.vh + kv_head), span_in), toff, row_bytes, doff, w);
    }
  };
  // tile order: per chunk, the pooled tile (code -(c + 1)) if the chunk has unselected
  // blocks, then its exact blocks (code = block index)
  int it_c = 0, it_phase = 0;
  uint64_t it_bits = 0;
  auto next_tile = [&]() -> int {
    while (it_c < nchunks) {
      if (it_phase == 0) {
        it_phase = 1;
        it_bits = uniform64(sel_s[it_c]);
        if (uniform64(prox_s[it_c])) return -(it_c + 1);
      }
      if (it_bits) {
        const int jbk = it_c * 64 + __builtin_ctzll(it_bits);
        it_bits &= it_bits - 1;
        return jbk;
      }
      ++it_c;
      it_phase = 0;
    }
    return kEndB;
  };

  int roff[8];
  row_offsets(lane, roff);
  int toff[4][2];
  tr_offsets(lane, toff);
  const int last_n = a.N - (a.nb - 1) * kBlock;
  const float last_bias = __log2f((float)last_n);

  floatx16 dqT[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) dqT[mt] = floatx16{};
  int cur = next_tile();
  int buf = 0;
  if (cur != kEndB) issue(cur, 0);
  while (cur != kEndB) {
    const int nxt = next_tile();
    wait_vm0();
    lds_barrier();                                           // tile cur landed; other buffer free
    if (nxt != kEndB) issue(nxt, buf ^ 1);
    const unsigned char* K = Kl[buf];
    const unsigned char* V = Vl[buf];
    floatx16 s0, s1, d0, d1;
    row_product(K, roff, qreg, s0, s1);                      // S^T = K Q^T (rows = keys)
    row_product(V, roff, greg, d0, d1);                      // dP^T = V dO^T
    uint64_t colmask;
    float b_full, b_last;
    int last_key;
    if (cur < 0) {
      const int cc = -cur - 1;
      colmask = uniform64(prox_s[cc]);
      b_full = 6.0f;                                         // log2 64
      b_last = last_bias;
      last_key = a.nb - 1 - cc * 64;
    } else {
      const int nvalid = min(kBlock, a.N - cur * kBlock);
      colmask = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
      b_full = 0.f;
      b_last = 0.f;
      last_key = -1;
    }
    bf16x8 pd[4];
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
      const float x0 = __builtin_fmaf(s0[idx], kScaleLog2B, (key0 == last_key ? b_last : b_full) - lse);
      const float x1 = __builtin_fmaf(s1[idx], kScaleLog2B, (key0 + 32 == last_key ? b_last : b_full) - lse);
      const float p0 = ((colmask >> key0) & 1) ? __builtin_amdgcn_exp2f(x0) : 0.f;
      const float p1 = ((colmask >> (key0 + 32)) & 1) ? __builtin_amdgcn_exp2f(x1) : 0.f;
      pd[idx >> 3][idx & 7] = (__bf16)(p0 * (d0[idx] - dd));
      pd[2 + (idx >> 3)][idx & 7] = (__bf16)(p1 * (d1[idx] - dd));
    }
    tr_product(dqT, K, toff, pd);                            // dQ^T += K^T dS^T
    buf ^= 1;
    cur = nxt;
  }

  if (qrow < a.N) {
    uint16_t* dst = a.dq + head_off + (size_t)qrow * rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2v pk;
        pk[0] = pack_bf16x2(dqT[mt][4 * g] * kScaleB, dqT[mt][4 * g + 1] * kScaleB);
        pk[1] = pack_bf16x2(dqT[mt][4 * g + 2] * kScaleB, dqT[mt][4 * g + 3] * kScaleB);
        *(uint2v*)(dst + 32 * mt + 8 * g + 4 * kg) = pk;
      }
  }
}

}  // namespace

hipError_t launch_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                           const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, Shape s,
                           const Workspace& ws, hipStream_t stream) {
  if (!ws.lse || !ws.mrow || !ws.mcol || !ws.ld || !ws.dkbar || !ws.dvbar || !ws.kh || !ws.vh)
    return hipErrorInvalidValue;
  const int nchunks = ws.nbp / 64;
  if (nchunks > kMaxChunksB) return hipErrorInvalidValue;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = nchunks; a.tp = ws.nbp * kBlock;
  a.kbar_h = ws.kbar_h; a.vbar_h = ws.vbar_h; a.kh = ws.kh; a.vh = ws.vh;
  a.lse = ws.lse; a.mrow = ws.mrow; a.mcol = ws.mcol; a.ld = ws.ld;
  a.dkbar = ws.dkbar; a.dvbar = ws.dvbar;
  // pooled keys: enough (chunk, query range) workgroups to fill the chip twice over
  const int bhc = s.B * s.H * nchunks;
  int nrange = (2048 + bhc - 1) / bhc;
  if (nrange < (ws.nb + kMaxRange - 1) / kMaxRange) nrange = (ws.nb + kMaxRange - 1) / kMaxRange;
  if (nrange > ws.nb) nrange = ws.nb;
  if (nrange < 1) nrange = 1;
  a.bpr = (ws.nb + nrange - 1) / nrange;
  a.nrange = (ws.nb + a.bpr - 1) / a.bpr;

  const size_t rows16 = (size_t)s.B * s.N * s.H * 16;
  hipLaunchKernelGGL(bwd_init_kernel, dim3(1024), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_rowdot_kernel, dim3((unsigned)((rows16 + 255) / 256)), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t nt = (size_t)s.B * s.H * ws.nb * nchunks;
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<true>, dim3(bhc * a.nrange), dim3(128), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<false>, dim3(s.B * s.H * ws.nb), dim3(128), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(s.B * s.H * ws.nb), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace solattn
