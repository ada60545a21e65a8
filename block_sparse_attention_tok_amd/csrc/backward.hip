// Sol-Attn and Sol-Attn2 backward passes with the forward's routing (and Sol-Attn2's key
// groups) held fixed, for gfx950.  The Sol-Attn2 part (its tail, anchors and group means) is
// the second half of this file; its exact tokens reuse the Sol-Attn kernels below.
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
  // Sol-Attn2 (sol2 = 1): no pooled tiles; the exact keys' epilogue adds their group's
  // gradient (ghi: group bits per key block, gdk / gdv: [B][H][nbp][2][128]) and the dQ
  // epilogue the tail terms (dlam [B][H][tp], tmu and aextra [B][H][2 nbp][128]).
  int sol2;
  const uint64_t* ghi; const float* gdk; const float* gdv;
  const float* dlam; const float* tmu; const float* aextra;
  // work orders (NULL = block order): query blocks by descending number of exact key blocks
  // (the dQ pass) and key blocks by descending number of query blocks that select them (the
  // exact dK / dV pass), [B][H][nbp] each
  const int* qord; const int* kord;
};

// Slot swizzle of a 64 x 256-byte tile that is read both by rows (16 consecutive rows,
// one logical chunk: 16 distinct slots) and transposed (4 consecutive rows x 4 chunks:
// 16 distinct slots).
__device__ __forceinline__ int swz_d(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct DmaOffsetsD {
  uint32_t o[4];
};

// Wave w, instruction n fills rows 32 w + 4 n + lane / 16, slot lane % 16 (see dma_tile_asm).
__device__ __forceinline__ DmaOffsetsD dma_offsets_d(uint32_t row_bytes, int w, int lane) {
  const int row = 32 * w + (lane >> 4);
  DmaOffsetsD d;
#pragma unroll
  for (int n = 0; n < 4; ++n) d.o[n] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_d(row + 4 * n)) << 4);
  return d;
}

typedef int intx4 __attribute__((ext_vector_type(4)));

// Buffer resource as four SGPRs (the form an asm operand takes): base, stride 0,
// num_records = bytes, raw-buffer flags (as make_rsrc).
__device__ __forceinline__ intx4 rsrc4(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return intx4{(int)__builtin_amdgcn_readfirstlane((uint32_t)p),
               (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu),
               (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// DMA of wave w's half of a 64 x 128 bf16 tile into LDS: eight buffer_load_dwordx4 ... lds
// (1 KB each, rows and slots as dma_offsets_d), rows past the resource's end reading as
// zeros.  Issued from asm: the tile loops read one buffer while the DMA fills the other, the
// buffer chosen at run time, and for a DMA that it issues itself the compiler cannot tell the
// two apart and waits for the DMA before every LDS read of the tile.  These asm loads are not
// tracked by the compiler: every read of the buffer they fill is ordered by the loop's own
// vmcnt wait and barrier.  The asm writes no register (M0 and SCC are clobbered) and carries
// its hazard padding: s_nop 4 for a resource or base written through v_readfirstlane just
// before, s_nop 0 between each M0 write and the load that uses it.
__device__ __forceinline__ void dma_tile_asm(unsigned char* lds, intx4 rsrc, uint32_t tile_off, uint32_t row_bytes,
                                             const DmaOffsetsD& off, int w) {
  uint32_t vo[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) vo[n] = off.o[n & 3] + tile_off + (uint32_t)n * 4 * row_bytes;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(lds + w * 8 * 1024));
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x400\n\ts_nop 0\n\tbuffer_load_dwordx4 %3, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x800\n\ts_nop 0\n\tbuffer_load_dwordx4 %4, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0xc00\n\ts_nop 0\n\tbuffer_load_dwordx4 %5, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x1000\n\ts_nop 0\n\tbuffer_load_dwordx4 %6, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x1400\n\ts_nop 0\n\tbuffer_load_dwordx4 %7, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x1800\n\ts_nop 0\n\tbuffer_load_dwordx4 %8, %0, 0 offen lds\n\t"
      "s_add_u32 m0, %1, 0x1c00\n\ts_nop 0\n\tbuffer_load_dwordx4 %9, %0, 0 offen lds"
      ::"s"(rsrc), "s"(base), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "v"(vo[5]), "v"(vo[6]),
        "v"(vo[7])
      : "memory", "m0", "scc");
}

// One 16-byte-per-lane load into LDS (dma16_buf) issued from asm, for the same reason.
__device__ __forceinline__ void dma16_asm(intx4 rsrc, uint32_t voffset, unsigned char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %0, 0 offen lds"
               ::"s"(rsrc), "s"(base), "v"(voffset)
               : "memory", "m0");
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

// Scheduling pattern for a run of kN MFMAs that take kR LDS reads each: every MFMA's reads
// are issued kAhead MFMAs before it, so that the LDS latency overlaps the products (left to
// itself the scheduler places each read just before its MFMA and waits for it).  Placed
// after the products it orders, in the same basic block; the closing sched_barrier keeps
// the instructions after it out of the pattern.
template <int kN, int kR, int kAhead>
__device__ __forceinline__ void sched_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kR * kAhead, 0);
#pragma unroll
  for (int i = 0; i < kN - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kR, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, kAhead, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Keeps a loop-carried accumulator in AGPRs, where its MFMAs read and write it: without the
// pin the register allocator keeps it in VGPRs and copies it to AGPRs and back every tile.
__device__ __forceinline__ void pin_agpr(floatx16 (&acc)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) asm volatile("" : "+a"(acc[mt]));
}

// row_product written as asm MFMAs, for the loops whose loop-carried accumulators take all
// the AGPRs they can get: the results c0 / c1 land in VGPRs, where the softmax VALU reads
// them, and the B fragments breg sit in AGPRs, so that the compiler's own MFMAs (the dK /
// dV / dQ products) keep their accumulators in AGPRs instead of copying them between
// register files on every tile.  Hazard padding carried by the asm: s_nop 1 before each
// pair of MFMAs (an operand written by a VALU op needs two wait states before an MFMA
// reads it); row_products_end() adds 21 wait states after the chains, before c0 / c1 are
// read (an MFMA result needs up to 19 before a VALU op reads it).  The A operands are all
// read from LDS before the first MFMA (the LDS read queue keeps them in order).
__device__ __forceinline__ void row_product_v(const unsigned char* L, const int (&roff)[8], const bf16x8 (&breg)[8],
                                              floatx16& c0, floatx16& c1) {
  bf16x8 a[16];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    a[2 * ks] = *(const bf16x8*)(L + roff[ks]);
    a[2 * ks + 1] = *(const bf16x8*)(L + 32 * 256 + roff[ks]);
  }
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %3, %4, 0"
      : "=&v"(c0), "=&v"(c1)
      : "v"(a[0]), "v"(a[1]), "a"(breg[0]));
#pragma unroll
  for (int ks = 1; ks < 8; ++ks)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %4, %1"
        : "+v"(c0), "+v"(c1)
        : "v"(a[2 * ks]), "v"(a[2 * ks + 1]), "a"(breg[ks]));
}

__device__ __forceinline__ void row_products_end(floatx16& s0, floatx16& s1, floatx16& d0, floatx16& d1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s0), "+v"(s1), "+v"(d0), "+v"(d1));
}

// One k-step of two row-product chains as asm (see row_product_v): c0 += a0 x b0 and
// c1 += a1 x b1, or c0 = a0 x b0, c1 = a1 x b1 for the first step.
template <bool kFirst>
__device__ __forceinline__ void mfma_pair(floatx16& c0, floatx16& c1, const bf16x8& a0, const bf16x8& a1,
                                          const bf16x8& b0, const bf16x8& b1) {
  if constexpr (kFirst)
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %5, 0"
        : "=&v"(c0), "=&v"(c1)
        : "v"(a0), "v"(a1), "a"(b0), "a"(b1));
  else
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %3, %5, %1"
        : "+v"(c0), "+v"(c1)
        : "v"(a0), "v"(a1), "a"(b0), "a"(b1));
}

// First k-step with c0 starting from its current value (a bias) and c1 from zero.
__device__ __forceinline__ void mfma_pair_c0(floatx16& c0, floatx16& c1, const bf16x8& a0, const bf16x8& a1,
                                             const bf16x8& b0, const bf16x8& b1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %3, %5, 0"
      : "+v"(c0), "=&v"(c1)
      : "v"(a0), "v"(a1), "a"(b0), "a"(b1));
}

// 21 wait states after the last MFMA of a chain before its results are read.
__device__ __forceinline__ void chain_end(floatx16& c0, floatx16& c1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(c0), "+v"(c1));
}

// acc += a x b as asm with acc in AGPRs: a loop-carried accumulator that every MFMA takes
// through this asm stays in the same AGPRs across the branches of a tile loop.  s_nop 1 for a
// b written by a VALU op just before; the final read of acc needs acc_end() first.
__device__ __forceinline__ void mfma_acc(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void acc_end(floatx16 (&acc)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
}

// The transposed-read A operand of tr_product for (mt, st).
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* L, const int (&toff)[4][2], int mt, int st) {
  const uint2v lo = lds_read_tr16(L + toff[mt][0] + st * 16 * 256);
  const uint2v hi = lds_read_tr16(L + toff[mt][1] + st * 16 * 256);
  return __builtin_bit_cast(bf16x8, uint4v{lo[0], lo[1], hi[0], hi[1]});
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
    const int j0 = __builtin_amdgcn_readfirstlane(item % a.nb);
    bh = __builtin_amdgcn_readfirstlane(item / a.nb);
    jb = a.kord ? __builtin_amdgcn_readfirstlane(a.kord[(size_t)bh * a.nbp + j0]) : j0;
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
    dma_tile_asm(Ql[buf], rsrc4(a.q + head_off, span_in), toff, row_bytes, doff, w);
    dma_tile_asm(Gl[buf], rsrc4(a.dout + head_off, span_in), toff, row_bytes, doff, w);
    if (w == 0)   // 64 (lse, D) pairs = 512 bytes; lanes 32..63 repeat lanes 0..31 into the copy half
      dma16_asm(rsrc4(a.ld + (size_t)bh * a.tp * 2, (uint32_t)a.tp * 8), (uint32_t)i * 512 + (lane & 31) * 16,
                (unsigned char*)St[buf]);
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
    // (lse, D) pairs of rows 32 half + 8 q4 + 4 kg + 0..3 (32 bytes each), read before the
    // products so that they have arrived when the softmax needs them
    floatx4 ldr[2][4][2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float* st = St[buf] + 2 * (32 * half + 8 * q4 + 4 * kg);
        ldr[half][q4][0] = *(const floatx4*)st;
        ldr[half][q4][1] = *(const floatx4*)(st + 4);
      }
    floatx16 s0, s1, d0, d1;
    row_product_v(Q, roff, kreg, s0, s1);                    // S = Q K^T (rows = queries)
    row_product_v(G, roff, vreg, d0, d1);                    // dP = dO V^T
    row_products_end(s0, s1, d0, d1);
    bf16x8 pp[4], pd[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const floatx4 ld0 = ldr[half][q4][0];
        const floatx4 ld1 = ldr[half][q4][1];
        const float lse4[4] = {ld0[0], ld0[2], ld1[0], ld1[2]};
        const float dd4[4] = {ld0[1], ld0[3], ld1[1], ld1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * q4 + e;
          const float sv = half ? s1[idx] : s0[idx];
          const float dv = half ? d1[idx] : d0[idx];
          // exact keys: a key column past the sequence only feeds its own dK / dV column,
          // which is not stored, so it needs no mask
          const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, kScaleLog2B, bias - lse4[e]));
          const float p = kPooled ? (ok ? e2 : 0.f) : e2;
          const float ds = p * (dv - dd4[e]);
          pp[2 * half + (idx >> 3)][idx & 7] = (__bf16)p;
          pd[2 * half + (idx >> 3)][idx & 7] = (__bf16)ds;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    tr_product(dvT, G, toff, pp);                            // dV^T += dO^T P
    tr_product(dkT, Q, toff, pd);                            // dK^T += Q^T dS
    sched_reads_ahead<32, 2, 4>();
    pin_agpr(dvT);
    pin_agpr(dkT);
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
    const int n_blk = jb == a.nb - 1 ? last_n : kBlock;
    float inv_n;
    const float* gk;
    const float* gv;
    if (a.sol2) {
      // Sol-Attn2: the key's group (G_hi if its bit is set) passes 1/n_g of its gradient
      const uint64_t hi = a.ghi[(size_t)bh * a.nbp + jb];
      const int grp = ((hi >> (32 * w + l32)) & 1ull) ? 0 : 1;
      const int nh = __popcll(hi);
      inv_n = 1.0f / (float)(grp == 0 ? nh : n_blk - nh);
      gk = a.gdk + (((size_t)bh * a.nbp + jb) * 2 + grp) * kDim;
      gv = a.gdv + (((size_t)bh * a.nbp + jb) * 2 + grp) * kDim;
    } else {
      inv_n = 1.0f / (float)n_blk;
      gk = a.dkbar + ((size_t)bh * a.nbp + jb) * kDim;
      gv = a.dvbar + ((size_t)bh * a.nbp + jb) * kDim;
    }
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
  const int i0 = __builtin_amdgcn_readfirstlane(item % a.nb);
  const int bh = __builtin_amdgcn_readfirstlane(item / a.nb);
  const int i = a.qord ? __builtin_amdgcn_readfirstlane(a.qord[(size_t)bh * a.nbp + i0]) : i0;
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
    prox_s[cc] = a.sol2 ? 0ull : validm & ~selm;            // Sol-Attn2: the tail has its own kernels
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
      dma_tile_asm(Kl[buf], rsrc4(a.kbar_h + pooled_head, span_pool), toff, row_bytes, doff, w);
      dma_tile_asm(Vl[buf], rsrc4(a.vbar_h + pooled_head, span_pool), toff, row_bytes, doff, w);
    } else {
      const uint32_t toff = (uint32_t)code * 64 * row_bytes;
      dma_tile_asm(Kl[buf], rsrc4(a.kh + kv_head, span_in), toff, row_bytes, doff, w);
      dma_tile_asm(Vl[buf], rsrc4(a.vh + kv_head, span_in), toff, row_bytes, doff, w);
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
  pin_agpr(dqT);

  // Each tile is hand-interleaved so that the softmax of one 32-key half runs under the MFMAs
  // of the other (one wave per SIMD leaves no other wave to fill the gaps): S^T, dP^T of keys
  // 0..31; then those of keys 32..63 with the dS of keys 0..31 between their MFMAs; then
  // dQ^T over keys 0..31 with the dS of keys 32..63; then dQ^T over keys 32..63.  Each
  // sched_barrier keeps the code between two of them in place.  A pooled tile's weights
  // log2 n_j and masks, and a partial block's masks, enter as the initial value of the S^T
  // accumulators (bias / scale, or -inf), so that every tile runs the same code; every MFMA
  // that touches dQ^T is asm on AGPRs, which keeps the accumulator in place.
  auto ds_pair = [&](const floatx16& sv, const floatx16& dv, bf16x8 (&pd)[4], int half, int j) {
    const int idx = 2 * j;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[idx], kScaleLog2B, -lse));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[idx + 1], kScaleLog2B, -lse));
    pd[2 * half + (idx >> 3)][idx & 7] = (__bf16)(p0 * (dv[idx] - dd));
    pd[2 * half + (idx >> 3)][(idx & 7) + 1] = (__bf16)(p1 * (dv[idx + 1] - dd));
  };
  auto load_tr = [&](const unsigned char* K, bf16x8 (&ta)[8], int half) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int st = 0; st < 2; ++st) ta[2 * mt + st] = tr_operand(K, toff, mt, 2 * half + st);
  };

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
    const bool full = cur >= 0 && cur * kBlock + kBlock <= a.N;
    floatx16 s0, s1, d0, d1;
    if (!full) {
      // initial S^T rows: 0 for a counted key of an exact block, log2 n_j / scale for a
      // pooled key of an unselected block, -inf for the rest
      uint64_t colmask;
      float b_full, b_last;
      int last_key;
      if (cur < 0) {
        const int cc = -cur - 1;
        colmask = uniform64(prox_s[cc]);
        b_full = 6.0f / kScaleLog2B;                         // log2 64
        b_last = last_bias / kScaleLog2B;
        last_key = a.nb - 1 - cc * 64;
      } else {
        const int nvalid = min(kBlock, a.N - cur * kBlock);
        colmask = (1ull << nvalid) - 1;                      // nvalid < 64 here
        b_full = 0.f;
        b_last = 0.f;
        last_key = -1;
      }
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) {
        const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
        s0[idx] = ((colmask >> key0) & 1) ? (key0 == last_key ? b_last : b_full) : kNegInf;
        s1[idx] = ((colmask >> (key0 + 32)) & 1) ? (key0 + 32 == last_key ? b_last : b_full) : kNegInf;
      }
    }
    bf16x8 ka[8], va[8], kb[8], vb[8], pd[4], ta[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      ka[ks] = *(const bf16x8*)(K + roff[ks]);
      va[ks] = *(const bf16x8*)(V + roff[ks]);
    }
    if (full) mfma_pair<true>(s0, d0, ka[0], va[0], qreg[0], greg[0]);
    else mfma_pair_c0(s0, d0, ka[0], va[0], qreg[0], greg[0]);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) mfma_pair<false>(s0, d0, ka[ks], va[ks], qreg[ks], greg[ks]);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kb[ks] = *(const bf16x8*)(K + 32 * 256 + roff[ks]);
      vb[ks] = *(const bf16x8*)(V + 32 * 256 + roff[ks]);
    }
    if (full) mfma_pair<true>(s1, d1, kb[0], vb[0], qreg[0], greg[0]);
    else mfma_pair_c0(s1, d1, kb[0], vb[0], qreg[0], greg[0]);
    chain_end(s0, d0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 1; ks < 8; ++ks) {
      mfma_pair<false>(s1, d1, kb[ks], vb[ks], qreg[ks], greg[ks]);
      ds_pair(s0, d0, pd, 0, ks - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_tr(K, ta, 0);
    ds_pair(s0, d0, pd, 0, 7);
    chain_end(s1, d1);
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T over keys 0..31 (k-steps 0, 1), one dS pair of keys 32..63 per MFMA
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mfma_acc(dqT[i >> 1], ta[i], pd[i & 1]);
      ds_pair(s1, d1, pd, 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_tr(K, ta, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) mfma_acc(dqT[i >> 1], ta[i], pd[2 + (i & 1)]);
    buf ^= 1;
    cur = nxt;
  }
  acc_end(dqT);

  if (qrow < a.N) {
    uint16_t* dst = a.dq + head_off + (size_t)qrow * rs;
    if (a.sol2) {
      // Sol-Attn2 tail terms of row t in anchor a = (i, w): s dlambda_t mu_a (through
      // lambda_t) plus the anchor's share of dq-bar_a
      const size_t arow = ((size_t)bh * a.nbp + i) * 2 + w;
      const float sdl = a.dlam[(size_t)bh * a.tp + qrow] * kScaleB;
      const float* mu = a.tmu + arow * kDim;
      const float* ax = a.aextra + arow * kDim;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * mt + 8 * g + 4 * kg;
          const floatx4 m4 = *(const floatx4*)(mu + d0);
          const floatx4 x4 = *(const floatx4*)(ax + d0);
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(dqT[mt][4 * g + e], kScaleB, __builtin_fmaf(sdl, m4[e], x4[e]));
          uint2v pk;
          pk[0] = pack_bf16x2(r[0], r[1]);
          pk[1] = pack_bf16x2(r[2], r[3]);
          *(uint2v*)(dst + d0) = pk;
        }
    } else {
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
}

// ===========================================================================
// Sol-Attn2 backward (draft, Method, Stage A1 passage: routing and groups fixed).  With the
// tail of anchor a written as a softmax over groups g with logits l_g = ln n_g + s q-bar_a .
// k-bar_g, probabilities pi_g, mu_a = sum pi_g k-bar_g, nu_a = sum pi_g v-bar_g, and each
// row's tail logit lambda_t = ln Z_a + s (q'_t - q-bar_a) . mu_a, the gradient splits into
//   rows:     dlambda_t = P_t,tail (dO_t . nu_a - D_t),  dq_t += s dlambda_t mu_a;
//   anchors:  dlnZ_a = sum_t dlambda_t,  dmu_a = s sum_t dlambda_t (q'_t - q-bar_a),
//             dnu_a = sum_t P_t,tail dO_t;
//   groups:   dl_g = pi_g (dmu_a . k-bar_g + dnu_a . v-bar_g + c_a) with
//             c_a = dlnZ_a - dmu_a . mu_a - dnu_a . nu_a -- the backward of an attention of
//             anchors over groups with "output gradient" [dmu_a | dnu_a], "values"
//             [k-bar_g | v-bar_g] and D = -c_a -- giving dq-bar_a = s sum_g dl_g k-bar_g -
//             s dlnZ_a mu_a, dk-bar_g = s sum_a dl_g q-bar_a + sum_a pi_g dmu_a and
//             dv-bar_g = sum_a pi_g dnu_a;
//   means:    every row of anchor a gets dq-bar_a / n_a, every token of group g gets
//             dk-bar_g / n_g and dv-bar_g / n_g (added by the exact-key kernel's epilogue).
// The E4M3 quantizer of Q and K is passed straight through: the exact products run on the
// dequantized q', k' rounded to bf16.
// ===========================================================================
struct Bwd2Args {
  int B, N, H, nb, nbp, nbw, tp;
  const uint16_t* v; const uint16_t* dout;                          // BTHD
  const float* ofp;                                                 // [B][H][tp][128] fp32 output rows
  const uint8_t* q8; const uint8_t* k8; const float* qscale; const float* kscale;
  const float* qanc; const float* tmu; const float* tnu; const float* tlz; const float* lse;
  const uint16_t* gk; const uint16_t* gv; const float* glogn;       // group rows [B][H][2 nbp]
  const uint64_t* sel; const uint64_t* mcol;
  uint16_t* qd; uint16_t* kd; uint16_t* kh; uint16_t* vh;
  float* ld; float* dlam;
  uint16_t* qab; uint16_t* dmub; uint16_t* dnub; float* alz; float* aextra;
  float* gdk; float* gdv;
};

// bf16 copies of q' = s_q E4M3(q / s_q) and k' (BTHD, and k' head-major) and a head-major
// copy of v; 16 threads per (b, n, h) row, 8 dims each.
__global__ __launch_bounds__(256) void bwd2_prep_kernel(Bwd2Args a) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = t >> 4;
  if (row >= (size_t)a.B * a.N * a.H) return;
  const int c = (int)(t & 15);
  const int h = (int)(row % a.H);
  const size_t n = (row / a.H) % a.N, b = row / ((size_t)a.H * a.N);
  const size_t bh = b * a.H + h;
  const size_t src8 = (bh * a.tp + n) * kDim + 8 * c;
  const size_t blk = bh * a.nbp + n / kBlock;
  const float sq = a.qscale[blk], sk = a.kscale[blk];
  const uint2v cq = *(const uint2v*)(a.q8 + src8);
  const uint2v ck = *(const uint2v*)(a.k8 + src8);
  uint4v oq, ok;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    auto q01 = __builtin_amdgcn_cvt_pk_f32_fp8(cq[m], false), q23 = __builtin_amdgcn_cvt_pk_f32_fp8(cq[m], true);
    auto k01 = __builtin_amdgcn_cvt_pk_f32_fp8(ck[m], false), k23 = __builtin_amdgcn_cvt_pk_f32_fp8(ck[m], true);
    oq[2 * m] = pack_bf16x2(q01[0] * sq, q01[1] * sq);
    oq[2 * m + 1] = pack_bf16x2(q23[0] * sq, q23[1] * sq);
    ok[2 * m] = pack_bf16x2(k01[0] * sk, k01[1] * sk);
    ok[2 * m + 1] = pack_bf16x2(k23[0] * sk, k23[1] * sk);
  }
  const size_t dst = row * kDim + 8 * c;
  const size_t dsth = (bh * a.N + n) * kDim + 8 * c;
  *(uint4v*)(a.qd + dst) = oq;
  *(uint4v*)(a.kd + dst) = ok;
  *(uint4v*)(a.kh + dsth) = ok;
  *(uint4v*)(a.vh + dsth) = *(const uint4v*)(a.v + dst);
}

// Per query block i (< nbp; blocks past the sequence give empty anchors): each row's
// (lse, D) pair for the exact kernels and dlambda_t; each anchor's bf16 q-bar_a, dmu_a,
// dnu_a, its (log2 Z_a, -c_a) pair (log2 Z_a = +inf for an anchor without rows or tail,
// which zeroes its group probabilities) and the first part of dq-bar_a / n_a.
// Threads: phase 1 row tid / 4, dims 32 (tid % 4) ..; phase 2 anchor tid / 128, dim tid % 128.
__global__ __launch_bounds__(256) void bwd2_anchor_kernel(Bwd2Args a) {
  __shared__ float mu_s[2][kDim], nu_s[2][kDim];
  __shared__ float dl_s[64], pt_s[64];
  __shared__ float red_s[4][2];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int n_i = i < a.nb ? min(kBlock, a.N - i * kBlock) : 0;
  const size_t blk = (size_t)bh * a.nbp + i;
  const float sq = i < a.nb ? a.qscale[blk] : 1.f;
  for (int e = tid; e < 2 * kDim; e += 256) {
    const int w = e >> 7, d = e & (kDim - 1);
    const bool live = n_i > 32 * w;
    mu_s[w][d] = live ? a.tmu[(blk * 2 + w) * kDim + d] : 0.f;
    nu_s[w][d] = live ? a.tnu[(blk * 2 + w) * kDim + d] : 0.f;
  }
  __syncthreads();

  // phase 1: D_t = dO_t . O_t (O_t the forward's fp32 row: with bf16 rows the rounding of
  // O would swamp dlambda_t where the tail carries nearly all of a row's weight, and
  // dlambda_t is then a small difference), dO_t . nu_a and q'_t . mu_a over the row's
  // four quarters
  {
    const int r = tid >> 2, c = tid & 3, wa = r >> 5;
    const int t = i * kBlock + r;
    const bool valid = r < n_i;
    float od = 0.f, nd = 0.f, qm = 0.f;
    if (valid) {
      const size_t g0 = (((size_t)b * a.N + t) * a.H + h) * kDim + 32 * c;
      const floatx4* op = (const floatx4*)(a.ofp + ((size_t)bh * a.tp + t) * kDim + 32 * c);
      const uint4v* gp = (const uint4v*)(a.dout + g0);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint4v g = gp[m];
        const floatx4 x0 = op[2 * m], x1 = op[2 * m + 1];
        const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 32 * c + 8 * m + 2 * e;
          const float g0v = bf16_lo(g[e]), g1v = bf16_hi(g[e]);
          od += g0v * xs[2 * e] + g1v * xs[2 * e + 1];
          nd += g0v * nu_s[wa][d] + g1v * nu_s[wa][d + 1];
        }
      }
      const uint4v* qp = (const uint4v*)(a.q8 + ((size_t)bh * a.tp + t) * kDim + 32 * c);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4v cw = qp[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(cw[e], false), f23 = __builtin_amdgcn_cvt_pk_f32_fp8(cw[e], true);
          const float* mu = mu_s[wa] + 32 * c + 16 * m + 4 * e;
          qm += f01[0] * mu[0] + f01[1] * mu[1] + f23[0] * mu[2] + f23[1] * mu[3];
        }
      }
    }
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
      od += __shfl_xor(od, o);
      nd += __shfl_xor(nd, o);
      qm += __shfl_xor(qm, o);
    }
    const float tl = n_i > 32 * wa ? a.tlz[blk * 2 + wa] : kNegInf;
    const float lse2 = valid ? a.lse[(size_t)bh * a.tp + t] : __builtin_inff();
    float dl = 0.f, pt = 0.f;
    if (valid && tl != kNegInf) {
      pt = __builtin_amdgcn_exp2f(tl + qm * sq * kScaleLog2B - lse2);
      dl = pt * (nd - od);
    }
    if (c == 0) {
      const size_t rr = (size_t)bh * a.tp + t;
      a.ld[2 * rr] = lse2;
      a.ld[2 * rr + 1] = valid ? od : 0.f;
      a.dlam[rr] = dl;
      dl_s[r] = dl;
      pt_s[r] = pt;
    }
  }
  __syncthreads();

  // phase 2: the anchor sums
  const int w2 = tid >> 7, d = tid & (kDim - 1);
  const size_t arow = blk * 2 + w2;
  const int n_a = w2 == 0 ? min(n_i, 32) : max(n_i - 32, 0);
  float sdq = 0.f, snu = 0.f, dlnz = 0.f;
  for (int rr = 0; rr < n_a; ++rr) {
    const int t = i * kBlock + 32 * w2 + rr;
    const float dlv = dl_s[32 * w2 + rr], ptv = pt_s[32 * w2 + rr];
    dlnz += dlv;
    const uint32_t code = a.q8[((size_t)bh * a.tp + t) * kDim + d];
    const float qv = __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0] * sq;
    const float gv = bf16_bits_to_f32(a.dout[(((size_t)b * a.N + t) * a.H + h) * kDim + d]);
    sdq = __builtin_fmaf(dlv, qv, sdq);
    snu = __builtin_fmaf(ptv, gv, snu);
  }
  const float qa = n_a > 0 ? a.qanc[arow * kDim + d] : 0.f;
  const float mu = mu_s[w2][d], nu = nu_s[w2][d];
  const float dmu = kScaleB * (sdq - dlnz * qa);
  const __bf16 dmu_b = (__bf16)dmu, dnu_b = (__bf16)snu, qa_b = (__bf16)qa;
  a.qab[arow * kDim + d] = __builtin_bit_cast(uint16_t, qa_b);
  a.dmub[arow * kDim + d] = __builtin_bit_cast(uint16_t, dmu_b);
  a.dnub[arow * kDim + d] = __builtin_bit_cast(uint16_t, dnu_b);
  a.aextra[arow * kDim + d] = n_a > 0 ? -kScaleB * dlnz * mu / (float)n_a : 0.f;
  // c_a uses the bf16 dmu_a, dnu_a that the group products see
  float pc = (float)dmu_b * mu + (float)dnu_b * nu;
  float pq = qa * mu;
  pc = wave_sum(pc);
  pq = wave_sum(pq);
  if ((tid & 63) == 0) {
    red_s[tid >> 6][0] = pc;
    red_s[tid >> 6][1] = pq;
  }
  __syncthreads();
  if (d == 0) {
    const float ct = red_s[2 * w2][0] + red_s[2 * w2 + 1][0];
    const float qt = red_s[2 * w2][1] + red_s[2 * w2 + 1][1];
    const float tl = n_a > 0 ? a.tlz[arow] : kNegInf;
    const bool live = tl != kNegInf;
    a.alz[arow * 2] = live ? tl + qt * kScaleLog2B : __builtin_inff();
    a.alz[arow * 2 + 1] = live ? ct - dlnz : 0.f;
  }
}

// dP accumulation (no zeroing): s0 / s1 += rows 0..31 / 32..63 of the tile at L times breg.
__device__ __forceinline__ void row_product_acc(const unsigned char* L, const int (&roff)[8], const bf16x8 (&breg)[8],
                                                floatx16& s0, floatx16& s1) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 a0 = *(const bf16x8*)(L + roff[ks]);
    const bf16x8 a1 = *(const bf16x8*)(L + 32 * 256 + roff[ks]);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, breg[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, breg[ks], s1, 0, 0, 0);
  }
}

// dq-bar_a: one workgroup per (b, h, 64 anchors = 32 query blocks), two waves of 32 anchors
// (one per lane column), over the tiles of 64 groups (32 key blocks) whose blocks lie in
// the sequence: S^T = K-bar Q-bar^T, dP^T = K-bar dmu^T + V-bar dnu^T (rows = groups),
// dS^T = P^T (dP^T - D), dq-bar^T += K-bar^T dS^T.  Adds s dq-bar_a / n_a to aextra.
__global__ __launch_bounds__(128, 1) void bwd2_tail_dq_kernel(Bwd2Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char Kl[2][16384];
  __shared__ __attribute__((aligned(16))) unsigned char Vl[2][16384];
  __shared__ __attribute__((aligned(16))) float Bl[2][256];     // ln n_g of the tile's groups + copies
  const int nt = (a.nb + 31) / 32;
  const int item = xcd_remap(blockIdx.x, a.B * a.H * nt);
  const int at = __builtin_amdgcn_readfirstlane(item % nt);
  const int bh = __builtin_amdgcn_readfirstlane(item / nt);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int al = 32 * w + l32;
  const size_t rows_bh = (size_t)bh * 2 * a.nbp;
  const size_t arow = rows_bh + 64 * at + al;
  const int ia = 32 * at + (al >> 1);
  const bool a_ok = ia < a.nb;
  bf16x8 qreg[8], mreg[8], nreg[8];
  load_row_frags(a.qab + arow * kDim, qreg, kg);
  load_row_frags(a.dmub + arow * kDim, mreg, kg);
  load_row_frags(a.dnub + arow * kDim, nreg, kg);
  const float lz = a.alz[arow * 2], dd = a.alz[arow * 2 + 1];
  const uint64_t* selrow = a.sel + ((size_t)bh * a.nb + (a_ok ? ia : 0)) * a.nbw;

  const uint32_t row_bytes = kDim * 2;
  const uint32_t span = (uint32_t)(2 * a.nbp) * row_bytes;
  const DmaOffsetsD doff = dma_offsets_d(row_bytes, w, lane);
  auto issue = [&](int gt, int buf) {
    const uint32_t toff = (uint32_t)gt * 64 * row_bytes;
    dma_tile_asm(Kl[buf], rsrc4(a.gk + rows_bh * kDim, span), toff, row_bytes, doff, w);
    dma_tile_asm(Vl[buf], rsrc4(a.gv + rows_bh * kDim, span), toff, row_bytes, doff, w);
    if (w == 0)   // 64 floats = 256 bytes; lanes 16..63 repeat lanes 0..15 into the copies
      dma16_asm(rsrc4(a.glogn + rows_bh, (uint32_t)(2 * a.nbp) * 4), (uint32_t)gt * 256 + (lane & 15) * 16,
                (unsigned char*)Bl[buf]);
  };
  int roff[8];
  row_offsets(lane, roff);
  int toff[4][2];
  tr_offsets(lane, toff);

  floatx16 dqT[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) dqT[mt] = floatx16{};
  issue(0, 0);
  int buf = 0;
  for (int gt = 0; gt < nt; ++gt) {
    wait_vm0();
    lds_barrier();                                           // tile gt landed; other buffer free
    if (gt + 1 < nt) issue(gt + 1, buf ^ 1);
    const unsigned char* K = Kl[buf];
    const unsigned char* V = Vl[buf];
    floatx16 s0, s1, d0, d1;
    row_product(K, roff, qreg, s0, s1);                      // S^T (rows = groups)
    row_product(K, roff, mreg, d0, d1);                      // dP^T = K-bar dmu^T ...
    row_product_acc(V, roff, nreg, d0, d1);                  // ... + V-bar dnu^T
    // groups of blocks the anchor's query block selected are exact tokens, not tail
    const uint32_t exact = a_ok ? (uint32_t)(selrow[gt >> 1] >> (32 * (gt & 1))) : 0xffffffffu;
    bf16x8 pd[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const floatx4 b0 = *(const floatx4*)(Bl[buf] + 8 * q4 + 4 * kg);
      const floatx4 b1 = *(const floatx4*)(Bl[buf] + 32 + 8 * q4 + 4 * kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * q4 + e;
        const int r0 = 8 * q4 + 4 * kg + e;
        const bool ok0 = !((exact >> (r0 >> 1)) & 1u) && b0[e] != kNegInf;
        const bool ok1 = !((exact >> ((r0 + 32) >> 1)) & 1u) && b1[e] != kNegInf;
        const float p0 = ok0 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[idx], kScaleLog2B, b0[e] * kLog2e - lz)) : 0.f;
        const float p1 = ok1 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s1[idx], kScaleLog2B, b1[e] * kLog2e - lz)) : 0.f;
        pd[idx >> 3][idx & 7] = (__bf16)(p0 * (d0[idx] - dd));
        pd[2 + (idx >> 3)][idx & 7] = (__bf16)(p1 * (d1[idx] - dd));
      }
    }
    tr_product(dqT, K, toff, pd);                            // dq-bar^T += K-bar^T dS^T
    buf ^= 1;
  }

  const int n_i = a_ok ? min(kBlock, a.N - ia * kBlock) : 0;
  const int n_a = (al & 1) ? max(n_i - 32, 0) : min(n_i, 32);
  if (n_a > 0) {
    const float f = kScaleB / (float)n_a;
    float* dst = a.aextra + arow * kDim;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * kg;
        floatx4 x = *(floatx4*)(dst + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(dqT[mt][4 * g + e], f, x[e]);
        *(floatx4*)(dst + d0) = x;
      }
  }
}

// dk-bar_g, dv-bar_g: one workgroup per (b, h, 64 groups = 32 key blocks), two waves of 32
// groups (one per lane column), over the tiles of 64 anchors whose blocks lie in the
// sequence: S = Q-bar K-bar^T, dP = dmu K-bar^T + dnu V-bar^T (rows = anchors),
// dS' = s P (dP - D), dv-bar^T += dnu^T P, dk-bar^T += Q-bar^T dS' + dmu^T P.
__global__ __launch_bounds__(128, 1) void bwd2_group_grad_kernel(Bwd2Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char Ql[2][16384];
  __shared__ __attribute__((aligned(16))) unsigned char Ml[2][16384];
  __shared__ __attribute__((aligned(16))) unsigned char Nl[2][16384];
  __shared__ __attribute__((aligned(16))) float St[2][256];     // (log2 Z_a, D) of 64 anchors + copy
  const int nt = (a.nb + 31) / 32;
  const int item = xcd_remap(blockIdx.x, a.B * a.H * nt);
  const int gt = __builtin_amdgcn_readfirstlane(item % nt);
  const int bh = __builtin_amdgcn_readfirstlane(item / nt);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gl = 32 * w + l32;
  const size_t rows_bh = (size_t)bh * 2 * a.nbp;
  const size_t grow = rows_bh + 64 * gt + gl;
  const int jg = 32 * gt + (gl >> 1);
  bf16x8 kreg[8], vreg[8];
  load_row_frags(a.gk + grow * kDim, kreg, kg);
  load_row_frags(a.gv + grow * kDim, vreg, kg);
  const float lnb = a.glogn[grow];
  const bool g_ok = jg < a.nb && lnb != kNegInf;
  const float bias = g_ok ? lnb * kLog2e : 0.f;
  const uint64_t* mc = a.mcol + ((size_t)bh * a.nb + (jg < a.nb ? jg : 0)) * a.nbw;

  const uint32_t row_bytes = kDim * 2;
  const uint32_t span = (uint32_t)(2 * a.nbp) * row_bytes;
  const DmaOffsetsD doff = dma_offsets_d(row_bytes, w, lane);
  auto issue = [&](int at, int buf) {
    const uint32_t toff = (uint32_t)at * 64 * row_bytes;
    dma_tile_asm(Ql[buf], rsrc4(a.qab + rows_bh * kDim, span), toff, row_bytes, doff, w);
    dma_tile_asm(Ml[buf], rsrc4(a.dmub + rows_bh * kDim, span), toff, row_bytes, doff, w);
    dma_tile_asm(Nl[buf], rsrc4(a.dnub + rows_bh * kDim, span), toff, row_bytes, doff, w);
    if (w == 0)   // 64 (log2 Z, D) pairs = 512 bytes; lanes 32..63 repeat lanes 0..31 into the copy
      dma16_asm(rsrc4(a.alz + rows_bh * 2, (uint32_t)(2 * a.nbp) * 8), (uint32_t)at * 512 + (lane & 31) * 16,
                (unsigned char*)St[buf]);
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
  issue(0, 0);
  int buf = 0;
  for (int at = 0; at < nt; ++at) {
    wait_vm0();
    lds_barrier();                                           // tile at landed; other buffer free
    if (at + 1 < nt) issue(at + 1, buf ^ 1);
    const unsigned char* Q = Ql[buf];
    const unsigned char* M = Ml[buf];
    const unsigned char* Nn = Nl[buf];
    floatx16 s0, s1, d0, d1;
    row_product(Q, roff, kreg, s0, s1);                      // S (rows = anchors)
    row_product(M, roff, kreg, d0, d1);                      // dP = dmu K-bar^T ...
    row_product_acc(Nn, roff, vreg, d0, d1);                 // ... + dnu V-bar^T
    // anchors whose query block selected the group's block see its tokens exactly
    const uint32_t exact = g_ok ? (uint32_t)(mc[at >> 1] >> (32 * (at & 1))) : 0xffffffffu;
    bf16x8 pp[4], pd[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float* st = St[buf] + 2 * (32 * half + 8 * q4 + 4 * kg);
        const floatx4 ld0 = *(const floatx4*)st;
        const floatx4 ld1 = *(const floatx4*)(st + 4);
        const float lz4[4] = {ld0[0], ld0[2], ld1[0], ld1[2]};
        const float dd4[4] = {ld0[1], ld0[3], ld1[1], ld1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = 4 * q4 + e;
          const int r = 32 * half + 8 * q4 + 4 * kg + e;       // anchor row of the tile
          const bool ok = !((exact >> (r >> 1)) & 1u) && 32 * at + (r >> 1) < a.nb;
          const float sv = half ? s1[idx] : s0[idx];
          const float dv = half ? d1[idx] : d0[idx];
          const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sv, kScaleLog2B, bias - lz4[e])) : 0.f;
          pp[2 * half + (idx >> 3)][idx & 7] = (__bf16)p;
          pd[2 * half + (idx >> 3)][idx & 7] = (__bf16)(p * (dv - dd4[e]) * kScaleB);
        }
      }
    }
    tr_product(dvT, Nn, toff, pp);                           // dv-bar^T += dnu^T P
    tr_product(dkT, M, toff, pp);                            // dk-bar^T += dmu^T P
    tr_product(dkT, Q, toff, pd);                            //          + Q-bar^T dS'
    buf ^= 1;
  }

  float* gk = a.gdk + grow * kDim;
  float* gv = a.gdv + grow * kDim;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mt + 8 * g + 4 * kg;
      floatx4 k4, v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = dkT[mt][4 * g + e];
        v4[e] = dvT[mt][4 * g + e];
      }
      *(floatx4*)(gk + d0) = k4;
      *(floatx4*)(gv + d0) = v4;
    }
}

// Work orders of the exact-token passes, one workgroup per (batch, head) and kind: y = 0 sorts
// the query blocks by their number of exact key blocks (popcounts of the routing rows), y = 1
// the key blocks by how many query blocks select them (popcounts of the transposed rows), both
// descending, so that the longest work items start first and the workgroups that share an
// XCD's L2 stream their tiles at similar rates.  The orders only schedule work.
__global__ __launch_bounds__(256) void bwd_order_kernel(const uint64_t* __restrict__ mrow,
                                                        const uint64_t* __restrict__ mcol, int nb, int nbw,
                                                        int nbp, int* __restrict__ qord, int* __restrict__ kord) {
  extern __shared__ int sm[];
  int* slot = sm;                                        // [nb + 1]
  unsigned short* qc = (unsigned short*)(sm + nb + 1);   // [nb] counts (<= nb <= 8192)
  __shared__ int part[256];
  const int bh = blockIdx.x, kind = blockIdx.y;
  const uint64_t* words = (kind == 0 ? mrow : mcol) + (size_t)bh * nb * nbw;
  for (int i = threadIdx.x; i < nb; i += 256) {
    int c = 0;
    for (int cc = 0; cc < nbw; ++cc) c += __builtin_popcountll(words[(size_t)i * nbw + cc]);
    qc[i] = c;
  }
  __syncthreads();
  sort_desc_counts(qc, slot, part, nb, (kind == 0 ? qord : kord) + (size_t)bh * nbp);
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
  a.sol2 = 0;
  a.ghi = nullptr; a.gdk = nullptr; a.gdv = nullptr; a.dlam = nullptr; a.tmu = nullptr; a.aextra = nullptr;
  a.qord = ws.bqord; a.kord = ws.bkord;
  // pooled keys: (chunk, query range) workgroups for about one wave of workgroups over the
  // chip (two per CU) and no more: the ranges of a chunk finish together and add into the
  // same dkbar / dvbar rows, and those atomics cost more than the extra occupancy gains
  // (operator shape, 256 (b, h, chunk) items, ms per backward: 1 / 2 / 3 / 4 ranges 9.37 /
  // 8.86 / 9.06 / 8.99 on one box; 4 / 8 / 16 / 32 ranges 9.33 / 9.62 / 10.2 / 11.9 on another)
  const int bhc = s.B * s.H * nchunks;
  int nrange = (512 + bhc - 1) / bhc;
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
  if (a.qord != nullptr && a.kord != nullptr) {
    hipLaunchKernelGGL(bwd_order_kernel, dim3(s.B * s.H, 2), dim3(256),
                       (ws.nb + 1) * sizeof(int) + ws.nb * sizeof(unsigned short), stream, ws.mrow, ws.mcol, ws.nb,
                       nchunks, ws.nbp, ws.bqord, ws.bkord);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_kv_kernel<true>, dim3(bhc * a.nrange), dim3(128), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<false>, dim3(s.B * s.H * ws.nb), dim3(128), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(s.B * s.H * ws.nb), dim3(128), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward2(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                            const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, Shape s,
                            const Workspace& ws, hipStream_t stream) {
  (void)q;
  (void)k;   // the backward reads the forward's E4M3 codes and scales from the workspace
  if (!ws.lse || !ws.sel || !ws.mcol || !ws.ld || !ws.kh || !ws.vh || !ws.qd || !ws.kd || !ws.dlam || !ws.qab ||
      !ws.dmub || !ws.dnub || !ws.alz || !ws.aextra || !ws.gdk || !ws.gdv || !ws.q8 || !ws.k8 || !ws.qscale ||
      !ws.kscale || !ws.qanc || !ws.tmu || !ws.tnu || !ws.tlz || !ws.gk || !ws.gv || !ws.glogn || !ws.ghi ||
      !ws.ofp)
    return hipErrorInvalidValue;
  const int nchunks = ws.nbp / 64;
  if (nchunks > kMaxChunksB) return hipErrorInvalidValue;
  Bwd2Args t;
  t.B = s.B; t.N = s.N; t.H = s.H; t.nb = ws.nb; t.nbp = ws.nbp; t.nbw = nchunks; t.tp = ws.nbp * kBlock;
  t.v = v; t.dout = dout; t.ofp = ws.ofp;
  t.q8 = ws.q8; t.k8 = ws.k8; t.qscale = ws.qscale; t.kscale = ws.kscale;
  t.qanc = ws.qanc; t.tmu = ws.tmu; t.tnu = ws.tnu; t.tlz = ws.tlz; t.lse = ws.lse;
  t.gk = ws.gk; t.gv = ws.gv; t.glogn = ws.glogn;
  t.sel = ws.sel; t.mcol = ws.mcol;
  t.qd = ws.qd; t.kd = ws.kd; t.kh = ws.kh; t.vh = ws.vh;
  t.ld = ws.ld; t.dlam = ws.dlam;
  t.qab = ws.qab; t.dmub = ws.dmub; t.dnub = ws.dnub; t.alz = ws.alz; t.aextra = ws.aextra;
  t.gdk = ws.gdk; t.gdv = ws.gdv;

  BwdArgs a;
  a.q = ws.qd; a.k = ws.kd; a.v = v; a.out = out; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = nchunks; a.tp = ws.nbp * kBlock;
  a.kbar_h = nullptr; a.vbar_h = nullptr; a.kh = ws.kh; a.vh = ws.vh;
  a.lse = ws.lse; a.mrow = ws.sel; a.mcol = ws.mcol; a.ld = ws.ld;
  a.dkbar = nullptr; a.dvbar = nullptr;
  a.nrange = 1; a.bpr = ws.nb;
  a.sol2 = 1;
  a.ghi = ws.ghi; a.gdk = ws.gdk; a.gdv = ws.gdv; a.dlam = ws.dlam; a.tmu = ws.tmu; a.aextra = ws.aextra;
  a.qord = ws.bqord; a.kord = ws.bkord;

  const size_t rows16 = (size_t)s.B * s.N * s.H * 16;
  const int nt = (ws.nb + 31) / 32;
  const int bhn = s.B * s.H;
  hipLaunchKernelGGL(bwd2_prep_kernel, dim3((unsigned)((rows16 + 255) / 256)), dim3(256), 0, stream, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t ntr = (size_t)bhn * ws.nb * nchunks;
  hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((ntr + 255) / 256)), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.qord != nullptr && a.kord != nullptr) {
    hipLaunchKernelGGL(bwd_order_kernel, dim3(bhn, 2), dim3(256),
                       (ws.nb + 1) * sizeof(int) + ws.nb * sizeof(unsigned short), stream, ws.sel, ws.mcol, ws.nb,
                       nchunks, ws.nbp, ws.bqord, ws.bkord);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd2_anchor_kernel, dim3(ws.nbp, bhn), dim3(256), 0, stream, t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd2_tail_dq_kernel, dim3(bhn * nt), dim3(128), 0, stream, t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd2_group_grad_kernel, dim3(bhn * nt), dim3(128), 0, stream, t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<false>, dim3(bhn * ws.nb), dim3(128), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(bhn * ws.nb), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace solattn
