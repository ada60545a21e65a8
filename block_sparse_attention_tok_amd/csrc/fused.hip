// Fused Sol-Attn forward kernel for gfx950 (Sol-Attn stage 2).
//
// Sol-Attn paper (arXiv 2607.24027) §3.2, Figure 4 and "Hardware-Aligned
// Implementation": each program keeps one query block on chip and one
// online-softmax state in registers; it streams the pooled keys / values in
// chunks, folds every unselected block in through its proxy (token-to-block tile
// Q_i K-bar^T with weight n_j and the V sum V-hat_j) and runs exact attention on
// the original K/V blocks of the selected indices.  The selection is made here,
// chunk by chunk (§3.1 Eq. (4), §3.2 Eq. (6)): each block's proxy score
// s_ij = Q-bar_i . K-bar_j / sqrt(d), from the fp32 block means of stage 1,
// against the query block's threshold tau_i, with the sink's blocks forced exact.
// The decisions live in LDS only; no proxy score or routing map is written to
// memory (the test export may copy the words out).
//
// gfx950 mapping: one workgroup = one (batch, head, 64-row query block, key
// split), two wave64s of 32 query rows; __launch_bounds__(128, 2) keeps two
// waves per SIMD; workgroups are ordered so that each XCD walks its own heads.
//   * Routing: lane l of a wave scores key block 64 c + l of chunk c (128 fp32
//     FMAs over the block means, Q-bar_i broadcast from LDS), and one ballot
//     against tau_i gives the chunk's 64-bit selection word; the two waves take
//     alternate chunks of the split while the first pooled tile's DMA is in
//     flight.  The per-chunk selection and proxy masks stay in LDS.
//   * The tile stream is the pooled tile of every chunk (K-bar / V-bar = V-hat/n
//     rows with logit bias log2 n_j; selected and padding columns masked), then
//     the selected exact blocks chunk by chunk.
//   * The first pooled tile fixes a per-row reference m_ref, the largest pooled
//     logit log2(e) q . K-bar_j / sqrt(d) of its chunk.  Because a block's mean of
//     exponentials is at least the exponential of its mean logit, the softmax
//     denominator measured against m_ref is >= 1, so every tile takes
//     P = 2^(x - m_ref) with no running maximum and no O rescale; a workgroup
//     whose O or l overflows reruns its tiles with the usual rescaling.
//   * Tiles move HBM -> LDS with buffer_load ... lds (no VGPR staging; the
//     buffer's range check covers every lane offset) into one K and one V
//     buffer whose 16-byte slots are XOR-swizzled per row; the V load of tile t
//     overlaps S_t and its exponentials, the K load of tile t+1 overlaps PV_t.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wave's query rows in registers): one query per lane, so the row max is
//     in-lane plus one v_permlane32_swap; row sums use v_dot2 on the bf16 P.
//   * O^T += V^T P^T: A = V^T gathered from the row-major V tile with
//     ds_read_b64_tr_b16, B = P straight from the S^T accumulator (the k order
//     inside each MFMA is permuted identically on both operands).
//   * Several key splits write fp32 normalized partial rows and their
//     log2-sum-exp; a small merge kernel combines them and rounds each output
//     to bf16 once.
#include "common.h"
#include "kernels.h"
#include "pipe.h"

namespace solattn {

constexpr float kScale = 0.08838834764831845f;        // 1/sqrt(128)
constexpr float kScaleLog2 = kScale * kLog2e;
constexpr int kMaxChunks = 128;                         // nbp / 64 <= 128 (tokens <= 524288)
constexpr int kEnd = -0x7fffffff;

struct FusedArgs {
  const uint16_t* q; uint16_t* out;
  int B, N, H, nb, nbp, nbw;
  int S, cps;                   // key-range splits and routing chunks per split
  float* opart; float* olse;    // split partials (S > 1): fp32 normalized rows, log2-sum-exp
  const uint16_t* kbar_h; const uint16_t* vbar_h;
  const uint16_t* kh; const uint16_t* vh;   // head-major copies of k and v ([B][H][N][128])
  const float* qbar;            // [B][H][nbp][128] fp32 query-block means
  const float* kbar_t;          // [B][H][32][nbp][4] fp32 key-block means, 4-dim interleaved
  const float* tau_i;           // [B][H][nbp] thresholds
  int sink_b0, sink_b1;
  uint64_t* mask_out;           // the selection words used, sink included (NULL = none)
  unsigned long long* pairs;    // += selected token pairs n_i n_j of this work item (NULL = none)
  float* lse;                   // [B][H][tp] base-2 log-sum-exp per query row (NULL = none)
  int tp;
  const int* order;             // [B][H][nbp] query blocks by descending exact-block count (NULL = block order)
};

// Tile order: first the pooled tile of every chunk c (code -(c + 1)), then the selected
// blocks chunk by chunk (code = block index).
struct TileIter {
  int c;
  int phase;           // 0: pooled tiles, 1: exact blocks
  uint64_t bits;
};

// Chunks are numbered locally from c0 (the split's first chunk); returned codes are global.
__device__ __forceinline__ int next_tile(TileIter& it, const uint64_t* sel_s, int nchunks, int c0) {
  if (it.phase == 0) {
    if (it.c < nchunks) return -(c0 + it.c++ + 1);
    it.phase = 1;
    it.c = 0;
    it.bits = nchunks > 0 ? uniform64(sel_s[0]) : 0ull;
  }
  while (it.c < nchunks) {
    if (it.bits) {
      const int jb = (c0 + it.c) * 64 + __builtin_ctzll(it.bits);
      it.bits &= it.bits - 1;
      return jb;
    }
    if (++it.c < nchunks) it.bits = uniform64(sel_s[it.c]);
  }
  return kEnd;
}

// K operand reads are issued this many score MFMAs ahead of the MFMA that consumes them.
constexpr int kSAhead = 4;

enum TileMode { kExactFull = 0, kExactPartial = 1, kProxy = 2 };

__global__ __launch_bounds__(128, 2) void sol_fused_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char Kl[64 * 256];
  __shared__ __attribute__((aligned(1024))) unsigned char Vl[64 * 256];
  __shared__ uint64_t sel_s[kMaxChunks], prox_s[kMaxChunks];
  __shared__ float4 qbar_s[kDim / 4];                        // Q-bar_i (fp32), read by every lane
  __shared__ int redo_s[2];

  // Work item order: query block fastest, then key split, then (batch, head), so the
  // workgroups that run together on one XCD share a head and a key range.  Within a (head,
  // split) the query blocks come by descending exact-block count over the split's key range
  // (the order array): the longest items start first, and the workgroups that share an
  // XCD's L2 at a time stream their selected tiles at similar rates.
  const int total = a.B * a.H * a.S * a.nb;
  const int item = xcd_remap(blockIdx.x, total);
  // The divisions run on the VALU; readfirstlane keeps the (uniform) indices in
  // SGPRs so addresses and buffer resources derived from them stay scalar.
  const int i0 = __builtin_amdgcn_readfirstlane(item % a.nb);
  const int rest = __builtin_amdgcn_readfirstlane(item / a.nb);
  const int split = __builtin_amdgcn_readfirstlane(rest % a.S);
  const int bh = __builtin_amdgcn_readfirstlane(rest / a.S);
  const int i = a.order ? __builtin_amdgcn_readfirstlane(a.order[((size_t)bh * a.S + split) * a.nbp + i0]) : i0;
  const int h = __builtin_amdgcn_readfirstlane(bh % a.H), b = __builtin_amdgcn_readfirstlane(bh / a.H);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, kg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t rs = (size_t)a.H * kDim;                      // elements between tokens (BTHD)
  const size_t head_off = (size_t)b * a.N * rs + (size_t)h * kDim;

  const int qrow = i * kBlock + w * 32 + l32;
  bf16x8 qreg[8];
  {
    const uint4v* src = (const uint4v*)(a.q + head_off + (size_t)(qrow < a.N ? qrow : a.N - 1) * rs);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, src[2 * ks + kg]);
  }
  if (tid < kDim / 4) qbar_s[tid] = ((const float4*)(a.qbar + ((size_t)bh * a.nbp + i) * kDim))[tid];
  __syncthreads();

  // Buffer resources over this head's rows of the head-major k / v copies and of the
  // pooled K-bar / V-bar (both 256-byte rows, one head contiguous), so one set of lane
  // offsets serves every tile; built at each use from kernel arguments so they stay in
  // SGPRs.  Rows past the end of either read as zeros.
  const uint32_t row_bytes = kDim * 2;
  const uint32_t span_in = (uint32_t)a.N * row_bytes;
  const uint32_t span_pool = (uint32_t)a.nbp * row_bytes;
  const size_t pooled_head = (size_t)bh * a.nbp * kDim;
  const size_t kv_head = (size_t)bh * a.N * kDim;
  const DmaOffsets doff = dma_offsets(row_bytes, w, lane);
  const int c_begin = split * a.cps;                        // this split's routing chunks
  const int c_end = min(a.nbp / 64, c_begin + a.cps);
  const int nchunks = c_end - c_begin;
  // Routing of the split's chunks (Sol-Attn paper §3.1 Eq. (4), §3.2 Eq. (6)).  The first
  // pooled tile's DMA does not depend on it and is issued first.  Wave w scores chunks
  // c_begin + w, c_begin + w + 2, ...: lane l takes key block j = 64 c + l (j < nbp, so the
  // padded fp32 means are in memory) and sums Q-bar_i . K-bar_j over the 128 dims in
  // ascending order with fp32 FMAs; s_ij > tau_i is one ballot.  The sink's blocks are
  // forced exact and the chunk's padding blocks cleared.
  auto pool = [&]() { return make_rsrc(uniform_ptr(a.kbar_h + pooled_head), span_pool); };
  dma_tile<false>(Kl, pool(), (uint32_t)c_begin * 64 * row_bytes, row_bytes, doff, w);
  {
    const float tau = a.tau_i[(size_t)bh * a.nbp + i];
    const float4* kt = (const float4*)a.kbar_t + (size_t)bh * 32 * a.nbp;
    for (int cc = w; cc < nchunks; cc += 2) {
      const int c = c_begin + cc;
      const float acc = proxy_dot(qbar_s, kt, a.nbp, 64 * c + lane);
      const uint64_t selm = exact_word(__ballot(acc * kScale > tau), c, a.nb, a.sink_b0, a.sink_b1);
      const int nvalid = a.nb - 64 * c;                      // valid blocks of the chunk (>= 1)
      const uint64_t validm = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
      if (lane == 0) {
        sel_s[cc] = selm;
        prox_s[cc] = validm & ~selm;
        if (a.mask_out) a.mask_out[((size_t)bh * a.nb + i) * a.nbw + c] = selm;
      }
    }
  }
  lds_barrier();
  if (a.pairs != nullptr && tid == 0) {
    // selected token pairs of this work item: n_i times the valid tokens of its exact blocks
    unsigned long long cols = 0;
    for (int cc = 0; cc < nchunks; ++cc) cols += 64ull * (unsigned)__builtin_popcountll(sel_s[cc]);
    const int last = a.nb - 1, last_n = a.N - last * kBlock;
    if (last >= 64 * c_begin && last < 64 * c_end && ((sel_s[last / 64 - c_begin] >> (last & 63)) & 1))
      cols -= (unsigned long long)(kBlock - last_n);
    atomicAdd(a.pairs, cols * (unsigned long long)min(kBlock, a.N - i * kBlock));
  }

  // ---- per-lane LDS offsets
  // S^T A operand: key row 32 mt + l32, k-step ks reads logical chunk 2 ks + kg, physical slot
  // (2 ks + kg) ^ swz_k(row) (row & 15 = l32 & 15 for both m-tiles).
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = l32 * 256 + 16 * ((2 * ks + kg) ^ swz_k(l32));
  int voff[4];                                               // V^T operand (transposed read)
  v_operand_offsets(lane, voff);

  // S^T = K Q^T for the 64-row K tile at LDS `kl` (two 32-key m-tiles), with the 8 DMA
  // instructions that `dma` issues (this tile's V) spread over the first products.
  auto scores = [&](const unsigned char* kl, floatx16& s0, floatx16& s1, auto&& dma) {
    s0 = floatx16{};
    s1 = floatx16{};
    bf16x8 ak[16];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      ak[2 * ks] = *(const bf16x8*)(kl + koff[ks]);
      ak[2 * ks + 1] = *(const bf16x8*)(kl + 32 * 256 + koff[ks]);
    }
    dma();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[2 * ks], qreg[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[2 * ks + 1], qreg[ks], s1, 0, 0, 0);
    }
    // each K operand read kSAhead products ahead of its MFMA
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kSAhead, 0);
#pragma unroll
    for (int i = 0; i < 16 - kSAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (i < 8 / kDmaPerProduct) __builtin_amdgcn_sched_group_barrier(kSchedVmem, kDmaPerProduct, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kSAhead, 0);
  };

  // ---- reference max.  Every unselected block j contributes n_j 2^(x_j) with
  // x_j = log2(e) q . K-bar_j / sqrt(d), and every selected block at least as much
  // (the mean of exp over a block is >= exp of the mean logit), so with m_ref = x_j of
  // any one block the softmax denominator is >= 1.  The first tile of the stream is the
  // pooled tile of the split's first chunk; m_ref is the largest x_j over its valid
  // blocks (selected or not), and every tile takes P = 2^(x - m_ref) with no running
  // maximum.  Logits above m_ref are representable up to ~2^127; a row that still
  // overflows sends the workgroup through the rescaling loop below.
  floatx16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  const int last_n = a.N - (a.nb - 1) * kBlock;
  const float last_bias = __log2f((float)last_n);

  // Issue the DMA of one buffer (K or V) of tile `code` (pooled tiles from K-bar / V-bar,
  // exact ones from the head-major copies).  The source is chosen with scalar selects, not
  // branches, so that the DMA can share a scheduling region with the products around it.
  auto issue = [&](int code_in, auto is_v_tag) {
    constexpr bool kV = decltype(is_v_tag)::value;
    const int code = __builtin_amdgcn_readfirstlane(code_in);
    const bool pooled = code < 0;
    const uint16_t* base = pooled ? (kV ? a.vbar_h : a.kbar_h) + pooled_head : (kV ? a.vh : a.kh) + kv_head;
    const uint32_t tile_off = (uint32_t)(pooled ? -code - 1 : code) * 64 * row_bytes;
    dma_tile<kV>(kV ? Vl : Kl, make_rsrc(uniform_ptr(base), pooled ? span_pool : span_in), tile_off, row_bytes,
                 doff, w);
  };

  // The tile stream of this split (pooled tiles first, then the exact blocks).
  // kSafe = false: every tile against m_ref, which the first pooled tile sets, with no
  // rescaling; kSafe = true: running max with the usual rescale of O and l throughout.
  // first_issued: the K DMA of the first tile is already in flight.
  auto run_tiles = [&](auto safe_tag, bool first_issued) {
    constexpr bool kSafe = decltype(safe_tag)::value;
    TileIter it{0, 0, 0};
    int cur = next_tile(it, sel_s, nchunks, c_begin);
    if (cur != kEnd && !first_issued) issue(cur, BoolTag<false>{});
    while (cur != kEnd) {
      const int nxt = next_tile(it, sel_s, nchunks, c_begin);
      wait_vm0();
      lds_barrier();                                         // K(cur) landed; V buffer free
      const int valid = cur < 0 ? kBlock : min(kBlock, a.N - cur * kBlock);

      floatx16 s0, s1;
      scores(Kl, s0, s1, [&]() { issue(cur, BoolTag<true>{}); });
      const int mode = cur < 0 ? kProxy : (valid == kBlock ? kExactFull : kExactPartial);
      bf16x8 pa[4];
      if constexpr (!kSafe) {
        // ---- P = 2^(x - m_ref) with the tile's mask / proxy weight n_j (m_ref is set by
        // the first tile, a pooled one, below; the exact tiles come after it)
        float p0[16], p1[16];
        const float neg_ref = -m_run;
        if (mode == kExactFull) {
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            p0[idx] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[idx], kScaleLog2, neg_ref));
            p1[idx] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[idx], kScaleLog2, neg_ref));
          }
        } else if (mode == kExactPartial) {
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[idx], kScaleLog2, neg_ref));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[idx], kScaleLog2, neg_ref));
            p0[idx] = key0 < valid ? e0 : 0.f;
            p1[idx] = key0 + 32 < valid ? e1 : 0.f;
          }
        } else {
          // pooled tile; the first one (the split's first chunk) fixes the reference
          // m_ref = its maximum pooled logit over every valid key, selected or not
          const int c = -cur - 1;
          const int nvalid = __builtin_amdgcn_readfirstlane(a.nb - c * 64);
          float mx = kNegInf;
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
            mx = fmaxf(mx, fmaxf(key0 < nvalid ? s0[idx] : kNegInf, key0 + 32 < nvalid ? s1[idx] : kNegInf));
          }
          m_run = m_run == kNegInf ? max_with_partner(mx) * kScaleLog2 : m_run;
          const uint64_t colmask = uniform64(prox_s[c - c_begin]);
          const int last_key = a.nb - 1 - c * 64;
          const float off_full = 6.0f - m_run;                  // log2(64) for full blocks
          const float off_last = last_bias - m_run;
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
            const float e0 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s0[idx], kScaleLog2, key0 == last_key ? off_last : off_full));
            const float e1 = __builtin_amdgcn_exp2f(
                __builtin_fmaf(s1[idx], kScaleLog2, key0 + 32 == last_key ? off_last : off_full));
            p0[idx] = ((colmask >> key0) & 1) ? e0 : 0.f;
            p1[idx] = ((colmask >> (key0 + 32)) & 1) ? e1 : 0.f;
          }
        }
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          pa[(idx >> 3)][idx & 7] = (__bf16)p0[idx];            // k-step st = keys 16 st .. 16 st + 15
          pa[2 + (idx >> 3)][idx & 7] = (__bf16)p1[idx];
        }
        // l sums the bf16 P that the PV product consumes.
#pragma unroll
        for (int st = 0; st < 4; ++st) l_run = add_bf16x8(pa[st], l_run);
      } else {
        // ---- logits (log2 units) with the tile's mask / bias, online softmax
        float scale = kScaleLog2;                             // applied inside the exp argument
        if (mode == kExactPartial) {
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
            s0[idx] = key0 < valid ? s0[idx] * kScaleLog2 : kNegInf;
            s1[idx] = key0 + 32 < valid ? s1[idx] * kScaleLog2 : kNegInf;
          }
          scale = 1.f;
        } else if (mode == kProxy) {
          const int c = -cur - 1;
          const uint64_t colmask = uniform64(prox_s[c - c_begin]);
          const int last_key = a.nb - 1 - c * 64;
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) {
            const int key0 = 8 * (idx >> 2) + 4 * kg + (idx & 3);
            const float b0 = key0 == last_key ? last_bias : 6.0f;
            const float b1 = key0 + 32 == last_key ? last_bias : 6.0f;
            s0[idx] = ((colmask >> key0) & 1) ? s0[idx] * kScaleLog2 + b0 : kNegInf;
            s1[idx] = ((colmask >> (key0 + 32)) & 1) ? s1[idx] * kScaleLog2 + b1 : kNegInf;
          }
          scale = 1.f;
        }
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int idx = 1; idx < 16; ++idx) mx = fmaxf(mx, fmaxf(s0[idx], s1[idx]));
        mx = max_with_partner(mx) * scale;                    // scale > 0 commutes with max
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        // Unconditional rescale (skipping it behind a wave-uniform branch made results
        // timing-dependent with two waves per SIMD).
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int idx = 0; idx < 16; ++idx) o[mt][idx] *= alpha;
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
          const float q0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[idx], scale, -m_use));
          const float q1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[idx], scale, -m_use));
          psum += q0 + q1;
          pa[(idx >> 3)][idx & 7] = (__bf16)q0;
          pa[2 + (idx >> 3)][idx & 7] = (__bf16)q1;
        }
        l_run += psum;
      }

      wait_vm0();
      lds_barrier();                                         // V(cur) landed; K buffer free
      // O^T += V^T P^T, with the next tile's K DMA (after the last tile, the current K again,
      // so that every iteration has the same shape; it lands before the loop exits)
      pv_tile_dma(o, Vl, voff, pa, [&]() { issue(nxt != kEnd ? nxt : cur, BoolTag<false>{}); });
      cur = nxt;
    }
    wait_vm0();
  };

  run_tiles(BoolTag<false>{}, true);
  float l_tot = sum_with_partner(l_run);
  float m_fin = m_run;
  {
    // Any non-finite O or l in the workgroup: rerun its tiles with rescaling.
    float chk = l_tot * 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int idx = 0; idx < 16; ++idx) chk = __builtin_fmaf(o[mt][idx], 0.f, chk);
    const uint64_t bad = __ballot(!(chk == 0.f));
    if (lane == 0) redo_s[w] = bad != 0;
    __syncthreads();
    if (redo_s[0] | redo_s[1]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) o[mt] = floatx16{};
      l_run = 0.f;
      m_run = kNegInf;
      run_tiles(BoolTag<true>{}, false);
      l_tot = sum_with_partner(l_run);
      m_fin = m_run;
    }
  }

  // ---- epilogue: O / l, bf16 RNE, BTHD store; with key splits, this split's normalized
  // row in fp32 and its log2-sum-exp m + log2 l instead (the merge rounds to bf16 once)
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < a.N) {
    const float lse2 = l_tot > 0.f ? m_fin + __log2f(l_tot) : kNegInf;
    if (a.S > 1) {
      float* dst = a.opart + ((size_t)split * a.B * a.N * rs) + head_off + (size_t)qrow * rs;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(float4*)(dst + 32 * mt + 8 * g + 4 * kg) = make_float4(o[mt][4 * g] * inv, o[mt][4 * g + 1] * inv,
                                                                    o[mt][4 * g + 2] * inv, o[mt][4 * g + 3] * inv);
      if (kg == 0) a.olse[((size_t)split * a.B * a.N + (size_t)b * a.N + qrow) * a.H + h] = lse2;
    } else if (a.out != nullptr) {
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
      if (a.lse != nullptr && kg == 0) a.lse[(size_t)bh * a.tp + qrow] = lse2;
    }
  }
}

// Stage 2's work order, first pass: the number of exact blocks of each query block within
// each 64-block routing chunk, decided exactly as the fused pass decides them (the same FMA
// sequence as proxy_dot, the same threshold test and sink rule), so that the counts are
// the fused pass's own.  A workgroup takes 16 query blocks, their fp32 means staged in LDS
// and read as broadcasts; each wave takes chunks w, w + 4, ..., two at a time so that each
// mean read feeds both; lane l scores key block 64 c + l.
__global__ __launch_bounds__(256) void count_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar_t,
                                                    const float* __restrict__ tau_i, int nb, int nbp, int sink_b0,
                                                    int sink_b1, uint8_t* __restrict__ wcnt) {
  __shared__ float4 qs[16][kDim / 4];
  const int bh = blockIdx.y, i0 = blockIdx.x * 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nchunks = nbp / 64;
  for (int t = threadIdx.x; t < 16 * kDim / 4; t += 256)     // rows i0 .. i0 + 15 < nbp
    qs[t >> 5][t & 31] = ((const float4*)(qbar + ((size_t)bh * nbp + i0) * kDim))[t];
  __syncthreads();
  const float4* kt = (const float4*)kbar_t + (size_t)bh * 32 * nbp;
  for (int c = w; c < nchunks; c += 8) {                  // chunks c and c + 4 together
    const bool two = c + 4 < nchunks;                     // uniform
    const int j0 = 64 * c + lane, j1 = two ? j0 + 256 : j0;
    float acc0[16], acc1[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc0[q] = acc1[q] = 0.f;
    for (int g = 0; g < 32; ++g) {
      const float4 kv0 = kt[(size_t)g * nbp + j0];
      const float4 kv1 = kt[(size_t)g * nbp + j1];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 qv = qs[q][g];
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
    int mine0 = 0, mine1 = 0;                            // lane q keeps query block i0 + q's counts
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float tau = tau_i[(size_t)bh * nbp + i0 + q];
      const uint64_t w0 = exact_word(__ballot(acc0[q] * kScale > tau), c, nb, sink_b0, sink_b1);
      const uint64_t w1 = exact_word(__ballot(acc1[q] * kScale > tau), two ? c + 4 : c, nb, sink_b0, sink_b1);
      if (lane == q) {
        mine0 = __builtin_popcountll(w0);
        mine1 = __builtin_popcountll(w1);
      }
    }
    if (lane < 16 && i0 + lane < nb) {
      wcnt[((size_t)bh * nchunks + c) * nbp + i0 + lane] = (uint8_t)mine0;
      if (two) wcnt[((size_t)bh * nchunks + c + 4) * nbp + i0 + lane] = (uint8_t)mine1;
    }
  }
}

// Second pass, one workgroup per (batch, head, key split): each query block's count over the
// split's routing chunks and a counting sort by descending count: a histogram of the counts,
// its scan from the largest count down, and one slot per block taken with an LDS atomic, so
// that the split's order[] is a permutation of 0 .. nb - 1 sorted by descending count
// (blocks with equal counts in any order: the order only schedules work, every block's
// result is the same).
__global__ __launch_bounds__(256) void order_kernel(const uint8_t* __restrict__ wcnt, int nb, int nbp, int cps,
                                                    int* __restrict__ qcount, int* __restrict__ order) {
  extern __shared__ int sm[];
  int* slot = sm;                                        // [nb + 1]
  unsigned short* qc = (unsigned short*)(sm + nb + 1);   // [nb] counts (<= nb <= 8192)
  __shared__ int part[256];
  const int sp = blockIdx.x, S = gridDim.x, bh = blockIdx.y, nchunks = nbp / 64, tid = threadIdx.x;
  const int c0 = sp * cps, c1 = min(nchunks, c0 + cps);
  const uint8_t* wc = wcnt + (size_t)bh * nchunks * nbp;
  const size_t row = ((size_t)bh * S + sp) * nbp;
  for (int i = tid; i < nb; i += 256) {
    int c = 0;
    for (int ch = c0; ch < c1; ++ch) c += wc[(size_t)ch * nbp + i];
    qc[i] = c;
    qcount[row + i] = c;
  }
  __syncthreads();
  sort_desc_counts(qc, slot, part, nb, order + row);
}

// Merge of the key-range splits: o = sum_s 2^(lse_s - lse) o_s / sum_s 2^(lse_s - lse), the
// fp32 partial rows o_s weighted by their softmax masses, rounded to bf16 once.  One thread
// per (row, 8 dims); partials are BTHD like the output.  With `lse` set, the first thread
// of each row also stores the merged log2-sum-exp at [b][h][n] (row stride tp).
__global__ __launch_bounds__(256) void merge_splits_kernel(const float4* __restrict__ opart,
                                                           const float* __restrict__ olse, int S,
                                                           size_t rows, uint4v* __restrict__ out,
                                                           float* __restrict__ lse, int N, int H, int tp) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * 16) return;
  const size_t row = t >> 4;
  float m = kNegInf;
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, olse[sp * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float ls = olse[sp * rows + row];
    const float wt = ls == kNegInf ? 0.f : __builtin_amdgcn_exp2f(ls - m);
    const float4 x0 = opart[(sp * rows * 16 + t) * 2];
    const float4 x1 = opart[(sp * rows * 16 + t) * 2 + 1];
    wsum += wt;
    acc[0] += wt * x0.x; acc[1] += wt * x0.y; acc[2] += wt * x0.z; acc[3] += wt * x0.w;
    acc[4] += wt * x1.x; acc[5] += wt * x1.y; acc[6] += wt * x1.z; acc[7] += wt * x1.w;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (lse != nullptr && (t & 15) == 0) {
    const size_t n = (row / H) % N, bq = row / ((size_t)H * N);
    lse[(bq * H + row % H) * tp + n] = wsum > 0.f ? m + __log2f(wsum) : kNegInf;
  }
  uint4v r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  out[t] = r;
}

// Clears the selected-pair counter on the stream (a kernel rather than a memset, so the
// call can also sit in a captured graph).
__global__ void zero_counter_kernel(unsigned long long* p) { *p = 0ull; }

hipError_t launch_order(Shape s, const Workspace& ws, int sink_b0, int sink_b1, hipStream_t stream) {
  if (ws.wcnt == nullptr || ws.qcount == nullptr || ws.order == nullptr) return hipSuccess;
  hipLaunchKernelGGL(count_kernel, dim3((ws.nb + 15) / 16, s.B * s.H), dim3(256), 0, stream, ws.qbar, ws.kbar_t,
                     ws.tau_i, ws.nb, ws.nbp, sink_b0, sink_b1, ws.wcnt);
  const int nchunks = ws.nbp / 64, S = ws.kv_splits, cps = (nchunks + S - 1) / S;
  hipLaunchKernelGGL(order_kernel, dim3(S, s.B * s.H), dim3(256),
                     (ws.nb + 1) * sizeof(int) + ws.nb * sizeof(unsigned short), stream, ws.wcnt, ws.nb, ws.nbp, cps,
                     ws.qcount, ws.order);
  return hipGetLastError();
}

hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                        Shape s, const Workspace& ws, int sink_b0, int sink_b1, uint64_t* mask_out,
                        unsigned long long* pairs, hipStream_t stream) {
  const int nchunks = ws.nbp / 64;
  const int S = ws.kv_splits;
  const int cps = (nchunks + S - 1) / S;
  if (cps > kMaxChunks || (S > 1 && (!ws.opart || !ws.olse)) || !ws.kh || !ws.vh || !ws.qbar || !ws.kbar_t ||
      !ws.tau_i)
    return hipErrorInvalidValue;
  FusedArgs a;
  a.q = q; a.out = out;   // k and v are read through stage 1's head-major copies
  a.B = s.B; a.N = s.N; a.H = s.H; a.nb = ws.nb; a.nbp = ws.nbp; a.nbw = (ws.nb + 63) / 64;
  a.S = S; a.cps = cps; a.opart = ws.opart; a.olse = ws.olse;
  a.kbar_h = ws.kbar_h; a.vbar_h = ws.vbar_h;
  a.kh = ws.kh; a.vh = ws.vh;
  a.qbar = ws.qbar; a.kbar_t = ws.kbar_t; a.tau_i = ws.tau_i;
  a.sink_b0 = sink_b0; a.sink_b1 = sink_b1; a.mask_out = mask_out;
  a.pairs = pairs;
  a.lse = ws.lse; a.tp = ws.nbp * kBlock;
  if (pairs != nullptr) {
    hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(1), 0, stream, pairs);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipError_t e1 = launch_order(s, ws, sink_b0, sink_b1, stream);
  if (e1 != hipSuccess) return e1;
  a.order = ws.order;
  const int total = s.B * s.H * S * ws.nb;
  hipLaunchKernelGGL(sol_fused_kernel, dim3(total), dim3(128), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1 || out == nullptr) return e;
  const size_t rows = (size_t)s.B * s.N * s.H;
  hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream,
                     (const float4*)ws.opart, ws.olse, S, rows, (uint4v*)out, ws.lse, s.N, s.H, ws.nbp * kBlock);
  return hipGetLastError();
}

}  // namespace solattn
