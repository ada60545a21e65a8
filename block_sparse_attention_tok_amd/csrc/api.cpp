// C-ABI entry points of libsolattn: host-side validation, workspace layout and
// launch sequencing.  Declarations and argument documentation: include/solattn.h.
#include "../../include/solattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

constexpr int64_t kBlock = 64;
constexpr int64_t kDim = 128;
constexpr int64_t kMaxIndex = (int64_t)1 << 31;
constexpr int64_t kMaxTokens = (int64_t)1 << 19;   // 524288: 128 routing chunks

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int check_shape(int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim) {
  if (batch < 1 || tokens < 1 || heads < 1) return SOL_ERR_SHAPE;
  if (head_dim != kDim) return SOL_ERR_HEAD_DIM;
  // element offsets and grid sizes stay inside 32-bit block counts / 64-bit offsets
  const int64_t nb = (tokens + kBlock - 1) / kBlock;
  if (tokens > kMaxTokens || heads >= 65536 || batch >= 65536) return SOL_ERR_SHAPE;
  if (batch * heads * nb * 16 >= kMaxIndex) return SOL_ERR_SHAPE;
  // one head's rows of one batch, padded to whole 64-row blocks, must fit a 32-bit
  // buffer range (tile loads address up to 63 rows past the last token)
  if ((nb * kBlock - 1) * heads * kDim * 2 + kDim * 2 > (int64_t)0xFFFFFFFF) return SOL_ERR_SHAPE;
  return SOL_OK;
}

int sink_range(int64_t tokens, int64_t sink_start, int64_t sink_tokens, int* b0, int* b1) {
  *b0 = 1;
  *b1 = 0;                                    // empty range
  if (sink_tokens < 0) return SOL_ERR_SINK;
  if (sink_tokens == 0) return SOL_OK;
  const int64_t s = sink_start < 0 ? tokens - sink_tokens : sink_start;
  if (s < 0 || s + sink_tokens > tokens) return SOL_ERR_SINK;
  *b0 = (int)(s / kBlock);
  *b1 = (int)((s + sink_tokens - 1) / kBlock);
  return SOL_OK;
}

constexpr int kMaxSplits = 16;
// Automatic split counts stay at or below this: each split keeps an fp32 partial row per
// (token, head) (512 bytes), so 4 splits hold at most twice the bytes of q, k, v and out.
constexpr int kMaxAutoSplits = 4;

// Effective split count: splits cover whole 64-block routing chunks.
int effective_splits(int64_t tokens, int requested) {
  const int64_t nb = (tokens + kBlock - 1) / kBlock;
  const int nchunks = (int)((nb + 63) / 64);
  int want = requested;
  if (want <= 0) {
    // automatic: none up to 8 chunks (the split merge costs more than it saves there), then
    // one split per six chunks, at most kMaxAutoSplits
    want = nchunks <= 8 ? 1 : (nchunks + 5) / 6;
    if (want > kMaxAutoSplits) want = kMaxAutoSplits;
  }
  if (want > kMaxSplits) want = kMaxSplits;
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  const int cps = (nchunks + want - 1) / want;            // chunks per split
  return (nchunks + cps - 1) / cps;
}

int layout(int variant, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim, sol_ws_layout* L,
           int kv_splits = 0) {
  int st = check_shape(batch, tokens, heads, head_dim);
  if (st != SOL_OK) return st;
  if (variant != SOL_VARIANT_SOL1 && variant != SOL_VARIANT_SOL2 && variant != SOL_VARIANT_SOL2_PV8 &&
      variant != SOL_VARIANT_SOL1_TRAIN && variant != SOL_VARIANT_SOL2_TRAIN)
    return SOL_ERR_ARG;
  std::memset(L, 0xff, sizeof(*L));          // every offset -1
  const int64_t nb = (tokens + kBlock - 1) / kBlock;
  const int64_t nbp = (nb + 63) / 64 * 64;
  const int64_t bh = batch * heads;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { int64_t o = off; off = align256(off + bytes); return o; };
  L->nb = nb;
  L->nbp = nbp;
  L->qbar = take(bh * nbp * kDim * 4);
  L->kbar_t = take(bh * nbp * kDim * 4);
  L->kbar_h = take(bh * nbp * kDim * 2);
  L->vbar_h = take(bh * nbp * kDim * 2);
  L->tau_i = take(bh * nbp * 4);
  L->kstat = take(bh * 2 * kDim * 4);
  L->kcov = take(bh * kDim * kDim * 4);
  L->kpart = take(bh * 16 * 2 * kDim * 8);
  L->kcovp = take(bh * 8 * kDim * kDim * 4);
  // Sol-Attn: head-major copies of K and V written by stage 1, the tile source of stage 2
  if (variant == SOL_VARIANT_SOL1 || variant == SOL_VARIANT_SOL1_TRAIN) {
    L->kh = take(bh * tokens * kDim * 2);
    L->vh = take(bh * tokens * kDim * 2);
    // stage 2's work order: exact-block counts per routing chunk and query block, their
    // sums over each key split's chunks, and each (head, split)'s query blocks by descending
    // count
    const int64_t splits = effective_splits(tokens, kv_splits);
    L->wcnt = take(bh * (nbp / 64) * nbp);
    L->qcount = take(bh * splits * nbp * 4);
    L->order = take(bh * splits * nbp * 4);
  }
  const bool sol2 = variant == SOL_VARIANT_SOL2 || variant == SOL_VARIANT_SOL2_PV8 || variant == SOL_VARIANT_SOL2_TRAIN;
  if (sol2) {
    const int64_t tp = nbp * kBlock;
    L->q8 = take(bh * tp * kDim);
    L->k8 = take(bh * tp * kDim);
    L->qscale = take(bh * nbp * 4);
    L->kscale = take(bh * nbp * 4);
    L->qhat = take(bh * kDim * 4);
    L->gk = take(bh * nbp * 2 * kDim * 2);
    L->gv = take(bh * nbp * 2 * kDim * 2);
    L->glogn = take(bh * nbp * 2 * 4);
    L->ghi = take(bh * nbp * 8);
    L->qanc = take(bh * nbp * 2 * kDim * 4);
    L->tmu = take(bh * nbp * 2 * kDim * 4);
    L->tnu = take(bh * nbp * 2 * kDim * 4);
    L->tlz = take(bh * nbp * 2 * 4);
    if (variant == SOL_VARIANT_SOL2_PV8) {
      L->v8t = take(bh * kDim * tp);
      L->vbmax = take(bh * nbp * 4);
      L->vscale = take(bh * 4);
    }
  }
  // split-KV partials (Sol-Attn only)
  const bool sol1 = variant == SOL_VARIANT_SOL1 || variant == SOL_VARIANT_SOL1_TRAIN;
  L->kv_splits = sol1 ? effective_splits(tokens, kv_splits) : 1;
  if (L->kv_splits > 1) {
    L->opart = take(L->kv_splits * bh * tokens * kDim * 4);
    L->olse = take(L->kv_splits * bh * tokens * 4);
  }
  // forward state for the backward, and backward scratch (Sol-Attn2 training)
  if (variant == SOL_VARIANT_SOL2_TRAIN) {
    const int64_t tp = nbp * kBlock;
    L->sel = take(bh * nb * (nbp / 64) * 8);
    L->lse = take(bh * tp * 4);
    L->ofp = take(bh * tp * kDim * 4);
    L->mcol = take(bh * nb * (nbp / 64) * 8);
    L->ld = take(bh * tp * 2 * 4);
    L->kh = take(bh * tokens * kDim * 2);
    L->vh = take(bh * tokens * kDim * 2);
    L->qd = take(bh * tokens * kDim * 2);
    L->kd = take(bh * tokens * kDim * 2);
    L->dlam = take(bh * tp * 4);
    L->qab = take(bh * 2 * nbp * kDim * 2);
    L->dmub = take(bh * 2 * nbp * kDim * 2);
    L->dnub = take(bh * 2 * nbp * kDim * 2);
    L->alz = take(bh * 2 * nbp * 2 * 4);
    L->aextra = take(bh * 2 * nbp * kDim * 4);
    L->gdk = take(bh * nbp * 2 * kDim * 4);
    L->gdv = take(bh * nbp * 2 * kDim * 4);
    L->bqord = take(bh * nbp * 4);
    L->bkord = take(bh * nbp * 4);
  }
  // forward state for the backward, and backward scratch (Sol-Attn training)
  if (variant == SOL_VARIANT_SOL1_TRAIN) {
    const int64_t tp = nbp * kBlock;
    L->lse = take(bh * tp * 4);
    L->mrow = take(bh * nb * (nbp / 64) * 8);
    L->mcol = take(bh * nb * (nbp / 64) * 8);
    L->ld = take(bh * tp * 2 * 4);
    L->dkbar = take(bh * nbp * kDim * 4);
    L->dvbar = take(bh * nbp * kDim * 4);
    L->bqord = take(bh * nbp * 4);
    L->bkord = take(bh * nbp * 4);
  }
  L->total_bytes = off;
  return SOL_OK;
}

solattn::Workspace resolve(const sol_ws_layout& L, void* ws) {
  char* base = (char*)ws;
  auto at = [&](int64_t o) -> char* { return o < 0 ? nullptr : base + o; };
  solattn::Workspace w;
  w.nb = (int)L.nb;
  w.nbp = (int)L.nbp;
  w.qbar = (float*)at(L.qbar);
  w.kbar_t = (float*)at(L.kbar_t);
  w.kbar_h = (uint16_t*)at(L.kbar_h);
  w.kh = (uint16_t*)at(L.kh);
  w.vh = (uint16_t*)at(L.vh);
  w.vbar_h = (uint16_t*)at(L.vbar_h);
  w.tau_i = (float*)at(L.tau_i);
  w.kstat = (float*)at(L.kstat);
  w.kcov = (float*)at(L.kcov);
  w.kpart = (double*)at(L.kpart);
  w.q8 = (uint8_t*)at(L.q8);
  w.k8 = (uint8_t*)at(L.k8);
  w.qscale = (float*)at(L.qscale);
  w.kscale = (float*)at(L.kscale);
  w.qhat = (float*)at(L.qhat);
  w.gk = (uint16_t*)at(L.gk);
  w.gv = (uint16_t*)at(L.gv);
  w.glogn = (float*)at(L.glogn);
  w.ghi = (uint64_t*)at(L.ghi);
  w.qanc = (float*)at(L.qanc);
  w.kv_splits = (int)L.kv_splits;
  w.opart = (float*)at(L.opart);
  w.olse = (float*)at(L.olse);
  w.sel = (uint64_t*)at(L.sel);
  w.tmu = (float*)at(L.tmu);
  w.tnu = (float*)at(L.tnu);
  w.tlz = (float*)at(L.tlz);
  w.v8t = (uint8_t*)at(L.v8t);
  w.vbmax = (float*)at(L.vbmax);
  w.vscale = (float*)at(L.vscale);
  w.lse = (float*)at(L.lse);
  w.mrow = (uint64_t*)at(L.mrow);
  w.mcol = (uint64_t*)at(L.mcol);
  w.ld = (float*)at(L.ld);
  w.dkbar = (float*)at(L.dkbar);
  w.dvbar = (float*)at(L.dvbar);
  w.qd = (uint16_t*)at(L.qd);
  w.kd = (uint16_t*)at(L.kd);
  w.dlam = (float*)at(L.dlam);
  w.qab = (uint16_t*)at(L.qab);
  w.dmub = (uint16_t*)at(L.dmub);
  w.dnub = (uint16_t*)at(L.dnub);
  w.alz = (float*)at(L.alz);
  w.aextra = (float*)at(L.aextra);
  w.gdk = (float*)at(L.gdk);
  w.gdv = (float*)at(L.gdv);
  w.ofp = (float*)at(L.ofp);
  w.kcovp = (float*)at(L.kcovp);
  w.wcnt = (uint8_t*)at(L.wcnt);
  w.qcount = (int*)at(L.qcount);
  w.order = (int*)at(L.order);
  w.bqord = (int*)at(L.bqord);
  w.bkord = (int*)at(L.bkord);
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Common argument checks; fills the layout on success.
int prologue(int variant, const void* q, const void* k, const void* v, int64_t batch, int64_t tokens,
             int64_t heads, int64_t head_dim, void* workspace, size_t workspace_bytes, sol_ws_layout* L,
             int kv_splits = 0) {
  if (!q || !k || !v || !workspace) return SOL_ERR_NULL;
  int st = layout(variant, batch, tokens, heads, head_dim, L, kv_splits);
  if (st != SOL_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || ((uintptr_t)workspace & 255)) return SOL_ERR_ARG;
  if ((int64_t)workspace_bytes < L->total_bytes) return SOL_ERR_WORKSPACE;
  return SOL_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SOL_OK : SOL_ERR_HIP; }

solattn::Shape shape_of(int64_t batch, int64_t tokens, int64_t heads) {
  return solattn::Shape{(int)batch, (int)tokens, (int)heads};
}

int check_kv(int kv_splits) { return (kv_splits >= 0 && kv_splits <= kMaxSplits) ? SOL_OK : SOL_ERR_ARG; }

int check_thresh(int thresh) { return (thresh == SOL_THRESH_DIAG || thresh == SOL_THRESH_EXACT) ? SOL_OK : SOL_ERR_ARG; }

}  // namespace

extern "C" {

const char* sol_status_string(int status) {
  switch (status) {
    case SOL_OK: return "ok";
    case SOL_ERR_NULL: return "null pointer argument";
    case SOL_ERR_SHAPE: return "invalid shape (batch, tokens and heads must be >= 1 and fit the index range)";
    case SOL_ERR_HEAD_DIM: return "head_dim must be 128";
    case SOL_ERR_TAU: return "tau must be finite";
    case SOL_ERR_SINK: return "sink range must lie inside [0, tokens) and sink_tokens must be >= 0";
    case SOL_ERR_WORKSPACE: return "workspace smaller than sol_attn_workspace_bytes()";
    case SOL_ERR_HIP: return "HIP runtime or kernel launch error";
    case SOL_ERR_ARG: return "invalid argument (threshold type, variant or pointer alignment)";
    case SOL_ERR_SCRATCH:
      return "the shape needs more workspace than sol_attn_noalloc's static scratch holds "
             "(SOL_NOALLOC_SCRATCH_BYTES); use sol_attn with a caller workspace";
    default: return "unknown status";
  }
}

int sol_attn_validate(int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim, float tau,
                      int64_t sink_start, int64_t sink_tokens, int thresh) {
  int st = check_shape(batch, tokens, heads, head_dim);
  if (st != SOL_OK) return st;
  if (!std::isfinite(tau)) return SOL_ERR_TAU;
  int b0, b1;
  st = sink_range(tokens, sink_start, sink_tokens, &b0, &b1);
  if (st != SOL_OK) return st;
  return check_thresh(thresh);
}

size_t sol_attn_workspace_bytes(int variant, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim) {
  sol_ws_layout L;
  if (layout(variant, batch, tokens, heads, head_dim, &L) != SOL_OK) return 0;
  return (size_t)L.total_bytes;
}

int sol_attn_workspace_layout(int variant, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                              sol_ws_layout* out) {
  if (!out) return SOL_ERR_NULL;
  return layout(variant, batch, tokens, heads, head_dim, out);
}

int sol_attn_kv_splits(int64_t batch, int64_t tokens, int64_t heads, int kv_splits) {
  if (check_shape(batch, tokens, heads, kDim) != SOL_OK || check_kv(kv_splits) != SOL_OK) return 0;
  return effective_splits(tokens, kv_splits);
}

size_t sol_attn_workspace_bytes_kv(int variant, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                                   int kv_splits) {
  sol_ws_layout L;
  if (check_kv(kv_splits) != SOL_OK) return 0;
  if (layout(variant, batch, tokens, heads, head_dim, &L, kv_splits) != SOL_OK) return 0;
  return (size_t)L.total_bytes;
}

int sol_attn_workspace_layout_kv(int variant, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                                 int kv_splits, sol_ws_layout* out) {
  if (!out) return SOL_ERR_NULL;
  if (check_kv(kv_splits) != SOL_OK) return SOL_ERR_ARG;
  return layout(variant, batch, tokens, heads, head_dim, out, kv_splits);
}

int sol_attn_prepare(const void* q, const void* k, const void* v, int64_t batch, int64_t tokens, int64_t heads,
                     int64_t head_dim, float tau, int thresh, void* workspace, size_t workspace_bytes,
                     void* stream) {
  sol_ws_layout L;
  // the split-KV partials sit at the end of the layout and stage 1 does not use them
  int st = prologue(SOL_VARIANT_SOL1, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L, 1);
  if (st != SOL_OK) return st;
  if (!std::isfinite(tau)) return SOL_ERR_TAU;
  if ((st = check_thresh(thresh)) != SOL_OK) return st;
  solattn::Workspace w = resolve(L, workspace);
  solattn::Shape s = shape_of(batch, tokens, heads);
  hipStream_t hs = (hipStream_t)stream;
  st = hip_status(solattn::launch_summary((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s, w, hs));
  if (st != SOL_OK) return st;
  // the routing itself happens inside the fused kernel of stage 2
  return hip_status(solattn::launch_threshold(s, w, tau, thresh == SOL_THRESH_EXACT, hs));
}

// Sol-Attn2 stage 2 parts: the routing + tail pass, the exact pass, or both in order.
enum { kStage2Tail = 1, kStage2Exact = 2, kStage2Both = 3 };

static int fused_common(int variant, const void* q, const void* k, const void* v, void* out, int64_t batch,
                        int64_t tokens, int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens,
                        void* workspace, size_t workspace_bytes, uint64_t* mask_bits, void* stream,
                        bool out_required, int kv_splits = 0, int stage2 = kStage2Both,
                        uint64_t* selected_pairs = nullptr) {
  sol_ws_layout L;
  if (check_kv(kv_splits) != SOL_OK) return SOL_ERR_ARG;
  int st = prologue(variant, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L, kv_splits);
  if (st != SOL_OK) return st;
  if (out_required && !out) return SOL_ERR_NULL;
  if (out && !aligned16(out)) return SOL_ERR_ARG;
  int b0, b1;
  if ((st = sink_range(tokens, sink_start, sink_tokens, &b0, &b1)) != SOL_OK) return st;
  solattn::Workspace w = resolve(L, workspace);
  solattn::Shape s = shape_of(batch, tokens, heads);
  if (variant == SOL_VARIANT_SOL1 || variant == SOL_VARIANT_SOL1_TRAIN)
    return hip_status(solattn::launch_fused((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                            (uint16_t*)out, s, w, b0, b1, mask_bits ? mask_bits : w.mrow,
                                            (unsigned long long*)selected_pairs, (hipStream_t)stream));
  hipStream_t hs = (hipStream_t)stream;
  if (stage2 & kStage2Tail) {
    if ((st = hip_status(solattn::launch_tail2(s, w, b0, b1, hs))) != SOL_OK) return st;
  }
  if (!(stage2 & kStage2Exact)) return SOL_OK;
  // the exact pass exports its routing words for the test export and the training forward
  uint64_t* words = mask_bits ? mask_bits : (variant == SOL_VARIANT_SOL2_TRAIN ? w.sel : nullptr);
  return hip_status(solattn::launch_fused2((const uint16_t*)v, (uint16_t*)out, s, w,
                                           variant == SOL_VARIANT_SOL2_PV8, (unsigned long long*)selected_pairs,
                                           b0, b1, words, hs));
}

int sol_attn_fused(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                   int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return fused_common(SOL_VARIANT_SOL1, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, true);
}

int sol_attn_fused_kv(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                      int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens, int kv_splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return fused_common(SOL_VARIANT_SOL1, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, false, kv_splits);
}

int sol_attn(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens, int64_t heads,
             int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens, int thresh, void* workspace,
             size_t workspace_bytes, void* stream) {
  if (!out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  st = sol_attn_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return sol_attn_fused(q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens, workspace,
                        workspace_bytes, stream);
}

int sol_attn_forward_train(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                           int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens,
                           int thresh, void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  sol_ws_layout L;
  st = prologue(SOL_VARIANT_SOL1_TRAIN, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L);
  if (st != SOL_OK) return st;
  st = sol_attn_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return fused_common(SOL_VARIANT_SOL1_TRAIN, q, k, v, out, batch, tokens, heads, head_dim, sink_start,
                      sink_tokens, workspace, workspace_bytes, nullptr, stream, true);
}

int sol_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, void* dq,
                      void* dk, void* dv, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !dout || !dq || !dk || !dv) return SOL_ERR_NULL;
  sol_ws_layout L;
  int st = prologue(SOL_VARIANT_SOL1_TRAIN, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L);
  if (st != SOL_OK) return st;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return SOL_ERR_ARG;
  solattn::Workspace w = resolve(L, workspace);
  return hip_status(solattn::launch_backward((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                             (const uint16_t*)out, (const uint16_t*)dout, (uint16_t*)dq,
                                             (uint16_t*)dk, (uint16_t*)dv, shape_of(batch, tokens, heads), w,
                                             (hipStream_t)stream));
}

int sol_attn_debug_routing(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                           int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens,
                           int thresh, int kv_splits, void* workspace, size_t workspace_bytes, uint64_t* mask_bits,
                           uint64_t* selected_pairs, void* stream) {
  if (!mask_bits) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  if ((st = check_kv(kv_splits)) != SOL_OK) return st;
  st = sol_attn_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return fused_common(SOL_VARIANT_SOL1, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, mask_bits, stream, false, kv_splits, kStage2Both, selected_pairs);
}

static int prepare2(int variant, const void* q, const void* k, const void* v, int64_t batch, int64_t tokens,
                    int64_t heads, int64_t head_dim, float tau, int thresh, void* workspace, size_t workspace_bytes,
                    void* stream) {
  sol_ws_layout L;
  int st = prologue(variant, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L);
  if (st != SOL_OK) return st;
  if (!std::isfinite(tau)) return SOL_ERR_TAU;
  if ((st = check_thresh(thresh)) != SOL_OK) return st;
  solattn::Workspace w = resolve(L, workspace);
  solattn::Shape s = shape_of(batch, tokens, heads);
  hipStream_t hs = (hipStream_t)stream;
  st = hip_status(solattn::launch_quant_summary((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s, w, hs));
  if (st != SOL_OK) return st;
  st = hip_status(solattn::launch_threshold(s, w, tau, thresh == SOL_THRESH_EXACT, hs));
  if (st != SOL_OK) return st;
  st = hip_status(solattn::launch_qhat(s, w, hs));
  if (st != SOL_OK) return st;
  st = hip_status(solattn::launch_groups((const uint16_t*)v, s, w, hs));
  if (st != SOL_OK || variant != SOL_VARIANT_SOL2_PV8) return st;
  return hip_status(solattn::launch_vquant((const uint16_t*)v, s, w, hs));
}

int sol_attn2_prepare(const void* q, const void* k, const void* v, int64_t batch, int64_t tokens, int64_t heads,
                      int64_t head_dim, float tau, int thresh, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return prepare2(SOL_VARIANT_SOL2, q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace,
                  workspace_bytes, stream);
}

int sol_attn2_pv8_prepare(const void* q, const void* k, const void* v, int64_t batch, int64_t tokens,
                          int64_t heads, int64_t head_dim, float tau, int thresh, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return prepare2(SOL_VARIANT_SOL2_PV8, q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace,
                  workspace_bytes, stream);
}

int sol_attn2_pv8_exact(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                        int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return fused_common(SOL_VARIANT_SOL2_PV8, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, true, 0, kStage2Exact);
}

int sol_attn2_pv8(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                  int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  st = sol_attn2_pv8_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes,
                             stream);
  if (st != SOL_OK) return st;
  return fused_common(SOL_VARIANT_SOL2_PV8, q, k, v, out, batch, tokens, heads, head_dim, sink_start,
                      sink_tokens, workspace, workspace_bytes, nullptr, stream, true, 0, kStage2Both);
}

int sol_attn2_fused(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                    int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return fused_common(SOL_VARIANT_SOL2, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, true);
}

int sol_attn2_tail(const void* q, const void* k, const void* v, int64_t batch, int64_t tokens, int64_t heads,
                   int64_t head_dim, int64_t sink_start, int64_t sink_tokens, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return fused_common(SOL_VARIANT_SOL2, q, k, v, nullptr, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, false, 0, kStage2Tail);
}

int sol_attn2_exact(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                    int64_t heads, int64_t head_dim, int64_t sink_start, int64_t sink_tokens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return fused_common(SOL_VARIANT_SOL2, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, nullptr, stream, true, 0, kStage2Exact);
}

int sol_attn2(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens, int64_t heads,
              int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens, int thresh, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  st = sol_attn2_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return sol_attn2_fused(q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens, workspace,
                         workspace_bytes, stream);
}

int sol_attn2_forward_train(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                            int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens,
                            int thresh, void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  st = prepare2(SOL_VARIANT_SOL2_TRAIN, q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace,
                workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return fused_common(SOL_VARIANT_SOL2_TRAIN, q, k, v, out, batch, tokens, heads, head_dim, sink_start,
                      sink_tokens, workspace, workspace_bytes, nullptr, stream, true);
}

int sol_attn2_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, void* dq,
                       void* dk, void* dv, int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !dout || !dq || !dk || !dv) return SOL_ERR_NULL;
  sol_ws_layout L;
  int st = prologue(SOL_VARIANT_SOL2_TRAIN, q, k, v, batch, tokens, heads, head_dim, workspace, workspace_bytes, &L);
  if (st != SOL_OK) return st;
  if (!aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return SOL_ERR_ARG;
  solattn::Workspace w = resolve(L, workspace);
  return hip_status(solattn::launch_backward2((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                              (const uint16_t*)out, (const uint16_t*)dout, (uint16_t*)dq,
                                              (uint16_t*)dk, (uint16_t*)dv, shape_of(batch, tokens, heads), w,
                                              (hipStream_t)stream));
}

int sol_attn2_debug_routing(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                            int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens,
                            int thresh, int kv_splits, void* workspace, size_t workspace_bytes, uint64_t* mask_bits,
                            uint64_t* selected_pairs, void* stream) {
  if (!mask_bits) return SOL_ERR_NULL;
  if (kv_splits != 0 && kv_splits != 1) return SOL_ERR_ARG;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  st = sol_attn2_prepare(q, k, v, batch, tokens, heads, head_dim, tau, thresh, workspace, workspace_bytes, stream);
  if (st != SOL_OK) return st;
  return fused_common(SOL_VARIANT_SOL2, q, k, v, out, batch, tokens, heads, head_dim, sink_start, sink_tokens,
                      workspace, workspace_bytes, mask_bits, stream, false, 0, kStage2Both, selected_pairs);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// sol_attn_noalloc: sol_attn on a workspace held in a static device array, for callers
// that cannot allocate.  Each device that runs it holds its own copy of `scratch` until
// the process ends.  The array's name is only a host-side stand-in: its device address
// comes from hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to the kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SOL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];            // device address of `scratch` per device, once set up

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SOL_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SOL_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SOL_OK;
}

}  // namespace

extern "C" {

int sol_attn_noalloc(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t tokens,
                     int64_t heads, int64_t head_dim, float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                     void* stream) {
  if (!q || !k || !v || !out) return SOL_ERR_NULL;
  int st = sol_attn_validate(batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh);
  if (st != SOL_OK) return st;
  const size_t need = sol_attn_workspace_bytes(SOL_VARIANT_SOL1, batch, tokens, heads, head_dim);
  if (need == 0) return SOL_ERR_SHAPE;
  if (need > (size_t)SOL_NOALLOC_SCRATCH_BYTES) return SOL_ERR_SCRATCH;
  // Every array of the workspace is written by the call before it is read, so the
  // previous call's contents need no clearing.
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != SOL_OK) return st;
  return sol_attn(q, k, v, out, batch, tokens, heads, head_dim, tau, sink_start, sink_tokens, thresh, ws,
                  (size_t)SOL_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
