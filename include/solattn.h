/*
 * libsolattn -- Sol-Attn and Sol-Attn2 forward passes for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a plain address; the header says for each
 * whether it is host or device memory.  No call allocates device memory: the
 * caller passes a device workspace of at least sol_attn_workspace_bytes().
 * Launches are asynchronous on the caller's HIP stream (`stream` is a
 * hipStream_t passed as void*, NULL = the legacy default stream); the library
 * keeps no pointer after a call returns and holds no global state apart from
 * the loaded code object.  Calls that share a workspace must not overlap.
 *
 * Tensor contract (Sol-Attn README, "Usage" and "Core API"): q, k, v and out
 * are contiguous bfloat16 tensors of shape [batch, tokens, heads, head_dim]
 * (BTHD), head_dim == 128, all of the same shape; out is written in the same
 * layout.  The attention is non-causal and unmasked (stable-diffusion.cpp
 * "Sol-Attn" docs, "Use").
 *
 * Errors (stable-diffusion.cpp "Sol-Attn" docs: a non-finite threshold is
 * rejected, execution errors are never turned into dense attention): every
 * argument error is detected on the host before any launch and returned as a
 * sol_status; nothing is launched then and outputs are untouched.  A HIP
 * launch error is returned as SOL_ERR_HIP.  There is no fallback path.
 */
#ifndef SOLATTN_H
#define SOLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SOL_OK = 0,
    SOL_ERR_NULL = 1,        /* a required pointer is NULL */
    SOL_ERR_SHAPE = 2,       /* batch/tokens/heads < 1, tokens > 524288, or one head's rows
                                of one batch, padded to a multiple of 64, span more than 4 GiB */
    SOL_ERR_HEAD_DIM = 3,    /* head_dim != 128 */
    SOL_ERR_TAU = 4,         /* tau is NaN or infinite */
    SOL_ERR_SINK = 5,        /* sink_tokens < 0, or the sink range leaves [0, tokens) */
    SOL_ERR_WORKSPACE = 6,   /* workspace smaller than sol_attn_workspace_bytes() */
    SOL_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
    SOL_ERR_ARG = 8,         /* unknown threshold type or variant, bad alignment */
    SOL_ERR_SCRATCH = 9      /* sol_attn_noalloc: the shape's workspace exceeds its static scratch */
} sol_status;

/* Size of the static device scratch behind sol_attn_noalloc (128 MiB per device). */
#define SOL_NOALLOC_SCRATCH_BYTES (128u << 20)

/* Threshold estimator (Sol-Attn paper §3.1 Eq. (5) and its appendix
 * "Diagonal threshold estimator").  DIAG is the default hot path. */
typedef enum { SOL_THRESH_DIAG = 0, SOL_THRESH_EXACT = 1 } sol_thresh;

/* Variants for sol_attn_workspace_bytes / sol_attn_workspace_layout. */
typedef enum {
    SOL_VARIANT_SOL1 = 1,      /* Sol-Attn */
    SOL_VARIANT_SOL2 = 2,      /* Sol-Attn2: FP8 Q/K, bf16 V */
    SOL_VARIANT_SOL2_PV8 = 3,  /* Sol-Attn2 with ExpCast P and per-head FP8 V (FP8 PV) */
    SOL_VARIANT_SOL1_TRAIN = 4, /* Sol-Attn forward that keeps its state for sol_attn_backward */
    SOL_VARIANT_SOL2_TRAIN = 5  /* Sol-Attn2 forward that keeps its state for sol_attn2_backward */
} sol_variant;

/* Byte offsets into the workspace of the intermediate arrays (for tests and
 * tooling; the kernels own these arrays during a call).  nbp = number of
 * 64-token blocks rounded up to a multiple of 64; tp = nbp * 64.  An offset
 * of -1 means the array does not exist for the variant.  Arrays are indexed
 * [batch][head][...] unless shown otherwise.
 *   qbar     float [B][H][nbp][128]   Q block means (Sol-Attn2: of dequantized Q)
 *   kbar_t   float [B][H][32][nbp][4] K block means, 4-dim-interleaved
 *   kbar_h   bf16  [B][H][nbp][128]   K block means (MFMA operand)
 *   vbar_h   bf16  [B][H][nbp][128]   V block means V-hat_j / n_j (MFMA operand)
 *   tau_i    float [B][H][nbp]        per-query-block threshold tau_i
 *   kstat    float [B][H][2][128]     mu_K and v_K
 *   kcov     float [B][H][128][128]   covariance of the K block means (EXACT only)
 *   kpart    double [B][H][16][2][128] partial sums of K block means and their squares
 *   kcovp    float  [B][H][8][128][128] per-slice sums of the centred outer products of the
 *            K block means (thresh = SOL_THRESH_EXACT only)
 *   kh, vh   bf16  [B][H][N][128]     Sol-Attn: head-major copies of K and V (stage 1 writes
 *                                      them; stage 2 and the backward stream tiles from them)
 *   wcnt     uint8 [B][H][nbp/64][nbp] Sol-Attn: exact blocks of each query block within each
 *                                      64-block routing chunk (sink included), written by stage 2
 *                                      before its fused pass
 *   qcount   int32 [B][H][S][nbp]     Sol-Attn: exact blocks of each query block among the
 *                                      routing chunks of key split s (S = kv_splits)
 *   order    int32 [B][H][S][nbp]     Sol-Attn: the nb query blocks by descending qcount per
 *                                      (head, split) (equal counts in any order), the order in
 *                                      which the fused pass takes its work items; not a routing
 *                                      map: the fused pass still decides every block on chip
 *   q8, k8   uint8 [B][H][tp][128]    E4M3FN codes (Sol-Attn2)
 *   qscale, kscale float [B][H][nbp]  E4M3 block scales (Sol-Attn2)
 *   qhat     float [B][H][128]        mean-query direction (Sol-Attn2)
 *   gk, gv   bf16  [B][H][nbp][2][128] group mean keys / values (Sol-Attn2)
 *   glogn    float [B][H][nbp][2]     ln n_g, -inf for an empty group (Sol-Attn2)
 *   ghi      uint64 [B][H][nbp]       bit u set iff token u of the block is in G_hi (Sol-Attn2)
 *   qanc     float [B][H][nbp][2][128] 32-token anchor means of dequantized Q (Sol-Attn2)
 *   opart    float [S][B][N][H][128]   per-key-split normalized partial outputs (S = kv_splits > 1),
 *                                      fp32 so that the merge rounds each output to bf16 once
 *   olse     float [S][B][N][H]        per-key-split log2-sum-exp of the partial rows
 *   (No layout has a routing array for the forward: each fused kernel decides its blocks
 *   on chip.  The Sol-Attn2 training layout keeps the forward's words in sel, below.)
 *   tmu, tnu float [B][H][nbp][2][128] per-anchor tail key / value means mu_a, nu_a (Sol-Attn2)
 *   tlz      float [B][H][nbp][2]     log2 Z_a - log2(e) qbar_a . mu_a / sqrt(d); -inf if the
 *                                      anchor's tail is empty (Sol-Attn2)
 *   v8t      uint8 [B][H][128][tp]    E4M3 codes of V / s_V, dim-major; within each 64-token
 *                                      block, token 32 h + 8 q + 4 g + r sits at position
 *                                      32 g + 16 h + 4 q + r (the FP8 PV operand order;
 *                                      SOL_VARIANT_SOL2_PV8 only, like vbmax and vscale)
 *   vbmax    float [B][H][nbp]        max |V| per 64-token block
 *   vscale   float [B][H]             s_V = max |V| / 448 per head (1 for an all-zero head)
 *   lse      float [B][H][tp]         base-2 log of each query row's softmax denominator, in
 *                                      units of log2(e) q.k / sqrt(d) (SOL_VARIANT_SOL1_TRAIN,
 *                                      like the arrays below; written by sol_attn_forward_train)
 *   mrow     uint64 [B][H][nb][nbp/64] the forward's routing bits, one row per query block
 *   mcol     uint64 [B][H][nb][nbp/64] the same bits by key block (backward scratch)
 *   ld       float [B][H][tp][2]      (lse, dO . O) per query row (backward scratch)
 *   dkbar, dvbar float [B][H][nbp][128] gradients w.r.t. the pooled keys (times 1/sqrt(d))
 *                                      and pooled values (backward scratch)
 *   bqord, bkord int32 [B][H][nbp]   the backward's work orders (scratch; both training
 *                                      layouts): query blocks by descending number of exact key
 *                                      blocks, key blocks by descending number of query blocks
 *                                      that select them (equal counts in any order)
 * SOL_VARIANT_SOL2_TRAIN (the Sol-Attn2 arrays above, then): sel uint64 [B][H][nb][nbp/64]
 * (the routing words the forward's exact pass decided, bit j % 64 of word j / 64 set iff
 * block j is exact for query block i, sink included), lse and ld as for Sol-Attn
 * training (lse written by sol_attn2_forward_train), ofp float [B][H][tp][128] (the
 * forward's output rows before rounding to bf16, so that the backward's D_t = dO_t . O_t
 * does not inherit the output's rounding), mcol (sel by key block), kh / vh (dequantized
 * k' and v head-major), and the backward scratch
 *   qd, kd   bf16  [B][N][H][128]     dequantized q', k' (BTHD)
 *   dlam     float [B][H][tp]         gradient w.r.t. each row's tail logit
 *   qab, dmub, dnub bf16 [B][H][2 nbp][128] anchor means and the gradients w.r.t. mu_a, nu_a
 *   alz      float [B][H][2 nbp][2]   (log2 Z_a, -c_a) per anchor
 *   aextra   float [B][H][2 nbp][128] per-anchor share of dq through the anchor mean
 *   gdk, gdv float [B][H][nbp][2][128] gradients w.r.t. the group mean keys / values
 * The SOL_VARIANT_SOL2_PV8 layout is the SOL_VARIANT_SOL2 layout with v8t, vbmax and
 * vscale appended, so the Sol-Attn2 stage calls accept either workspace; likewise the
 * SOL_VARIANT_SOL1_TRAIN layout is the SOL_VARIANT_SOL1 one with the training arrays
 * appended, and the SOL_VARIANT_SOL2_TRAIN layout the SOL_VARIANT_SOL2 one.
 */
typedef struct {
    int64_t total_bytes;
    int64_t nb, nbp;
    int64_t qbar, kbar_t, kbar_h, vbar_h, tau_i, kstat, kcov, kpart;
    int64_t q8, k8, qscale, kscale, qhat, gk, gv, glogn, ghi, qanc;
    int64_t kv_splits, opart, olse;
    int64_t sel, tmu, tnu, tlz;
    int64_t v8t, vbmax, vscale;
    int64_t lse, mrow, mcol, ld, dkbar, dvbar;
    int64_t kh, vh;
    int64_t qd, kd, dlam, qab, dmub, dnub, alz, aextra, gdk, gdv;
    int64_t ofp, kcovp;
    int64_t wcnt, qcount, order;
    int64_t bqord, bkord;
} sol_ws_layout;

/* Static description of a status code (never NULL). */
const char* sol_status_string(int status);

/* Host-only argument check of the Sol-Attn contract; launches nothing and
 * needs no device.  sink_start < 0 means "suffix": the sink covers the last
 * sink_tokens tokens (Sol-Attn README, "Exact KV sink"); sink_tokens == 0
 * means no sink. */
int sol_attn_validate(int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                      float tau, int64_t sink_start, int64_t sink_tokens, int thresh);

/* Workspace size in bytes for `variant` (sol_variant) at this shape; 0 on a
 * shape error.  Host-only. */
size_t sol_attn_workspace_bytes(int variant, int64_t batch, int64_t tokens, int64_t heads,
                                int64_t head_dim);

/* Fill *layout (host pointer) with the workspace offsets; host-only. */
int sol_attn_workspace_layout(int variant, int64_t batch, int64_t tokens, int64_t heads,
                              int64_t head_dim, sol_ws_layout* layout);

/* Split-KV (Sol-Attn README, "Long-sequence tuning on H100": kv_splits).  The
 * fused Sol-Attn pass can split each query block's key range into S parts run by
 * separate workgroups and merged afterwards (fp32 partial rows with their
 * log-sum-exp, rounded to bf16 once by the merge); on MI355X this keeps the K/V
 * working set of the workgroups that run together on one XCD inside its L2.
 * kv_splits = 0 means automatic: no split up to 512 key blocks (8 routing chunks
 * of 64 blocks), then one split per six chunks rounded up, at most 4 (the fp32
 * partials then take at most twice the bytes of q, k, v and out).  Splits cover
 * whole routing chunks: a request r becomes ceil(C / ceil(C / r)) for C chunks
 * (never above C); explicit requests may ask for up to 16.
 * Host-only; returns the effective split count (>= 1), or 0 on a shape error. */
int sol_attn_kv_splits(int64_t batch, int64_t tokens, int64_t heads, int kv_splits);

/* Workspace size / layout for an explicit kv_splits (0 = automatic); the
 * functions above use the automatic value. */
size_t sol_attn_workspace_bytes_kv(int variant, int64_t batch, int64_t tokens, int64_t heads,
                                   int64_t head_dim, int kv_splits);
int sol_attn_workspace_layout_kv(int variant, int64_t batch, int64_t tokens, int64_t heads,
                                 int64_t head_dim, int kv_splits, sol_ws_layout* layout);

/*
 * Sol-Attn forward (Sol-Attn paper §3, Figure 4; Sol-Attn README "Core API",
 * "Exact KV sink").  q, k, v: device, bf16 BTHD, read-only.  out: device,
 * bf16 BTHD, written.  tau: the threshold coefficient beta of Eq. (4);
 * higher selects fewer blocks; 0 is not dense.  sink_start/sink_tokens: the
 * exact KV sink (every 64-token KV block overlapping the range is exact for
 * every query).  thresh: sol_thresh.  workspace: device, >=
 * sol_attn_workspace_bytes(SOL_VARIANT_SOL1, ...), 256-byte aligned.
 * Runs sol_attn_prepare then sol_attn_fused.
 */
int sol_attn(const void* q, const void* k, const void* v, void* out,
             int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
             float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
             void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 of sol_attn: block summaries (Q/K means, V sums as means), the
 * per-query-block threshold tau_i (paper §3.1 Eqs. (4)-(5); the paper keeps
 * only this threshold computation outside the attention kernel, §4.5), and the
 * head-major K / V copies.  Writes the workspace arrays qbar..kpart, kh and vh.
 * Same arguments as sol_attn minus out and the sink. */
int sol_attn_prepare(const void* q, const void* k, const void* v,
                     int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                     float tau, int thresh, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 of sol_attn: the fused routing + proxy-reuse + exact online-softmax
 * kernel (paper §3.2 "Hardware-Aligned Implementation", Eq. (6)): each query
 * block's proxy scores s_ij = Q-bar_i . K-bar_j / sqrt(d) are compared with tau_i
 * chunk by chunk inside the kernel (the sink's blocks forced exact) and the
 * decisions stay on chip.  Reads the workspace written by sol_attn_prepare for
 * the same q, k, v and shape. */
int sol_attn_fused(const void* q, const void* k, const void* v, void* out,
                   int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                   int64_t sink_start, int64_t sink_tokens,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 with an explicit kv_splits (0 = automatic); the workspace must be
 * sized by sol_attn_workspace_bytes_kv for the same kv_splits.  Runs the fused
 * kernel and, for more than one split, the merge kernel.  out may be NULL: then
 * only the fused kernel runs (split partials are still written to the workspace,
 * the final output store and the merge are skipped), e.g. to time that kernel. */
int sol_attn_fused_kv(const void* q, const void* k, const void* v, void* out,
                      int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                      int64_t sink_start, int64_t sink_tokens, int kv_splits,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Training forward (Sol-Attn paper §6 "Limitations and Future Work" names backward
 * support as the missing piece; the Sol-Attn2 draft, Method, Stage A1 passage, fixes
 * its meaning: the block selection stays fixed during the backward pass).  Same
 * arguments, output and errors as sol_attn with automatic kv_splits, on a workspace
 * of at least sol_attn_workspace_bytes(SOL_VARIANT_SOL1_TRAIN, ...) bytes; the call
 * also leaves in the workspace the routing bits it used (mrow) and each query row's
 * log-sum-exp (lse), which sol_attn_backward reads.  The workspace must then be left
 * untouched until the backward call. */
int sol_attn_forward_train(const void* q, const void* k, const void* v, void* out,
                           int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                           float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Backward of sol_attn_forward_train with its routing fixed: the gradients of
 * sum(dout * out) w.r.t. q, k and v.  The forward is one softmax over the tokens of
 * the exact blocks and one pooled key per unselected block (K mean, logit bias
 * ln n_j, value V mean; Sol-Attn paper §3.2), so the gradient reaches every exact
 * token directly and every token of an unselected block as 1/n_j of its pooled
 * key's and value's gradient (the block means).  q, k, v, out: the tensors of the
 * forward call (device, bf16 BTHD, unchanged since); dout: device bf16 BTHD, the
 * gradient of the output; dq, dk, dv: device bf16 BTHD outputs, fully written.
 * workspace: the forward's (SOL_VARIANT_SOL1_TRAIN layout), which this call also uses
 * as scratch; the shape must be the forward's.  Errors: SOL_ERR_NULL for a NULL
 * pointer, SOL_ERR_ARG for pointers not 16-byte aligned, shape and workspace errors as
 * sol_attn; nothing is launched then.  The pooled-key gradients are summed with fp32
 * atomics, so the last bits of dk and dv can differ between runs. */
int sol_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      void* dq, void* dk, void* dv, int64_t batch, int64_t tokens, int64_t heads,
                      int64_t head_dim, void* workspace, size_t workspace_bytes, void* stream);

/* Sol-Attn2 training forward (draft, Method, Stage A1 passage: block selection and the
 * key groups stay fixed in the backward).  Same arguments, output and errors as
 * sol_attn2, on a workspace of at least sol_attn_workspace_bytes(SOL_VARIANT_SOL2_TRAIN,
 * ...) bytes; the call also leaves in the workspace everything sol_attn2_backward reads:
 * the E4M3 codes and scales, the routing bits (sel), the group bits, sizes and means,
 * each anchor's tail (mu_a, nu_a, Z_a) and each row's log-sum-exp (lse).  The workspace
 * must then be left untouched until the backward call. */
int sol_attn2_forward_train(const void* q, const void* k, const void* v, void* out,
                            int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                            float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Backward of sol_attn2_forward_train with its routing and groups fixed: the gradients of
 * sum(dout * out) w.r.t. q, k and v (draft, Method, Eqs. (1)-(3), differentiated with the
 * selection and the memberships constant).  Gradients reach every exact token directly;
 * every anchor's queries through its tail logit and, as 1/n_a shares, through its mean
 * q-bar_a; every token of an unselected block, as 1/n_g of its group's mean-key and
 * mean-value gradients.  The E4M3 quantizer of q and k is passed straight through (the
 * gradient w.r.t. the dequantized value is the gradient returned), and the exact products
 * use the dequantized q', k' rounded to bf16.  q, k, v, out: the tensors of the forward
 * call (device, bf16 BTHD, unchanged since); dout: device bf16 BTHD; dq, dk, dv: device
 * bf16 BTHD outputs, fully written.  workspace: the forward's (SOL_VARIANT_SOL2_TRAIN
 * layout), also used as scratch; the shape must be the forward's.  Errors as
 * sol_attn_backward.  No atomics: results are deterministic. */
int sol_attn2_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       void* dq, void* dk, void* dv, int64_t batch, int64_t tokens, int64_t heads,
                       int64_t head_dim, void* workspace, size_t workspace_bytes, void* stream);

/* Test and tooling export, not part of the hot path: like sol_attn (with an
 * explicit kv_splits, 0 = automatic, and a workspace sized for it), and the
 * fused kernel also writes the routing decision it made, as bit masks
 * mask_bits[b][h][i][w] (device, uint64, nbw = ceil(nb/64) words per query
 * block; bit (j % 64) of word j / 64 set iff KV block j was exact for query
 * block i).  selected_pairs (device, one uint64, may be NULL) receives the
 * number of selected token pairs, sum over exact (i, j) of n_i n_j with n the
 * valid tokens of a block, counted by the fused kernel from the words it used
 * (the realised token-pair sparsity is 1 - selected_pairs / (B H N^2); Sol-Attn2
 * draft, "FP8 Kernel Performance", reports sparsity over token pairs); the call
 * clears it first.  `out` may be NULL to skip the output store.  Errors as
 * sol_attn; SOL_ERR_NULL if mask_bits is NULL. */
int sol_attn_debug_routing(const void* q, const void* k, const void* v, void* out,
                           int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                           float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                           int kv_splits, void* workspace, size_t workspace_bytes, uint64_t* mask_bits,
                           uint64_t* selected_pairs, void* stream);

/*
 * Sol-Attn2 forward with the complementary tail (Sol-Attn2 draft, Method,
 * Eqs. (1)-(3); "FP8 quantization and ExpCast"): Q and K are quantized to
 * OCP E4M3FN with one fp32 scale per (batch, head, 64-token block); V stays
 * bf16; routing on the dequantized block means with the same threshold rule;
 * each unselected key block contributes two key groups to a per-32-token-
 * anchor tail with first-order mass correction; exact and tail terms share
 * one denominator.  Arguments as sol_attn; workspace >=
 * sol_attn_workspace_bytes(SOL_VARIANT_SOL2, ...).
 */
int sol_attn2(const void* q, const void* k, const void* v, void* out,
              int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
              float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
              void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 of sol_attn2: quantization, block summaries, threshold, mean-query
 * direction and key-group summaries (workspace arrays listed above). */
int sol_attn2_prepare(const void* q, const void* k, const void* v,
                      int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                      float tau, int thresh, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2 of sol_attn2 (Sol-Attn2 draft, Method, Eqs. (1)-(3)): sol_attn2_tail
 * then sol_attn2_exact on the same workspace and stream. */
int sol_attn2_fused(const void* q, const void* k, const void* v, void* out,
                    int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                    int64_t sink_start, int64_t sink_tokens,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2a (Sol-Attn2 draft, Method, Eq. (1)): per 32-token anchor the tail over the
 * groups of the unselected blocks: log2 Z_a, mu_a, nu_a (workspace arrays tmu, tnu,
 * tlz).  The pass routes its 32 query blocks per workgroup on chip (proxy scores of
 * the dequantized fp32 block means against tau_i, the sink forced) with the same fp32
 * arithmetic as stage 2b, so both stages take the same decisions; no routing map is
 * written.  Needs stage 1 on this workspace.  q, k, v are only validated (the pass
 * reads the workspace). */
int sol_attn2_tail(const void* q, const void* k, const void* v,
                   int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                   int64_t sink_start, int64_t sink_tokens,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2b (Sol-Attn2 draft, Eqs. (2), (3); "FP8 quantization and ExpCast"): routes
 * its query block on chip (as stage 2a: sink_start / sink_tokens must be the ones
 * stage 2a was given), then exact attention over the selected blocks with FP8 Q K^T
 * and bf16 P V, combined with the anchor tail through delta_t and one shared
 * denominator; writes out (device, bf16 BTHD, non-NULL).  Needs stage 2a on this
 * workspace. */
int sol_attn2_exact(const void* q, const void* k, const void* v, void* out,
                    int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                    int64_t sink_start, int64_t sink_tokens,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sol-Attn2 with FP8 PV (Sol-Attn2 draft, "FP8 quantization and ExpCast"): as
 * sol_attn2, but V is quantized with one E4M3 scale per head and the exact
 * weights are ExpCast bytes c(u) = clip(RNE(8u + 55.65), 0, 120), u the base-2
 * score minus the online pivot; the same decoded bytes weight V (FP8 MFMA) and
 * form the exact part of the denominator.  Workspace >=
 * sol_attn_workspace_bytes(SOL_VARIANT_SOL2_PV8, ...).
 */
int sol_attn2_pv8(const void* q, const void* k, const void* v, void* out,
                  int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                  float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 of sol_attn2_pv8: sol_attn2_prepare plus the per-head V scale and the
 * E4M3 V codes (workspace arrays vbmax, vscale, v8t). */
int sol_attn2_pv8_prepare(const void* q, const void* k, const void* v,
                          int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                          float tau, int thresh, void* workspace, size_t workspace_bytes, void* stream);

/* Stage 2b of sol_attn2_pv8 (after sol_attn2_tail on the same workspace, with the
 * same sink): exact attention with FP8 Q K^T and FP8 P V (ExpCast P), combined with
 * the tail. */
int sol_attn2_pv8_exact(const void* q, const void* k, const void* v, void* out,
                        int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                        int64_t sink_start, int64_t sink_tokens,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Sol-Attn2 routing export, as sol_attn_debug_routing (kv_splits must be 0 or 1:
 * the Sol-Attn2 pass is not split); selected_pairs is counted by the exact pass. */
int sol_attn2_debug_routing(const void* q, const void* k, const void* v, void* out,
                            int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                            float tau, int64_t sink_start, int64_t sink_tokens, int thresh,
                            int kv_splits, void* workspace, size_t workspace_bytes, uint64_t* mask_bits,
                            uint64_t* selected_pairs, void* stream);

/*
 * sol_attn without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, output and errors as sol_attn minus the workspace: the workspace is a
 * static device array of SOL_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per
 * device (its address is looked up once per device, on the first call with that device
 * current); nothing is allocated or freed, here or later.  The current device must be the
 * one `stream` belongs to.  Shapes whose Sol-Attn workspace (sol_attn_workspace_bytes with
 * SOL_VARIANT_SOL1) exceeds the scratch are rejected with SOL_ERR_SCRATCH before any
 * launch (e.g. B=1, H=12, 14040 tokens needs 88 MiB and fits; B=1, H=32, 32768 tokens
 * needs 1059 MiB and does not).  Every call on a device shares that device's scratch: calls
 * that overlap on one device (other streams, other host threads) race and must be
 * serialized by the caller.  The scratch keeps the last call's contents; the call writes
 * every array it reads, so nothing needs clearing between calls.
 */
int sol_attn_noalloc(const void* q, const void* k, const void* v, void* out,
                     int64_t batch, int64_t tokens, int64_t heads, int64_t head_dim,
                     float tau, int64_t sink_start, int64_t sink_tokens, int thresh, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H */
