// Internal launcher declarations shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

// Workspace pointers resolved from the byte layout (see include/solattn.h).
struct Workspace {
  int nb, nbp;
  float* qbar;      // [B][H][nbp][128]
  float* kbar_t;    // [B][H][32][nbp][4]
  uint16_t* kbar_h; // [B][H][nbp][128] bf16
  uint16_t* vbar_h; // [B][H][nbp][128] bf16
  uint16_t* kh;     // [B][H][N][128] bf16 head-major copy of K (Sol-Attn)
  uint16_t* vh;     // [B][H][N][128] bf16 head-major copy of V (Sol-Attn)
  float* tau_i;     // [B][H][nbp]
  float* kstat;     // [B][H][2][128]
  float* kcov;      // [B][H][128][128]
  double* kpart;    // [B][H][16][2][128] partial key-mean statistics
  uint8_t* q8;      // [B][H][tp][128]
  uint8_t* k8;
  float* qscale;    // [B][H][nbp]
  float* kscale;
  float* qhat;      // [B][H][128]
  uint16_t* gk;     // [B][H][nbp][2][128] bf16
  uint16_t* gv;
  float* glogn;     // [B][H][nbp][2]
  uint64_t* ghi;    // [B][H][nbp]
  float* qanc;      // [B][H][nbp][2][128]
  int kv_splits;    // key-range splits of the fused Sol-Attn pass (1 = none)
  float* opart;     // [S][B][N][H][128] fp32 normalized partial outputs
  float* olse;      // [S][B][N][H] log2-sum-exp of the partial rows
  uint64_t* sel;    // [B][H][nb][nbp / 64] Sol-Attn2 training: the forward's routing bits
  float* tmu;       // [B][H][nbp][2][128] Sol-Attn2 tail key means per anchor
  float* tnu;       // [B][H][nbp][2][128] Sol-Attn2 tail value means per anchor
  float* tlz;       // [B][H][nbp][2] log2 Z_a - log2(e) qbar_a . mu_a / sqrt(d)
  uint8_t* v8t;     // [B][H][128][tp] E4M3 V codes, PV operand order within each 64-token block
  float* vbmax;     // [B][H][nbp] max |V| per block
  float* vscale;    // [B][H] per-head V scale
  // Sol-Attn training layout: state the forward leaves for the backward, and backward scratch
  float* lse;       // [B][H][tp] base-2 log-sum-exp of each query row (forward output)
  uint64_t* mrow;   // [B][H][nb][nbp / 64] routing bits of the forward, one row per query block
  uint64_t* mcol;   // [B][H][nb][nbp / 64] the same bits transposed, one row per key block
  float* ld;        // [B][H][tp][2] (lse, D = dO . O) per query row
  float* dkbar;     // [B][H][nbp][128] gradient w.r.t. the pooled keys K-bar_j (times 1/sqrt(d))
  float* dvbar;     // [B][H][nbp][128] gradient w.r.t. the pooled values V-bar_j
  // Sol-Attn2 training layout (the forward's lse, mcol and ld above are shared): backward scratch
  uint16_t* qd;     // [B][N][H][128] bf16 dequantized q' (BTHD)
  uint16_t* kd;     // [B][N][H][128] bf16 dequantized k' (BTHD); kh / vh hold k' and v head-major
  float* dlam;      // [B][H][tp] gradient w.r.t. each row's tail logit lambda_t
  uint16_t* qab;    // [B][H][2 nbp][128] bf16 anchor means q-bar_a
  uint16_t* dmub;   // [B][H][2 nbp][128] bf16 gradient w.r.t. mu_a
  uint16_t* dnub;   // [B][H][2 nbp][128] bf16 gradient w.r.t. nu_a
  float* alz;       // [B][H][2 nbp][2] (log2 Z_a, -c_a) per anchor
  float* aextra;    // [B][H][2 nbp][128] per-anchor share of dq through q-bar_a (added to each row)
  float* gdk;       // [B][H][nbp][2][128] gradient w.r.t. the group mean keys (with 1/sqrt(d))
  float* gdv;       // [B][H][nbp][2][128] gradient w.r.t. the group mean values
  float* ofp;       // [B][H][tp][128] the Sol-Attn2 training forward's output rows in fp32
  float* kcovp;     // [B][H][8][128][128] per-slice centred key-mean outer products (exact threshold)
  uint8_t* wcnt;    // [B][H][nbp / 64][nbp] Sol-Attn: exact blocks per (routing chunk, query block)
  int* qcount;      // [B][H][S][nbp] Sol-Attn: exact blocks per query block within each key split
  int* order;       // [B][H][S][nbp] Sol-Attn: query blocks by descending qcount per (head, split) (stage 2's work order)
  int* bqord;       // [B][H][nbp] training: query blocks by descending exact-block count (dQ pass order)
  int* bkord;       // [B][H][nbp] training: key blocks by descending selecting-block count (dK / dV pass order)
};

struct Shape {
  int B, N, H;
};

// Sol-Attn stage 1: block means / sums.
hipError_t launch_summary(const uint16_t* q, const uint16_t* k, const uint16_t* v, Shape s,
                          const Workspace& ws, hipStream_t stream);
// Key statistics and per-query-block thresholds (diag or exact).
hipError_t launch_threshold(Shape s, const Workspace& ws, float tau, int exact, hipStream_t stream);
// Sol-Attn stage 2: fused routing + proxy reuse + exact attention.  mask_out (optional)
// receives the selection words the kernel used; pairs (optional) is cleared and then
// receives the number of selected token pairs sum n_i n_j.
// Stage 2's work order: per-chunk and per-block exact-block counts and each head's query
// blocks by descending count (ws.wcnt, ws.qcount, ws.order); returns hipSuccess without
// launching if the workspace has no such arrays.
hipError_t launch_order(Shape s, const Workspace& ws, int sink_b0, int sink_b1, hipStream_t stream);
hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                        Shape s, const Workspace& ws, int sink_b0, int sink_b1, uint64_t* mask_out,
                        unsigned long long* pairs, hipStream_t stream);

// Sol-Attn2 stage 1: FP8 quantization of Q/K with block means of the dequantized values
// and V block means; then the mean-query direction and key groups.
hipError_t launch_quant_summary(const uint16_t* q, const uint16_t* k, const uint16_t* v, Shape s,
                                const Workspace& ws, hipStream_t stream);
hipError_t launch_qhat(Shape s, const Workspace& ws, hipStream_t stream);
hipError_t launch_groups(const uint16_t* v, Shape s, const Workspace& ws, hipStream_t stream);
// Sol-Attn2 stage 2: the complementary tail per anchor (writes tmu, tnu, tlz), then the exact
// FP8 pass combined with the tail.  Both route on chip with the same fp32 arithmetic, the
// blocks [sink_b0, sink_b1] forced; the exact pass writes its routing words to mask_out when
// that is not NULL (training forward, test export).
hipError_t launch_tail2(Shape s, const Workspace& ws, int sink_b0, int sink_b1, hipStream_t stream);
hipError_t launch_fused2(const uint16_t* v, uint16_t* out, Shape s, const Workspace& ws, bool pv8,
                         unsigned long long* pairs, int sink_b0, int sink_b1, uint64_t* mask_out,
                         hipStream_t stream);
// Sol-Attn backward with the forward's routing fixed: D and the transposed masks, the
// pooled-key gradients, dK / dV per key block, then dQ per query block.
hipError_t launch_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                           const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, Shape s,
                           const Workspace& ws, hipStream_t stream);
// Sol-Attn2 backward with the forward's routing and groups fixed: dequantized copies, the
// per-anchor tail gradients, the group gradients, then the exact dK / dV and dQ passes.
hipError_t launch_backward2(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* out,
                            const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv, Shape s,
                            const Workspace& ws, hipStream_t stream);
// FP8 PV variant, stage 1 addition: per-head V scale and the E4M3 V codes (v8t).
hipError_t launch_vquant(const uint16_t* v, Shape s, const Workspace& ws, hipStream_t stream);

}  // namespace solattn
