"""Sol-Attn backward pass with fixed routing, float64 CPU oracle (test infrastructure only).

The Sol-Attn paper (arXiv 2607.24027) leaves training to future work (§6,
"Limitations and Future Work": a trainable implementation with backward support).
The Sol-Attn2 draft (Method, "Routing and complementary approximation", the
Stage A1 passage) fixes what such a backward is: block selection stays fixed
during the backward pass, and gradients flow through Q, K, V and the joint
normalization.  For Sol-Attn this is the gradient of the forward output of
``oracle.sol_attn`` with the masks held constant:

    o_t = [sum_{u in E_i} e^{z_tu} v_u + sum_{j in U_i} e^{zt_tj} V-hat_j]
          / [sum_{u in E_i} e^{z_tu} + sum_{j in U_i} n_j e^{zt_tj}],
    z_tu = q_t . k_u / sqrt(d),   zt_tj = q_t . K-bar_j / sqrt(d),

with K-bar_j the mean and V-hat_j the sum of block j (paper §3.2).  Writing
V-hat_j = n_j V-bar_j, this is one softmax over an augmented key set: the
tokens u of the exact blocks (logit z_tu, value v_u) and one pooled key per
unselected block (logit zt_tj + ln n_j, value V-bar_j).  With L_t the log of
the denominator, P = e^{logit - L_t}, dP = dO_t . value and D_t = dO_t . o_t,
the logit gradient is dS = P (dP - D_t), and

    dq_t  = sum_u dS_tu k_u / sqrt(d) + sum_j dS~_tj K-bar_j / sqrt(d)
    dk_u  = sum_t dS_tu q_t / sqrt(d)         (exact pairs)
          + (1/n_j) sum_t dS~_tj q_t / sqrt(d)  (u in block j; K-bar_j is a mean)
    dv_u  = sum_t P_tu dO_t                   (exact pairs)
          + (1/n_j) sum_t P~_tj dO_t            (u in block j; V-bar_j is a mean)

where the sums over t for the pooled key j run over the query tokens whose
block did not select j.  The functions below take these steps per query block
in float64; the pins (finite differences of the forward, SDPA's gradient when
everything is exact, the identical-key case) live in tests/.
"""
from __future__ import annotations

import math

import numpy as np

from .sol_attn import BLOCK, block_counts, block_means, block_ranges


def forward_with_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, block: int = BLOCK):
    """Sol-Attn output rows and the natural-log denominator L_t for one (batch, head) under
    fixed masks sel [nb, nb] (paper §3.2 output, masks as given)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    kbar, vbar = block_means(k, block), block_means(v, block)
    logn = np.log(block_counts(n, block))
    ranges = block_ranges(n, block)
    out = np.zeros((n, d))
    lse = np.zeros(n)
    for i, (s, e) in enumerate(ranges):
        ex, un = _split(ranges, sel[i])
        logits = np.concatenate([(q[s:e] @ k[ex].T) * scale, (q[s:e] @ kbar[un].T) * scale + logn[un]], axis=1)
        values = np.concatenate([v[ex], vbar[un]], axis=0)
        m = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - m)
        den = w.sum(axis=1)
        out[s:e] = (w @ values) / den[:, None]
        lse[s:e] = m[:, 0] + np.log(den)
    return out, lse


def _split(ranges, sel_row):
    ex = np.concatenate([np.arange(*ranges[j]) for j in np.flatnonzero(sel_row)] or [np.zeros(0, dtype=np.int64)])
    un = np.flatnonzero(~np.asarray(sel_row, dtype=bool))
    return ex.astype(np.int64), un


def _logit_grad(p: np.ndarray, dp: np.ndarray, D: np.ndarray) -> np.ndarray:
    """Softmax backward: gradient w.r.t. the logits, P (dP - D)."""
    return p * (dp - D)


def _per_token(g: np.ndarray, count: float) -> np.ndarray:
    """Gradient reaching each token of a block from its mean (1/n_j of the mean's gradient)."""
    return g / count


def backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, sel: np.ndarray,
                  block: int = BLOCK):
    """dq, dk, dv [N, d] of sum(dout * o) for one (batch, head) with the masks sel [nb, nb] fixed."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    counts = block_counts(n, block)
    kbar, vbar = block_means(k, block), block_means(v, block)
    logn = np.log(counts)
    ranges = block_ranges(n, block)
    nb = len(ranges)
    out, lse = forward_with_lse(q, k, v, sel, block)
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    dkbar = np.zeros((nb, d))                 # gradient w.r.t. the pooled keys K-bar_j
    dvbar = np.zeros((nb, d))                 # gradient w.r.t. the pooled values V-bar_j
    for i, (s, e) in enumerate(ranges):
        ex, un = _split(ranges, sel[i])
        qb, gb = q[s:e], dout[s:e]
        L = lse[s:e, None]
        D = (gb * out[s:e]).sum(axis=1, keepdims=True)
        # exact tokens
        p = np.exp((qb @ k[ex].T) * scale - L)
        ds = _logit_grad(p, gb @ v[ex].T, D)
        # pooled keys of the unselected blocks (bias ln n_j, value V-bar_j)
        pt = np.exp((qb @ kbar[un].T) * scale + logn[un] - L)
        dst = _logit_grad(pt, gb @ vbar[un].T, D)
        dq[s:e] = (ds @ k[ex] + dst @ kbar[un]) * scale
        dk[ex] += (ds.T @ qb) * scale
        dv[ex] += p.T @ gb
        dkbar[un] += (dst.T @ qb) * scale
        dvbar[un] += pt.T @ gb
    # K-bar_j and V-bar_j are means over block j: each token gets 1/n_j of their gradient
    for j, (s, e) in enumerate(ranges):
        dk[s:e] += _per_token(dkbar[j], counts[j])
        dv[s:e] += _per_token(dvbar[j], counts[j])
    return dq, dk, dv


def backward(q, k, v, dout, sel):
    """BTHD [B, N, H, d] inputs and masks [B, H, nb, nb] -> dq, dk, dv float64 [B, N, H, d]."""
    from .sol_attn import _head
    B, N, H, D = q.shape
    dq, dk, dv = (np.zeros((B, N, H, D)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            g = backward_head(_head(q, b, h), _head(k, b, h), _head(v, b, h), _head(dout, b, h), sel[b, h])
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = g
    return dq, dk, dv
