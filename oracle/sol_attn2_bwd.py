"""Sol-Attn2 backward pass with routing and grouping fixed, float64 CPU oracle (test infrastructure only).

The Sol-Attn2 draft (Method, "Routing and complementary approximation", the Stage A1
passage) fixes what its backward is: block selection and the key groups stay fixed during
the backward pass, and gradients flow through Q, K, V, the tail approximation and the
joint normalization.  This module is the gradient of the forward of ``oracle.sol_attn2``
(draft Eqs. (1)-(3)) with the masks and the group memberships held constant.  The E4M3
quantization of Q and K is read as straight-through: the gradient with respect to the
dequantized q', k' is the gradient passed to q, k (the draft gives no rule for it).

Forward, per (batch, head), anchor a (32 tokens of query block i), token t in a:
    E = tokens of the exact blocks of i;  tail groups g of the other blocks, with
    n_g, k-bar_g = mean k, v-bar_g = mean v;  q-bar_a = mean of q over the anchor;
    l_g = ln n_g + s q-bar_a . k-bar_g,   pi_g = e^{l_g} / Z_a,   ln Z_a = LSE_g(l_g),
    mu_a = sum pi_g k-bar_g,   nu_a = sum pi_g v-bar_g,
    lambda_t = ln Z_a + s (q_t - q-bar_a) . mu_a,   z_tu = s q_t . k_u  (u in E),
    o_t = softmax over {z_tu, lambda_t} applied to {v_u, nu_a}        (s = 1/sqrt d).

Backward (L = sum_t dO_t . o_t), with P the softmax weights and D_t = dO_t . o_t:
    dz_tu = P_tu (dO_t . v_u - D_t),   dlambda_t = P_t,tail (dO_t . nu_a - D_t);
    through lambda_t:  dq_t += s dlambda_t mu_a,  dq-bar_a -= s dlambda_t mu_a,
                       dmu_a += s dlambda_t (q_t - q-bar_a),  dlnZ_a += dlambda_t;
    through nu_a:      dnu_a += P_t,tail dO_t;
    through the group softmax (ln Z, mu, nu as functions of l_g, k-bar_g, v-bar_g):
        dl_g = pi_g [dlnZ_a + dmu_a . (k-bar_g - mu_a) + dnu_a . (v-bar_g - nu_a)],
        dk-bar_g += s dl_g q-bar_a + pi_g dmu_a,  dv-bar_g += pi_g dnu_a,
        dq-bar_a += s sum_g dl_g k-bar_g;
    means:  every token of anchor a gets dq-bar_a / n_a, every token of group g gets
            dk-bar_g / n_g and dv-bar_g / n_g;
    exact:  dq_t += s sum_u dz_tu k_u,  dk_u += s sum_t dz_tu q_t,  dv_u += sum_t P_tu dO_t.
The pins (central differences of the forward; for singleton groups with constant anchor
queries, dense attention's dk, dv and per-anchor sums of dq; the exact reduction to the
Sol-Attn backward for one whole-block group per block and single-token anchors) live in
tests/.
"""
from __future__ import annotations

import math

import numpy as np

from .sol_attn import BLOCK, block_ranges
from .sol_attn2 import ANCHOR, anchor_ranges


def _lse(x: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)


def _group_logit_grad(pi, dlnz, kb, mu, dmu, vb, nu, dnu):
    """dl_g = pi_g [dlnZ + dmu . (k-bar_g - mu) + dnu . (v-bar_g - nu)] (group softmax backward)."""
    return pi * (dlnz + (kb - mu) @ dmu + (vb - nu) @ dnu)


def _mean_grad(g: np.ndarray, count: float) -> np.ndarray:
    """Gradient reaching each member of a mean (an anchor's queries, a group's keys / values)."""
    return g / count


def group_masks_of(groups: list) -> list:
    """The member masks of ``oracle.sol_attn2`` groups (per block: list of bool arrays)."""
    return [[g[0] for g in gl] for gl in groups]


def _tail_groups(k: np.ndarray, v: np.ndarray, sel_row: np.ndarray, masks: list, block: int):
    """Global member indices, sizes and means of the tail groups of a query block."""
    ranges = block_ranges(k.shape[0], block)
    members, n_g, kb, vb = [], [], [], []
    for j in np.flatnonzero(~np.asarray(sel_row, dtype=bool)):
        s, _ = ranges[j]
        for m in masks[j]:
            idx = s + np.flatnonzero(m)
            if idx.size == 0:
                continue
            members.append(idx)
            n_g.append(float(idx.size))
            kb.append(k[idx].mean(axis=0))
            vb.append(v[idx].mean(axis=0))
    d = k.shape[1]
    if not members:
        return [], np.zeros(0), np.zeros((0, d)), np.zeros((0, d))
    return members, np.array(n_g), np.stack(kb), np.stack(vb)


def _exact_index(n: int, sel_row: np.ndarray, block: int) -> np.ndarray:
    ranges = block_ranges(n, block)
    return np.concatenate([np.arange(*ranges[j]) for j in np.flatnonzero(sel_row)] or
                          [np.zeros(0, dtype=np.int64)]).astype(np.int64)


def forward_fixed(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, masks: list,
                  anchor: int = ANCHOR, block: int = BLOCK):
    """Sol-Attn2 output rows and the natural-log denominator of each row for one (batch, head),
    with the routing sel [nb, nb] and the group memberships ``masks`` held fixed (q, k are
    the values the forward multiplies, i.e. the dequantized ones)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    s = 1.0 / math.sqrt(d)
    out = np.zeros((n, d))
    lse = np.zeros(n)
    for i in range(len(block_ranges(n, block))):
        ex = _exact_index(n, sel[i], block)
        _, n_g, kb, vb = _tail_groups(k, v, sel[i], masks, block)
        for a0, a1 in anchor_ranges(i, n, anchor, block):
            qa = q[a0:a1]
            qbar = qa.mean(axis=0)
            logits = (qa @ k[ex].T) * s
            vals = v[ex]
            if n_g.size:
                lg = np.log(n_g) + (kb @ qbar) * s
                lnz = _lse(lg)
                pi = np.exp(lg - lnz)
                mu, nu = pi @ kb, pi @ vb
                lam = lnz + ((qa - qbar) @ mu) * s
                logits = np.concatenate([logits, lam[:, None]], axis=1)
                vals = np.concatenate([vals, nu[None]], axis=0)
            L = _lse(logits, axis=1)
            out[a0:a1] = np.exp(logits - L[:, None]) @ vals
            lse[a0:a1] = L
    return out, lse


def backward_head2(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, sel: np.ndarray, masks: list,
                   anchor: int = ANCHOR, block: int = BLOCK):
    """dq, dk, dv [N, d] of sum(dout * o) for one (batch, head), routing and groups fixed."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    n, d = q.shape
    s = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, d))
    for i in range(len(block_ranges(n, block))):
        ex = _exact_index(n, sel[i], block)
        members, n_g, kb, vb = _tail_groups(k, v, sel[i], masks, block)
        has_tail = n_g.size > 0
        dkb, dvb = np.zeros_like(kb), np.zeros_like(vb)
        for a0, a1 in anchor_ranges(i, n, anchor, block):
            qa, ga = q[a0:a1], dout[a0:a1]
            na = a1 - a0
            qbar = qa.mean(axis=0)
            logits = (qa @ k[ex].T) * s
            vals = v[ex]
            if has_tail:
                lg = np.log(n_g) + (kb @ qbar) * s
                lnz = _lse(lg)
                pi = np.exp(lg - lnz)
                mu, nu = pi @ kb, pi @ vb
                lam = lnz + ((qa - qbar) @ mu) * s
                logits = np.concatenate([logits, lam[:, None]], axis=1)
                vals = np.concatenate([vals, nu[None]], axis=0)
            L = _lse(logits, axis=1)
            p = np.exp(logits - L[:, None])
            o = p @ vals
            D = (ga * o).sum(axis=1)
            dlogit = p * (ga @ vals.T - D[:, None])           # softmax backward over the row
            ne = ex.size
            dz = dlogit[:, :ne]
            dq[a0:a1] += (dz @ k[ex]) * s
            dk[ex] += (dz.T @ qa) * s
            dv[ex] += p[:, :ne].T @ ga
            if not has_tail:
                continue
            dlam = dlogit[:, ne]
            ptail = p[:, ne]
            # lambda_t = ln Z + s (q_t - q-bar) . mu
            dq[a0:a1] += s * dlam[:, None] * mu[None]
            dqbar = -s * dlam.sum() * mu
            dmu = s * (dlam @ (qa - qbar))
            dlnz = dlam.sum()
            dnu = ptail @ ga
            # ln Z, mu, nu through the group softmax
            dl = _group_logit_grad(pi, dlnz, kb, mu, dmu, vb, nu, dnu)
            dqbar += s * (dl @ kb)
            dkb += s * dl[:, None] * qbar[None] + pi[:, None] * dmu[None]
            dvb += pi[:, None] * dnu[None]
            dq[a0:a1] += _mean_grad(dqbar, na)                  # q-bar is the anchor's mean
        for g, idx in enumerate(members):                       # k-bar, v-bar are group means
            dk[idx] += _mean_grad(dkb[g], idx.size)
            dv[idx] += _mean_grad(dvb[g], idx.size)
    return dq, dk, dv


def backward2(q, k, v, dout, sel, groups_per_head):
    """BTHD inputs [B, N, H, d] (the dequantized q, k), masks [B, H, nb, nb] and the groups of
    each (b, h) (``oracle.sol_attn2`` group lists, indexed [b][h]) -> dq, dk, dv float64."""
    from .sol_attn import _head
    B, N, H, D = q.shape
    dq, dk, dv = (np.zeros((B, N, H, D)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            g = backward_head2(_head(q, b, h), _head(k, b, h), _head(v, b, h), _head(dout, b, h), sel[b, h],
                               group_masks_of(groups_per_head[b][h]))
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = g
    return dq, dk, dv
