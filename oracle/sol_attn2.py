"""Sol-Attn2 forward pass with the complementary tail, float64 CPU oracle (test infrastructure only).

Follows "Sol-Attn2: Sparse Attention with Complementary Approximation"
(draft, October 2026), cited below as "the draft": Method, "Routing and
complementary approximation" Eqs. (1)-(3); "How the outputs are combined"
(output table, Sol-Attn2 row); "FP8 quantization and ExpCast".

Steps, per (batch, head):

0. Quantize Q and K with one E4M3 scale per 64-token block (draft "FP8
   quantization"): s = max|X| / 448, X8 = E4M3(X / s), X' = s * X8.  V stays
   bf16.  All later steps use X' (the dequantized values).
1. Route on 64-token Q/K block means with the Sol-Attn threshold rule
   (draft: "Dot products of 64-token Q/K block means select the exact set
   E_i"; the reading is the diagonal threshold of ``oracle.sol_attn`` with
   tau calibrated to the target sparsity; sink blocks are exact).
2. Mean-query direction q-hat = mean of q' over all tokens of the (b, h).
   Each key block j splits into G_hi = {u : k'_u . q-hat >= mean_u k'_u . q-hat}
   and G_lo = the rest; an empty group is dropped.  Group sizes n_g, mean
   keys k-bar_g (of k') and mean values v-bar_g.
   The draft names the mean-query direction and a split of each block into
   two content groups by key projection without defining the direction's
   averaging set or the split point; this is a reading (per-(b,h) mean query,
   split at the block's mean projection of the dequantized keys, ties to
   G_hi).  It is pinned by a hand-worked example whose inputs separate it
   from the other plausible readings (tests/golden/sol2_groups.txt).
3. Anchors are the two 32-token halves of each 64-token query block (clipped
   to N); q-bar_a = mean of q' over the anchor.
4. Tail T_a = the groups of every key block j that is not exact for the
   anchor's query block (output table: "The tail contains only tokens
   outside E_i").  Eq. (1): w_ag = n_g exp(q-bar_a . k-bar_g / sqrt d),
   Z_a = sum w_ag, (mu_a, nu_a) = sum w_ag (k-bar_g, v-bar_g) / Z_a.
5. Eq. (2): delta_t = (q'_t - q-bar_a) . mu_a / sqrt d, Z-hat_t = Z_a e^{delta_t},
   U-hat_t = Z-hat_t nu_a.  Eq. (3): with z_tu = q'_t . k'_u / sqrt d over the
   exact tokens,  o_t = (sum e^{z} v + U-hat_t) / (sum e^{z} + Z-hat_t).
   An empty tail gives Z-hat = 0.

The oracle is parameterised by anchor size, grouping ("split2", "whole",
"singleton") and quantization on/off so that the reductions used as pins
(tests/test_oracle_sol_attn2.py) can be run.

FP8 PV option (pv="expcast"; draft "FP8 quantization and ExpCast"): V is
quantized with one E4M3 scale per (b, h) (s_V = max|V| / 448), and the exact
weights are ExpCast bytes, p-hat = decode(c((z - m) log2 e)), against the shared
online pivot m: the selected key blocks are taken in ascending order, m is
raised to each block's largest logit before that block's bytes are formed, and
the sums so far are rescaled by e^{m_old - m} (the pages give the pivot as
online; the reading takes the order and granularity of the tiled pass, one
64-token block at a time; `pivot_block` sets another granularity).  The same p-hat weights form the exact numerator
(with the dequantized V) and the exact part of the denominator.  The tail keeps
the bf16 group means of V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional

import numpy as np

from . import e4m3
from .e4m3 import expcast_weight
from .sol_attn import (BLOCK, block_counts, block_means, block_ranges, route,
                       sink_block_mask, _head)

ANCHOR = 32
LOG2E = 1.0 / math.log(2.0)


# ----------------------------------------------------------------------------
# Step 0: FP8 quantization of Q and K
# ----------------------------------------------------------------------------

def quantize_head(x: np.ndarray, block: int = BLOCK):
    """Per-64-token-block E4M3 quantization of one [N, d] head (draft "FP8 quantization").

    x holds the exact bf16 input values.  Returns (codes uint8 [N, d],
    scales float32 [nb], dequantized float64 [N, d]).
    """
    n, d = x.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    ranges = block_ranges(n, block)
    scales = np.zeros(len(ranges), dtype=np.float32)
    deq = np.zeros((n, d))
    for j, (s, e) in enumerate(ranges):
        c, sc = e4m3.quantize_block_fp32(x[s:e])
        codes[s:e] = c
        scales[j] = sc
        deq[s:e] = np.float64(sc) * e4m3.decode(c)
    return codes, scales, deq


# ----------------------------------------------------------------------------
# Step 2: key groups
# ----------------------------------------------------------------------------

def mean_query_direction(q: np.ndarray) -> np.ndarray:
    """q-hat = mean over every token of the (b, h) (reading of "the mean-query direction")."""
    return q.mean(axis=0)


def key_groups(k_blk: np.ndarray, v_blk: np.ndarray, qhat: np.ndarray, grouping: str = "split2"):
    """Content groups of one key block: list of (member mask, n_g, k-bar_g, v-bar_g).

    "split2": split by projection onto q-hat at the block's mean projection
    (ties join G_hi); "whole": one group; "singleton": one group per token.
    """
    n = k_blk.shape[0]
    if grouping == "whole":
        masks = [np.ones(n, dtype=bool)]
    elif grouping == "singleton":
        masks = [np.eye(n, dtype=bool)[u] for u in range(n)]
    elif grouping == "split2":
        p = k_blk @ qhat
        hi = p >= p.mean()
        masks = [hi, ~hi]
    else:
        raise ValueError(grouping)
    groups = []
    for m in masks:
        cnt = int(m.sum())
        if cnt == 0:
            continue
        groups.append((m, float(cnt), k_blk[m].mean(axis=0), v_blk[m].mean(axis=0)))
    return groups


def all_key_groups(k: np.ndarray, v: np.ndarray, qhat: np.ndarray, grouping: str = "split2",
                   block: int = BLOCK):
    """Groups of every key block: list (per block) of group lists."""
    return [key_groups(k[s:e], v[s:e], qhat, grouping) for s, e in block_ranges(k.shape[0], block)]


# ----------------------------------------------------------------------------
# Steps 3-5: anchors, tail statistics, output
# ----------------------------------------------------------------------------

def anchor_ranges(i: int, n_tokens: int, anchor: int = ANCHOR, block: int = BLOCK) -> list:
    """Anchors of query block i: consecutive `anchor`-token spans, clipped to N."""
    s, e = i * block, min(i * block + block, n_tokens)
    return [(a, min(a + anchor, e)) for a in range(s, e, anchor)]


def tail_stats(qbar_a: np.ndarray, groups: list, scale: float):
    """Draft Eq. (1): ln Z_a, mu_a, nu_a over the tail groups (ln Z = -inf for an empty tail)."""
    d = qbar_a.shape[0]
    if not groups:
        return -math.inf, np.zeros(d), np.zeros(d)
    n_g = np.array([g[1] for g in groups])
    kb = np.stack([g[2] for g in groups])
    vb = np.stack([g[3] for g in groups])
    logw = np.log(n_g) + (kb @ qbar_a) * scale        # ln w_ag
    m = logw.max()
    w = np.exp(logw - m)
    z = w.sum()
    ln_z = m + math.log(z)
    mu = (w @ kb) / z
    nu = (w @ vb) / z
    return ln_z, mu, nu


def attend_query_block2(q: np.ndarray, k: np.ndarray, v: np.ndarray, i: int, sel_row: np.ndarray,
                        groups: list, scale: float, anchor: int = ANCHOR, block: int = BLOCK,
                        return_parts: bool = False, pv: str = "bf16", v_exact: Optional[np.ndarray] = None,
                        pivot_block: int = BLOCK):
    """Output rows of query block i: exact blocks plus the first-order-corrected tail.

    return_parts also returns, per anchor, (range, ln Z_a, mu_a, nu_a) and
    per-token alpha_t = Z_E / (Z_E + Z-hat) (output table, Sol-Attn2 row).
    pv="expcast" uses ExpCast weights for the exact tokens and v_exact (the
    per-head FP8-dequantized V) as their values; the tail still uses `groups`.
    pivot_block: how many consecutive exact keys share one step of the online
    ExpCast pivot (the reading: one 64-token block; the pages fix no granularity).
    """
    n, d = q.shape
    s, e = i * block, min(i * block + block, n)
    ranges = block_ranges(n, block)
    ex_idx = np.concatenate([np.arange(*ranges[j]) for j in np.flatnonzero(sel_row)] or
                            [np.zeros(0, dtype=np.int64)])
    tail = [g for j in np.flatnonzero(~sel_row) for g in groups[j]]
    out = np.zeros((e - s, d))
    alpha = np.zeros(e - s)
    parts = []
    for a0, a1 in anchor_ranges(i, n, anchor, block):
        qa = q[a0:a1]
        qbar_a = qa.mean(axis=0)
        ln_z, mu, nu = tail_stats(qbar_a, tail, scale)
        z = (qa @ k[ex_idx].T) * scale                     # exact logits
        lam = ln_z + ((qa - qbar_a) @ mu) * scale          # ln Z-hat_t = ln Z_a + delta_t
        m = np.full(a1 - a0, -np.inf)
        if z.shape[1]:
            m = np.maximum(m, z.max(axis=1))
        if pv == "expcast" and z.shape[1]:
            # ExpCast with the shared online pivot: the selected blocks in ascending order,
            # the pivot p raised to each block's largest logit before its bytes are taken,
            # e^{z} ~ e^{p} p-hat((z - p) log2 e), earlier sums rescaled by e^{p_old - p}.
            p = np.full(a1 - a0, -np.inf)
            wnum = np.zeros((a1 - a0, d))
            wden = np.zeros(a1 - a0)
            col = 0
            steps = [(s0, min(s0 + pivot_block, be)) for j in np.flatnonzero(sel_row)
                     for bs, be in [ranges[j]] for s0 in range(bs, be, pivot_block)]
            for bs, be in steps:
                zj = z[:, col:col + (be - bs)]
                col += be - bs
                p_new = np.maximum(p, zj.max(axis=1))
                keep = np.where(np.isfinite(p), np.exp(p - p_new), 0.0)
                w = expcast_weight((zj - p_new[:, None]) * LOG2E)
                wnum = wnum * keep[:, None] + w @ v_exact[bs:be]
                wden = wden * keep + w.sum(axis=1)
                p = p_new
            mm = np.maximum(p, lam)
            ez_scale = np.exp(p - mm)
            zhat = np.exp(lam - mm)
            ze = wden * ez_scale
            num = wnum * ez_scale[:, None] + zhat[:, None] * nu[None, :]
        else:
            m = np.maximum(m, lam)
            ez = np.exp(z - m[:, None])
            zhat = np.exp(lam - m)
            ze = ez.sum(axis=1)
            num = ez @ v[ex_idx] + zhat[:, None] * nu[None, :]
        den = ze + zhat
        out[a0 - s:a1 - s] = num / den[:, None]
        alpha[a0 - s:a1 - s] = ze / den
        parts.append(((a0, a1), ln_z, mu, nu))
    if return_parts:
        return out, alpha, parts
    return out


@dataclasses.dataclass
class Head2Result:
    out: np.ndarray
    sel: np.ndarray
    s_hat: np.ndarray
    tau_i: np.ndarray
    q_deq: np.ndarray
    k_deq: np.ndarray
    q_codes: Optional[np.ndarray]
    k_codes: Optional[np.ndarray]
    q_scales: Optional[np.ndarray]
    k_scales: Optional[np.ndarray]
    qhat: np.ndarray
    groups: list


def quantize_head_v(v: np.ndarray):
    """One E4M3 scale for a whole (b, h) of V (draft "FP8 quantization": "V with one
    scale per head").  Returns (codes uint8 [N, d], scale float32, dequantized float64)."""
    c, s = e4m3.quantize_block_fp32(v)
    return c, s, np.float64(s) * e4m3.decode(c)


def sol_attn2_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float = 1.0,
                   sink_start: Optional[int] = None, sink_tokens: int = 0, thresh: str = "diag",
                   anchor: int = ANCHOR, grouping: str = "split2", quantize: bool = True,
                   query_blocks: Optional[Iterable[int]] = None, block: int = BLOCK,
                   pv: str = "bf16") -> Head2Result:
    """Sol-Attn2 for one (batch, head): q, k, v [N, d] holding the exact input values."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    scale = 1.0 / math.sqrt(d)
    if quantize:
        qc, qs, qd = quantize_head(q, block)
        kc, ks, kd = quantize_head(k, block)
    else:
        qc = qs = kc = ks = None
        qd, kd = q, k
    sink = sink_block_mask(n, sink_start, sink_tokens, block)
    sel, s_hat, tau_i, _, _ = route(block_means(qd, block), block_means(kd, block), tau, scale,
                                    sink, thresh)
    qhat = mean_query_direction(qd)
    groups = all_key_groups(kd, v, qhat, grouping, block)
    out = np.full((n, d), np.nan)
    nb = len(block_counts(n, block))
    v_exact = quantize_head_v(v)[2] if pv == "expcast" else None
    for i in (range(nb) if query_blocks is None else query_blocks):
        s, e = i * block, min(i * block + block, n)
        out[s:e] = attend_query_block2(qd, kd, v, i, sel[i], groups, scale, anchor, block, pv=pv, v_exact=v_exact)
    return Head2Result(out, sel, s_hat, tau_i, qd, kd, qc, kc, qs, ks, qhat, groups)


def sol_attn2(q, k, v, tau: float = 1.0, sink_start: Optional[int] = None, sink_tokens: int = 0,
              thresh: str = "diag", anchor: int = ANCHOR, grouping: str = "split2",
              quantize: bool = True, query_blocks=None, pv: str = "bf16"):
    """Sol-Attn2 over BTHD inputs [B, N, H, d].

    Returns dict(out [B,N,H,d], sel [B,H,nb,nb], s_hat, tau_i, q_codes/k_codes
    [B,N,H,d] uint8, q_scales/k_scales [B,H,nb] float32, group_hi [B,H,N] bool
    (True where token u is in its block's G_hi), qhat [B,H,d]).
    """
    B, N, H, D = q.shape
    nb = (N + BLOCK - 1) // BLOCK
    res = dict(out=np.full((B, N, H, D), np.nan), sel=np.zeros((B, H, nb, nb), dtype=bool),
               s_hat=np.zeros((B, H, nb, nb)), tau_i=np.zeros((B, H, nb)),
               q_codes=np.zeros((B, N, H, D), dtype=np.uint8),
               k_codes=np.zeros((B, N, H, D), dtype=np.uint8),
               q_scales=np.zeros((B, H, nb), dtype=np.float32),
               k_scales=np.zeros((B, H, nb), dtype=np.float32),
               group_hi=np.zeros((B, H, N), dtype=bool), qhat=np.zeros((B, H, D)))
    qb = None if query_blocks is None else list(query_blocks)
    for b in range(B):
        for h in range(H):
            r = sol_attn2_head(_head(q, b, h), _head(k, b, h), _head(v, b, h), tau, sink_start,
                               sink_tokens, thresh, anchor, grouping, quantize, qb, pv=pv)
            res["out"][b, :, h, :] = r.out
            res["sel"][b, h], res["s_hat"][b, h], res["tau_i"][b, h] = r.sel, r.s_hat, r.tau_i
            res["qhat"][b, h] = r.qhat
            if quantize:
                res["q_codes"][b, :, h, :], res["k_codes"][b, :, h, :] = r.q_codes, r.k_codes
                res["q_scales"][b, h], res["k_scales"][b, h] = r.q_scales, r.k_scales
            if grouping == "split2":
                for s, e in block_ranges(N):
                    p = r.k_deq[s:e] @ r.qhat
                    res["group_hi"][b, h, s:e] = p >= p.mean()
    return res
