"""Sol-Attn forward pass, float64 CPU oracle (test infrastructure only).

Follows "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
Attention Sparsification" (Li et al., arXiv 2607.24027), cited below as
"the Sol-Attn paper", the Sol-Attn README of the Sana ``sparse_backends``
package ("the README") and the stable-diffusion.cpp "Sol-Attn" docs page
("the GGML docs").

What is computed, per (batch, head), with blocks of 64 tokens:

1. Block j covers tokens [64 j, min(64 j + 64, N)) and holds n_j valid tokens.
   Q-bar_i and K-bar_j are means over the valid tokens, V-hat_j is the sum
   (paper §3.2 "Hardware-Aligned Implementation": KC holds pooled keys, VC
   summed values; GGML docs intro: "K means and V sums").
2. Proxy score s_ij = Q-bar_i . K-bar_j * scale (paper §2 Eq. (3)), with
   scale = 1/sqrt(d) everywhere (reading: the Sol-Attn2 draft writes
   z = q.k/sqrt(d); the paper's Eq. (1) omits the factor; routing is
   invariant to a positive scale).
3. Threshold tau_i = mu_i + beta * sigma_i (paper §3.1 Eq. (4)) with the
   diagonal estimator (paper appendix "Diagonal threshold estimator") or the
   full-covariance one (paper §3.1 Eq. (5) and the appendix "Threshold
   variance derivation").  The averages run over the nb key blocks with equal
   weight 1/nb (reading of the "N" in Eq. (5)); a negative variance clamps
   to 0.
4. Block j is exact for query block i iff s_ij > tau_i (strict, Eq. (4)), or
   j overlaps the exact KV sink (README "Exact KV sink"), or, optionally,
   |i - j| <= adjacent (GGML docs, implementation notes: an option that keeps
   neighbouring blocks exact; off by default, and not in the kernels).
5. For token t of block i (paper §3.2 "Proxy-Score Reuse as Approximate
   Correction", Figure 4): exact logits z_tu = q_t.k_u*scale over the tokens
   of the exact blocks, pooled logits zt_tj = q_t.K-bar_j*scale over the
   other blocks, and
        o_t = [sum_u e^{z_tu} v_u + sum_j e^{zt_tj} V-hat_j]
              / [sum_u e^{z_tu} + sum_j n_j e^{zt_tj}].
   The denominator is the paper's D_i (B = n_j for a partial block); the
   numerator is the zeroth-order Taylor term with the V sums (reading: the
   printed numerator equation is missing from the page).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------------------
# Blocks and summaries
# ----------------------------------------------------------------------------

def block_ranges(n_tokens: int, block: int = BLOCK) -> list:
    """[(start, stop)] of the 64-token blocks covering [0, n_tokens)."""
    return [(s, min(s + block, n_tokens)) for s in range(0, n_tokens, block)]


def block_counts(n_tokens: int, block: int = BLOCK) -> np.ndarray:
    """n_j: number of valid tokens in each block (the last may be partial)."""
    return np.array([e - s for s, e in block_ranges(n_tokens, block)], dtype=np.float64)


def block_means(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Per-block mean over valid tokens; x is [N, d] -> [nb, d]."""
    return np.stack([x[s:e].mean(axis=0) for s, e in block_ranges(x.shape[0], block)])


def block_sums(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Per-block sum over valid tokens; x is [N, d] -> [nb, d]."""
    return np.stack([x[s:e].sum(axis=0) for s, e in block_ranges(x.shape[0], block)])


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def proxy_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = Q-bar_i . K-bar_j * scale (paper §2 Eq. (3)); [nbq, nbk]."""
    return (qbar @ kbar.T) * scale


def diag_threshold(qbar: np.ndarray, kbar: np.ndarray, beta: float, scale: float):
    """Diagonal threshold estimator (paper appendix "Diagonal threshold estimator").

    mu_K = mean_j K-bar_j, v_K = mean_j K-bar_j (.) K-bar_j - mu_K (.) mu_K,
    mu_i = Q-bar_i . mu_K, sigma_i^2 = (Q-bar_i (.) Q-bar_i) . v_K, both in
    scaled-logit units; tau_i = mu_i + beta sigma_i (Eq. (4)).
    Returns (tau_i, mu_i, sigma_i).
    """
    mu_k = kbar.mean(axis=0)
    v_k = (kbar * kbar).mean(axis=0) - mu_k * mu_k
    mu_i = (qbar @ mu_k) * scale
    var_i = ((qbar * qbar) @ v_k) * scale * scale
    sigma_i = np.sqrt(np.maximum(var_i, 0.0))
    return mu_i + beta * sigma_i, mu_i, sigma_i


def exact_threshold(qbar: np.ndarray, kbar: np.ndarray, beta: float, scale: float):
    """Full-covariance threshold (paper §3.1 Eq. (5)).

    mu_i = Q-bar_i (mean_j K-bar_j)^T,
    sigma_i^2 = Q-bar_i (mean_j K-bar_j^T K-bar_j) Q-bar_i^T - mu_i^2.
    Returns (tau_i, mu_i, sigma_i) in scaled-logit units.
    """
    nb = kbar.shape[0]
    mu_k = kbar.mean(axis=0)
    second = (kbar.T @ kbar) / nb
    mu_i = (qbar @ mu_k) * scale
    var_i = np.einsum("id,de,ie->i", qbar, second, qbar) * scale * scale - mu_i * mu_i
    sigma_i = np.sqrt(np.maximum(var_i, 0.0))
    return mu_i + beta * sigma_i, mu_i, sigma_i


def sink_block_mask(n_tokens: int, sink_start: Optional[int], sink_tokens: int,
                    block: int = BLOCK) -> np.ndarray:
    """KV blocks overlapping the exact sink range (README "Exact KV sink").

    sink_start None (or negative) places the range at the end of the sequence
    (the README's suffix form).  sink_tokens == 0 means no sink.
    """
    nb = (n_tokens + block - 1) // block
    mask = np.zeros(nb, dtype=bool)
    if sink_tokens < 0:
        raise ValueError("sink_tokens must be >= 0")
    if sink_tokens == 0:
        return mask
    start = n_tokens - sink_tokens if (sink_start is None or sink_start < 0) else sink_start
    if start < 0 or start + sink_tokens > n_tokens:
        raise ValueError("sink range out of bounds")
    mask[start // block:(start + sink_tokens - 1) // block + 1] = True
    return mask


def route(qbar: np.ndarray, kbar: np.ndarray, beta: float, scale: float,
          sink: Optional[np.ndarray] = None, thresh: str = "diag", adjacent: int = -1):
    """Block selection (paper §3.1 Eq. (4)): sel_ij = s_ij > tau_i, or sink, or adjacency.

    Returns (sel [nb, nb] bool, s_hat, tau_i, mu_i, sigma_i).
    """
    if not math.isfinite(beta):
        raise ValueError("tau must be finite")
    s_hat = proxy_scores(qbar, kbar, scale)
    if thresh == "diag":
        tau_i, mu_i, sigma_i = diag_threshold(qbar, kbar, beta, scale)
    elif thresh == "exact":
        tau_i, mu_i, sigma_i = exact_threshold(qbar, kbar, beta, scale)
    else:
        raise ValueError(thresh)
    sel = s_hat > tau_i[:, None]
    if sink is not None:
        sel |= sink[None, :]
    if adjacent >= 0:
        idx = np.arange(qbar.shape[0])
        sel |= np.abs(idx[:, None] - np.arange(kbar.shape[0])[None, :]) <= adjacent
    return sel, s_hat, tau_i, mu_i, sigma_i


# ----------------------------------------------------------------------------
# Output
# ----------------------------------------------------------------------------

def attend_query_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, i: int, sel_row: np.ndarray,
                       kbar: np.ndarray, vsum: np.ndarray, counts: np.ndarray, scale: float,
                       block: int = BLOCK, approx: bool = True) -> np.ndarray:
    """Output rows of query block i: exact blocks token-level, the rest by proxy reuse.

    approx=False drops the unselected blocks entirely (plain block-sparse
    attention, paper §2 Eq. (2)); used only for the accuracy sanity check.
    """
    n = q.shape[0]
    s, e = i * block, min(i * block + block, n)
    qb = q[s:e]
    ranges = block_ranges(n, block)
    ex_idx = np.concatenate([np.arange(*ranges[j]) for j in np.flatnonzero(sel_row)] or
                            [np.zeros(0, dtype=np.int64)])
    un = np.flatnonzero(~sel_row) if approx else np.zeros(0, dtype=np.int64)
    z = (qb @ k[ex_idx].T) * scale                 # exact logits  [nq, n_exact]
    zt = (qb @ kbar[un].T) * scale                 # pooled logits [nq, n_unsel]
    m = np.full(qb.shape[0], -np.inf)
    if z.shape[1]:
        m = np.maximum(m, z.max(axis=1))
    if zt.shape[1]:
        m = np.maximum(m, zt.max(axis=1))
    ez = np.exp(z - m[:, None])
    ezt = np.exp(zt - m[:, None])
    num = ez @ v[ex_idx] + ezt @ vsum[un]
    den = ez.sum(axis=1) + ezt @ counts[un]
    return num / den[:, None]


@dataclasses.dataclass
class HeadResult:
    out: np.ndarray          # [N, d] float64 (NaN rows for query blocks not computed)
    sel: np.ndarray          # [nb, nb] bool
    s_hat: np.ndarray        # [nb, nb]
    tau_i: np.ndarray        # [nb]
    mu_i: np.ndarray
    sigma_i: np.ndarray
    counts: np.ndarray       # [nb]


def sol_attn_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float = 1.0,
                  sink_start: Optional[int] = None, sink_tokens: int = 0, thresh: str = "diag",
                  adjacent: int = -1, query_blocks: Optional[Iterable[int]] = None,
                  approx: bool = True, block: int = BLOCK) -> HeadResult:
    """Sol-Attn for one (batch, head): q, k, v are [N, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    scale = 1.0 / math.sqrt(d)
    qbar, kbar, vsum = block_means(q, block), block_means(k, block), block_sums(v, block)
    counts = block_counts(n, block)
    sink = sink_block_mask(n, sink_start, sink_tokens, block)
    sel, s_hat, tau_i, mu_i, sigma_i = route(qbar, kbar, tau, scale, sink, thresh, adjacent)
    nb = len(counts)
    out = np.full((n, d), np.nan)
    blocks = range(nb) if query_blocks is None else query_blocks
    for i in blocks:
        s, e = i * block, min(i * block + block, n)
        out[s:e] = attend_query_block(q, k, v, i, sel[i], kbar, vsum, counts, scale, block, approx)
    return HeadResult(out, sel, s_hat, tau_i, mu_i, sigma_i, counts)


def selected_pairs(sel: np.ndarray, n_tokens: int, block: int = BLOCK) -> int:
    """Exact token pairs sum_{exact (i, j)} n_i n_j over [..., nb, nb] masks, as an integer
    (the token-pair count behind the realised sparsity; Sol-Attn2 draft, "FP8 Kernel
    Performance", states sparsity over token pairs)."""
    c = block_counts(n_tokens, block).astype(np.int64)
    sel = np.asarray(sel, dtype=bool)
    return int((sel.astype(np.int64) * np.outer(c, c)).sum())


def realised_sparsity(sel: np.ndarray, n_tokens: int, block: int = BLOCK) -> float:
    """Token-pair sparsity 1 - sum_{exact (i,j)} n_i n_j / N^2 over [..., nb, nb] masks."""
    sel = np.asarray(sel, dtype=bool)
    lead = int(np.prod(sel.shape[:-2])) if sel.ndim > 2 else 1
    return 1.0 - selected_pairs(sel, n_tokens, block) / (lead * float(n_tokens) ** 2)


def _head(x, b: int, h: int) -> np.ndarray:
    """[B, N, H, d] tensor/array -> float64 [N, d] for one (b, h)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x[b, :, h, :].to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x[b, :, h, :], dtype=np.float64)


def sol_attn(q, k, v, tau: float = 1.0, sink_start: Optional[int] = None, sink_tokens: int = 0,
             thresh: str = "diag", adjacent: int = -1, query_blocks=None, approx: bool = True):
    """Sol-Attn over BTHD inputs [B, N, H, d] (README "Core API" layout).

    query_blocks: None for every query block, or an iterable of block indices
    computed for every (b, h) (routing is always computed in full).
    Returns dict(out [B,N,H,d] float64, sel [B,H,nb,nb], s_hat, tau_i, mu_i, sigma_i).
    """
    B, N, H, D = q.shape
    nb = (N + BLOCK - 1) // BLOCK
    out = np.full((B, N, H, D), np.nan)
    sel = np.zeros((B, H, nb, nb), dtype=bool)
    s_hat = np.zeros((B, H, nb, nb))
    tau_i = np.zeros((B, H, nb))
    mu_i = np.zeros((B, H, nb))
    sigma_i = np.zeros((B, H, nb))
    qb = None if query_blocks is None else list(query_blocks)
    for b in range(B):
        for h in range(H):
            r = sol_attn_head(_head(q, b, h), _head(k, b, h), _head(v, b, h), tau, sink_start,
                              sink_tokens, thresh, adjacent, qb, approx)
            out[b, :, h, :] = r.out
            sel[b, h], s_hat[b, h], tau_i[b, h] = r.sel, r.s_hat, r.tau_i
            mu_i[b, h], sigma_i[b, h] = r.mu_i, r.sigma_i
    return dict(out=out, sel=sel, s_hat=s_hat, tau_i=tau_i, mu_i=mu_i, sigma_i=sigma_i)


def routing_only(q, k, tau: float = 1.0, sink_start: Optional[int] = None, sink_tokens: int = 0,
                 thresh: str = "diag", adjacent: int = -1):
    """Masks, proxy scores and thresholds for BTHD q, k without computing outputs."""
    B, N, H, D = q.shape
    nb = (N + BLOCK - 1) // BLOCK
    scale = 1.0 / math.sqrt(D)
    sink = sink_block_mask(N, sink_start, sink_tokens)
    sel = np.zeros((B, H, nb, nb), dtype=bool)
    s_hat = np.zeros((B, H, nb, nb))
    tau_i = np.zeros((B, H, nb))
    for b in range(B):
        for h in range(H):
            qbar, kbar = block_means(_head(q, b, h)), block_means(_head(k, b, h))
            r = route(qbar, kbar, tau, scale, sink, thresh, adjacent)
            sel[b, h], s_hat[b, h], tau_i[b, h] = r[0], r[1], r[2]
    return dict(sel=sel, s_hat=s_hat, tau_i=tau_i)
