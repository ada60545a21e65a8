"""Pins of the Sol-Attn2 oracle (CPU only).

The draft's Eqs. (1)-(3) are checked through reductions with known answers:
singleton groups with a constant query per anchor reproduce dense attention;
anchor size 1 with whole-block groups reproduces Sol-Attn's proxy reuse; the
log-partition gradient identity; the "extra compressed key with an additive
bias" form (draft "FP8 quantization and ExpCast"); and an independent
scalar-loop implementation.  The group split rule and mean-query direction
are a reading of the pages ("parity unpinned"), so only their invariants are
checked here.
"""
import math

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import sol_attn as sa
from oracle import sol_attn2 as s2
from workloads import block_offset_tensor


def _rand_head(n, d, seed, offset=1.0):
    x = block_offset_tensor(1, n, 1, d, seed, offset)
    return x[0, :, 0, :].to(torch.float64).numpy()


def _sdpa(q, k, v, bias=None):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    mask = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[0, 0].numpy()


def test_singleton_groups_and_constant_anchor_queries_are_dense():
    """With one group per token and q_t = q-bar_a inside each anchor, delta_t = 0 and the tail
    mass/value are exact, so Eq. (3) is dense softmax attention."""
    n, d = 300, 16
    q0, k, v = (_rand_head(n, d, s) for s in (1, 2, 3))
    q = q0.copy()
    for a0 in range(0, n, 32):
        q[a0:a0 + 32] = q0[a0:a0 + 32].mean(axis=0)     # anchors never straddle a 64-block
    for tau in (0.0, 1.0):
        r = s2.sol_attn2_head(q, k, v, tau=tau, grouping="singleton", quantize=False)
        assert 0 < r.sel.sum() < r.sel.size
        np.testing.assert_allclose(r.out, _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("tau,sink", [(1.0, (None, 0)), (0.3, (0, 70))])
def test_anchor_one_whole_block_groups_reduce_to_sol_attn(tau, sink):
    """Anchor size 1 and one group per block: w = n_j e^{q.K-bar_j}, nu = sum w V-bar / Z and
    delta = 0, so Z nu = sum_j e^{q.K-bar_j} V-hat_j: exactly Sol-Attn's proxy reuse."""
    n, d = 333, 32
    q, k, v = (_rand_head(n, d, s) for s in (11, 12, 13))
    r2 = s2.sol_attn2_head(q, k, v, tau=tau, sink_start=sink[0], sink_tokens=sink[1],
                           anchor=1, grouping="whole", quantize=False)
    r1 = sa.sol_attn_head(q, k, v, tau=tau, sink_start=sink[0], sink_tokens=sink[1])
    np.testing.assert_array_equal(r2.sel, r1.sel)
    np.testing.assert_allclose(r2.out, r1.out, rtol=1e-10, atol=1e-12)


def test_everything_exact_is_dense():
    n, d = 200, 16
    q, k, v = (_rand_head(n, d, s) for s in (21, 22, 23))
    r = s2.sol_attn2_head(q, k, v, tau=1.0, sink_start=0, sink_tokens=n, quantize=False)
    np.testing.assert_allclose(r.out, _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


def test_log_partition_gradient_is_mu_over_sqrt_d():
    """Draft Eq. (2) rationale: d ln Z_a / d q-bar_a = mu_a / sqrt d (central differences)."""
    n, d = 256, 16
    k, v = _rand_head(n, d, 31), _rand_head(n, d, 32)
    q = _rand_head(n, d, 33)
    groups = [g for gl in s2.all_key_groups(k, v, q.mean(axis=0)) for g in gl]
    scale = 1 / math.sqrt(d)
    qa = q[:32].mean(axis=0)
    _, mu, _ = s2.tail_stats(qa, groups, scale)
    h = 1e-6
    grad = np.zeros(d)
    for c in range(d):
        e = np.zeros(d)
        e[c] = h
        grad[c] = (s2.tail_stats(qa + e, groups, scale)[0] - s2.tail_stats(qa - e, groups, scale)[0]) / (2 * h)
    np.testing.assert_allclose(grad, mu * scale, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("quantize", [False, True])
def test_extra_biased_key_form(quantize):
    """The corrected tail equals one extra key mu_a with value nu_a and additive logit bias
    ln Z_a - q-bar_a.mu_a/sqrt d (its logit is ln Z_a + delta_t); SDPA with that float bias
    must reproduce Eq. (3) for every anchor."""
    n, d = 256, 32
    q, k, v = (_rand_head(n, d, s) for s in (41, 42, 43))
    r = s2.sol_attn2_head(q, k, v, tau=0.8, quantize=quantize)
    scale = 1 / math.sqrt(d)
    ranges = sa.block_ranges(n)
    for i in range(len(ranges)):
        out, alpha, parts = s2.attend_query_block2(r.q_deq, r.k_deq, v, i, r.sel[i], r.groups, scale,
                                                   return_parts=True)
        assert np.all((alpha >= 0) & (alpha <= 1))      # output table: alpha_i in [0, 1]
        ex = np.concatenate([np.arange(*ranges[j]) for j in np.flatnonzero(r.sel[i])] or [np.zeros(0, int)])
        for (a0, a1), ln_z, mu, nu in parts:
            if not math.isfinite(ln_z):
                continue
            kk = np.vstack([r.k_deq[ex], mu[None]])
            vv = np.vstack([v[ex], nu[None]])
            bias = np.zeros((a1 - a0, len(ex) + 1))
            bias[:, -1] = ln_z - (r.q_deq[a0:a1].mean(axis=0) @ mu) * scale
            np.testing.assert_allclose(out[a0 - i * 64:a1 - i * 64], _sdpa(r.q_deq[a0:a1], kk, vv, bias),
                                       rtol=1e-10, atol=1e-12)


def test_empty_tail_is_exact_sparse_attention():
    """With no unselected block the tail is empty (Z-hat = 0): plain attention over E_i."""
    n, d = 200, 16
    q, k, v = (_rand_head(n, d, s) for s in (51, 52, 53))
    r = s2.sol_attn2_head(q, k, v, tau=1.0, sink_start=0, sink_tokens=n, quantize=True)
    np.testing.assert_allclose(r.out, _sdpa(r.q_deq, r.k_deq, v), rtol=1e-10, atol=1e-12)


def test_group_split_invariants():
    """Two groups per block partition it, preserve mass n_hi k-bar_hi + n_lo k-bar_lo = n K-bar, and
    split the key projections onto q-hat at the block mean."""
    n, d = 333, 32
    q, k, v = (_rand_head(n, d, s) for s in (61, 62, 63))
    qhat = q.mean(axis=0)
    for (s, e), gl in zip(sa.block_ranges(n), s2.all_key_groups(k, v, qhat)):
        assert 1 <= len(gl) <= 2
        assert sum(g[1] for g in gl) == e - s
        np.testing.assert_allclose(sum(g[1] * g[2] for g in gl), k[s:e].sum(axis=0), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sum(g[1] * g[3] for g in gl), v[s:e].sum(axis=0), rtol=1e-12, atol=1e-12)
        p = k[s:e] @ qhat
        hi = gl[0][0]
        assert np.all(p[hi] >= p.mean()) and np.all(p[~hi] < p.mean())
    # identical keys in a block: everything joins G_hi and G_lo is dropped
    kc = np.repeat(k[:1], 64, axis=0)
    assert len(s2.key_groups(kc, v[:64], qhat)) == 1


def test_anchor_ranges_partial_block():
    assert s2.anchor_ranges(0, 1000) == [(0, 32), (32, 64)]
    assert s2.anchor_ranges(15, 1000) == [(960, 992), (992, 1000)]
    assert s2.anchor_ranges(3, 200) == [(192, 200)]


@pytest.mark.parametrize("n,d,tau,grouping,sink", [
    (200, 8, 1.0, "split2", (None, 0)),
    (150, 16, 0.2, "split2", (64, 10)),
    (130, 8, 0.7, "whole", (None, 0)),
    (100, 8, 0.0, "singleton", (None, 20)),
])
def test_matches_scalar_loop_brute_force(n, d, tau, grouping, sink):
    q, k, v = (_rand_head(n, d, s, offset=1.5) for s in (71, 72, 73))
    r = s2.sol_attn2_head(q, k, v, tau=tau, sink_start=sink[0], sink_tokens=sink[1],
                          grouping=grouping, quantize=False)
    sb = tuple(np.flatnonzero(sa.sink_block_mask(n, sink[0], sink[1])))
    ob = np.array(brute.sol_attn2(q.tolist(), k.tolist(), v.tolist(), tau, sink_blocks=sb, grouping=grouping))
    np.testing.assert_allclose(r.out, ob, rtol=1e-11, atol=1e-12)


def test_quantized_routing_uses_dequantized_means():
    """Routing in Sol-Attn2 runs on block means of the dequantized Q/K (draft "Routing")."""
    n, d = 512, 128
    q, k, v = (_rand_head(n, d, s) for s in (81, 82, 83))
    r = s2.sol_attn2_head(q, k, v, tau=1.0, quantize=True)
    sel_ref = sa.route(sa.block_means(r.q_deq), sa.block_means(r.k_deq), 1.0, 1 / math.sqrt(d))[0]
    np.testing.assert_array_equal(r.sel, sel_ref)
    assert not np.array_equal(r.q_deq, q)
    assert np.abs(r.q_deq - q).max() < 0.1 * np.abs(q).max()
