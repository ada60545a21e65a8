"""Pins of the Sol-Attn2 backward oracle (CPU only).

oracle.sol_attn2_bwd differentiates the Sol-Attn2 forward (draft Eqs. (1)-(3)) with the
routing and the key groups fixed (draft, Method, Stage A1 passage).  Pins: its forward is
the pinned forward; its gradient matches central differences of that forward; with
singleton groups and a constant query per anchor it is dense attention's gradient (the
tail is exact there, to first order in q); with one-token anchors and one whole-block group
per block it is exactly the Sol-Attn backward (oracle.sol_attn_bwd).
"""
import math

import numpy as np
import pytest
import torch

from oracle import sol_attn2 as s2
from oracle import sol_attn2_bwd as b2
from oracle import sol_attn_bwd as sb
from workloads import block_offset_tensor


def _rand_head(n, d, seed, offset=1.0):
    x = block_offset_tensor(1, n, 1, d, seed, offset)
    return x[0, :, 0, :].to(torch.float64).numpy()


def _case(n, d, tau, seed, grouping="split2", sink=(None, 0)):
    q, k, v = (_rand_head(n, d, seed + i) for i in range(3))
    r = s2.sol_attn2_head(q, k, v, tau=tau, sink_start=sink[0], sink_tokens=sink[1], grouping=grouping,
                          quantize=False)
    return q, k, v, r


@pytest.mark.parametrize("n,tau,sink", [(200, 0.6, (None, 0)), (130, 0.2, (0, 40))])
def test_forward_fixed_is_the_pinned_forward(n, tau, sink):
    q, k, v, r = _case(n, 16, tau, 100 + n, sink=sink)
    out, lse = b2.forward_fixed(q, k, v, r.sel, b2.group_masks_of(r.groups))
    np.testing.assert_allclose(out, r.out, rtol=1e-12, atol=1e-13)
    assert np.isfinite(lse).all()


@pytest.mark.parametrize("n,d,tau,sink", [(200, 8, 0.5, (None, 0)), (161, 16, 0.1, (64, 30)), (96, 8, -0.3, (None, 0))])
def test_directional_derivatives_match_central_differences(n, d, tau, sink):
    q, k, v, r = _case(n, d, tau, 300 + n, sink=sink)
    assert 0 < r.sel.sum() < r.sel.size
    masks = b2.group_masks_of(r.groups)
    g = np.random.default_rng(n).standard_normal((n, d))
    dq, dk, dv = b2.backward_head2(q, k, v, g, r.sel, masks)
    rng = np.random.default_rng(7 + n)
    h = 1e-5
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        e = rng.standard_normal((n, d))
        args = {"q": q, "k": k, "v": v}

        def f(x):
            a = dict(args)
            a[which] = x
            return float((g * b2.forward_fixed(a["q"], a["k"], a["v"], r.sel, masks)[0]).sum())
        fd = (f(args[which] + h * e) - f(args[which] - h * e)) / (2 * h)
        an = float((grad * e).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_single_coordinates_through_the_tail():
    """One coordinate of a token in an exact block, of a tail group's member and of a query in
    an anchor whose tail is nonempty: central differences against the analytic gradient."""
    n, d = 150, 8
    q, k, v, r = _case(n, d, 0.4, 500)
    masks = b2.group_masks_of(r.groups)
    g = np.random.default_rng(1).standard_normal((n, d))
    dq, dk, dv = b2.backward_head2(q, k, v, g, r.sel, masks)
    h = 1e-6
    i0 = 0                                            # query block 0
    tail_blocks = np.flatnonzero(~r.sel[i0])
    exact_blocks = np.flatnonzero(r.sel[i0])
    assert tail_blocks.size and exact_blocks.size
    picks = [("q", 5, 3), ("k", 64 * tail_blocks[0] + 2, 1), ("k", 64 * exact_blocks[0] + 1, 4),
             ("v", 64 * tail_blocks[0] + 7, 0), ("v", min(n - 1, 64 * exact_blocks[0] + 3), 2)]
    for which, t, c in picks:
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}

        def f(delta):
            a = {key: val.copy() for key, val in arrs.items()}
            a[which][t, c] += delta
            return float((g * b2.forward_fixed(a["q"], a["k"], a["v"], r.sel, masks)[0]).sum())
        fd = (f(h) - f(-h)) / (2 * h)
        an = {"q": dq, "k": dk, "v": dv}[which][t, c]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, t, c, fd, an)


def test_singleton_groups_with_constant_anchor_queries_give_the_dense_gradient():
    """Singleton groups and one query value per anchor make the output dense attention as a
    function of K and V (every tail weight is exact while q_t = q-bar_a), so dk and dv equal
    dense attention's gradient (float64 torch autograd of softmax(QK^T / sqrt d) V).  Moving
    all of an anchor's queries together keeps them equal to their mean, so the anchor's sum
    of dq equals dense attention's too (a single query alone moves nu_a by 1/32 of its step,
    so dq itself differs)."""
    n, d = 192, 16
    q0, k, v = (_rand_head(n, d, s) for s in (601, 602, 603))
    q = q0.copy()
    for a0 in range(0, n, 32):
        q[a0:a0 + 32] = q0[a0:a0 + 32].mean(axis=0)
    r = s2.sol_attn2_head(q, k, v, tau=0.5, grouping="singleton", quantize=False)
    assert 0 < r.sel.sum() < r.sel.size
    g = np.random.default_rng(3).standard_normal((n, d))
    dq, dk, dv = b2.backward_head2(q, k, v, g, r.sel, b2.group_masks_of(r.groups))
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(qt @ kt.T / math.sqrt(d), dim=-1) @ vt
    (o * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-9, atol=1e-11)
    dq_dense = qt.grad.numpy()
    for a0 in range(0, n, 32):
        np.testing.assert_allclose(dq[a0:a0 + 32].sum(axis=0), dq_dense[a0:a0 + 32].sum(axis=0), rtol=1e-9,
                                   atol=1e-11)
    assert np.abs(dq - dq_dense).max() > 1e-3      # the per-token gradients do differ


@pytest.mark.parametrize("tau,sink", [(0.8, (None, 0)), (0.3, (0, 70))])
def test_single_token_anchors_and_whole_block_groups_are_the_sol_attn_backward(tau, sink):
    n, d = 233, 16
    q, k, v = (_rand_head(n, d, s) for s in (701, 702, 703))
    r = s2.sol_attn2_head(q, k, v, tau=tau, sink_start=sink[0], sink_tokens=sink[1], anchor=1, grouping="whole",
                          quantize=False)
    g = np.random.default_rng(5).standard_normal((n, d))
    got = b2.backward_head2(q, k, v, g, r.sel, b2.group_masks_of(r.groups), anchor=1)
    want = sb.backward_head(q, k, v, g, r.sel)
    for x, y in zip(got, want):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-12)
