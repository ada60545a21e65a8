"""Pins for the Sol-Attn backward oracle (no GPU).

The backward with fixed routing is the gradient of the forward output with the
masks held constant (Sol-Attn2 draft, Method, Stage A1 passage).  It is pinned by
finite differences of the pinned forward (oracle.sol_attn.attend_query_block), by
the gradient of torch's SDPA when every block is exact, and by the identical-key
case, where the proxy equals dense attention as a function of q and v.
"""
import math

import numpy as np
import pytest
import torch

from oracle import sol_attn as sa
from oracle import sol_attn_bwd as sb


def _inputs(n, d, seed, offset=1.0):
    g = np.random.default_rng(seed)
    nb = (n + 63) // 64
    out = []
    for _ in range(4):
        o = g.standard_normal((nb, d)) * offset
        out.append(g.standard_normal((n, d)) + o[np.arange(n) // 64])
    return out


def _masks(n, seed, density=0.4, sink=None):
    nb = (n + 63) // 64
    sel = np.random.default_rng(seed).random((nb, nb)) < density
    if sink is not None:
        sel[:, sink] = True
    return sel


def _forward(q, k, v, sel):
    """The pinned forward, block by block, with the masks given."""
    n, d = q.shape
    kbar, vsum, counts = sa.block_means(k), sa.block_sums(v), sa.block_counts(n)
    return np.concatenate([sa.attend_query_block(q, k, v, i, sel[i], kbar, vsum, counts, 1 / math.sqrt(d))
                           for i in range(len(counts))])


@pytest.mark.parametrize("n,seed", [(130, 1), (200, 2), (64, 3)])
def test_forward_with_lse_is_the_forward(n, seed):
    """The augmented-key form (pooled key K-bar_j, bias ln n_j, value V-bar_j) is the paper's
    output, and exp(L_t) is its denominator."""
    q, k, v, _ = _inputs(n, 32, seed)
    sel = _masks(n, seed)
    out, lse = sb.forward_with_lse(q, k, v, sel)
    np.testing.assert_allclose(out, _forward(q, k, v, sel), rtol=1e-12, atol=1e-12)
    # explicit denominator of one row in its block
    t = n - 1
    i = t // 64
    ranges = sa.block_ranges(n)
    kbar, counts = sa.block_means(k), sa.block_counts(n)
    den = 0.0
    for j, (s, e) in enumerate(ranges):
        if sel[i, j]:
            den += np.exp(q[t] @ k[s:e].T / math.sqrt(32)).sum()
        else:
            den += counts[j] * np.exp(q[t] @ kbar[j] / math.sqrt(32))
    assert abs(lse[t] - math.log(den)) < 1e-12


@pytest.mark.parametrize("n,d,seed,density", [(130, 32, 4, 0.4), (200, 16, 5, 0.2), (66, 128, 6, 0.5)])
def test_directional_derivatives_match_central_differences(n, d, seed, density):
    """<grad, direction> equals (f(x + eps dir) - f(x - eps dir)) / 2 eps for f = sum(dO * o)
    with the masks fixed, for q, k and v separately."""
    q, k, v, dout = _inputs(n, d, seed)
    sel = _masks(n, seed, density)
    grads = sb.backward_head(q, k, v, dout, sel)
    g = np.random.default_rng(seed + 100)
    eps = 1e-5
    for which in range(3):
        direction = g.standard_normal((n, d))
        args = [q, k, v]
        plus, minus = list(args), list(args)
        plus[which] = args[which] + eps * direction
        minus[which] = args[which] - eps * direction
        fd = ((dout * _forward(*plus, sel)).sum() - (dout * _forward(*minus, sel)).sum()) / (2 * eps)
        an = (grads[which] * direction).sum()
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_single_coordinates_in_exact_pooled_and_partial_blocks():
    """Coordinate derivatives where each gradient term lives: a token of a block that every
    query block selects, one that none selects (all of its dk / dv comes from the pooled key),
    and the 2-token partial block."""
    n, d = 130, 16
    q, k, v, dout = _inputs(n, d, 7)
    sel = np.zeros((3, 3), dtype=bool)
    sel[:, 0] = True                    # block 0 exact everywhere, block 1 pooled everywhere
    sel[1, 2] = True                    # the partial block is exact for query block 1 only
    grads = sb.backward_head(q, k, v, dout, sel)
    eps = 1e-6
    for which, t, c in [(1, 5, 3), (1, 70, 0), (1, 129, 7), (2, 70, 2), (2, 128, 9), (0, 100, 4), (2, 3, 1)]:
        args = [q.copy(), k.copy(), v.copy()]
        args[which][t, c] += eps
        fp = (dout * _forward(*args, sel)).sum()
        args[which][t, c] -= 2 * eps
        fm = (dout * _forward(*args, sel)).sum()
        fd = (fp - fm) / (2 * eps)
        assert abs(fd - grads[which][t, c]) <= 1e-6 * max(1.0, abs(fd)), (which, t, c)


@pytest.mark.parametrize("n", [64, 130, 257])
def test_everything_exact_is_the_gradient_of_sdpa(n):
    """All blocks selected: dq, dk, dv equal torch's float64 SDPA gradient."""
    d = 32
    q, k, v, dout = _inputs(n, d, 8)
    sel = np.ones(((n + 63) // 64,) * 2, dtype=bool)
    dq, dk, dv = sb.backward_head(q, k, v, dout, sel)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None])[0, 0]
    o.backward(torch.tensor(dout))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-11)


def test_identical_keys_agree_with_dense_gradients():
    """Keys constant within each block make the proxy exact as a function of q and v, so dq
    and dv equal dense attention's; dk keeps each block's sum, and a block that no query
    block selects gets the block mean of the dense dk on every token."""
    n, d = 200, 32
    q, _, v, dout = _inputs(n, d, 9)
    nb = 4
    k = np.repeat(np.random.default_rng(10).standard_normal((nb, d)), 64, axis=0)[:n]
    sel = _masks(n, 11, 0.4)
    sel[:, 1] = False                   # block 1 pooled for every query block
    dq, dk, dv = sb.backward_head(q, k, v, dout, sel)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None])[0, 0]
    o.backward(torch.tensor(dout))
    rq, rk, rv = tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()
    np.testing.assert_allclose(dq, rq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, rv, rtol=1e-9, atol=1e-11)
    for s, e in sa.block_ranges(n):
        np.testing.assert_allclose(dk[s:e].sum(0), rk[s:e].sum(0), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk[64:128], np.tile(rk[64:128].mean(0), (64, 1)), rtol=1e-9, atol=1e-11)
    assert not np.allclose(dk[64:128], rk[64:128])     # per-token dense dk differs


def test_bthd_wrapper_matches_per_head():
    B, N, H, d = 2, 100, 3, 16
    g = torch.Generator().manual_seed(12)
    q, k, v, do = (torch.randn(B, N, H, d, generator=g, dtype=torch.float64) for _ in range(4))
    sel = np.random.default_rng(13).random((B, H, 2, 2)) < 0.5
    dq, dk, dv = sb.backward(q, k, v, do, sel)
    r = sb.backward_head(q[1, :, 2].numpy(), k[1, :, 2].numpy(), v[1, :, 2].numpy(), do[1, :, 2].numpy(), sel[1, 2])
    np.testing.assert_array_equal(dq[1, :, 2], r[0])
    np.testing.assert_array_equal(dk[1, :, 2], r[1])
    np.testing.assert_array_equal(dv[1, :, 2], r[2])
