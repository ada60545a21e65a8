"""Pins of the Sol-Attn oracle against what the pages and the mathematics fix (CPU only).

Each test pins the oracle to something other than itself: textbook softmax
attention (torch SDPA in float64), closed-form cases, the paper's identities
and bounds, or an independent scalar-loop implementation.
"""
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import brute
from oracle import sol_attn as sa
from workloads import block_offset_tensor

BLOCK = 64


def _rand_head(n, d, seed, offset=1.0):
    """[N, d] float64 block-offset data rounded to bf16 values."""
    x = block_offset_tensor(1, n, 1, d, seed, offset)
    return x[0, :, 0, :].to(torch.float64).numpy()


def _sdpa(q, k, v, bias=None):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    mask = None if bias is None else torch.from_numpy(bias)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)[0, 0].numpy()


# ---------------------------------------------------------------------------
# Output pins
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,d", [(200, 16), (1024, 128), (333, 32)])
def test_whole_sequence_sink_is_dense(n, d):
    """Every block exact (a sink over [0, N)) reduces to softmax(QK^T/sqrt d)V (paper Eqs. (1)-(2))."""
    q, k, v = (_rand_head(n, d, s) for s in (1, 2, 3))
    r = sa.sol_attn_head(q, k, v, tau=1.0, sink_start=0, sink_tokens=n)
    assert r.sel.all()
    np.testing.assert_allclose(r.out, _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("tau", [-0.5, 0.0, 1.0, 2.0])
def test_identical_keys_make_the_approximation_exact(tau):
    """If every key of a block equals its mean, the proxy reuse is exact (paper §3.2 Taylor term, delta=0)."""
    n, d = 333, 32
    q, k, v = (_rand_head(n, d, s) for s in (11, 12, 13))
    kbar = sa.block_means(k)
    k_const = np.concatenate([np.repeat(kbar[j:j + 1], e - s, axis=0)
                              for j, (s, e) in enumerate(sa.block_ranges(n))])
    r = sa.sol_attn_head(q, k_const, v, tau=tau)
    assert r.sel.sum() < r.sel.size               # some blocks take the proxy branch
    np.testing.assert_allclose(r.out, _sdpa(q, k_const, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("tau,sink", [(1.0, None), (0.0, None), (1.5, (0, 70)), (0.5, (None, 40))])
def test_mean_key_replacement_identity(tau, sink):
    """Sol-Attn == textbook attention in which each query block's unselected KV blocks keep their
    values but have every key replaced by the block mean K-bar_j (so sum_u e^{q.K-bar} v_u =
    e^{q.K-bar} V-hat_j and the denominator gets n_j e^{q.K-bar}).  This pins the numerator,
    the denominator and the partial-block count given the masks."""
    n, d = 333, 32
    q, k, v = (_rand_head(n, d, s) for s in (21, 22, 23))
    ss, st = (None, 0) if sink is None else sink
    r = sa.sol_attn_head(q, k, v, tau=tau, sink_start=ss, sink_tokens=st)
    ranges = sa.block_ranges(n)
    kbar = sa.block_means(k)
    for i, (s, e) in enumerate(ranges):
        k_rep = k.copy()
        for j, (a, b) in enumerate(ranges):
            if not r.sel[i, j]:
                k_rep[a:b] = kbar[j]
        np.testing.assert_allclose(r.out[s:e], _sdpa(q[s:e], k_rep, v), rtol=1e-10, atol=1e-12)


def test_approximation_error_bound():
    """Paper appendix "Approximation error": for a query q and unselected block j with
    delta_u = q.(k_u - K-bar_j)/sqrt d, a = q.K-bar_j/sqrt d, eta = max|delta_u|:
    0 <= D - D~ <= 1/2 e^{a+eta} sum delta_u^2 and ||N - N~|| <= e^{a+eta} sum |delta_u| ||v_u||."""
    n, d = 256, 32
    q, k, v = (_rand_head(n, d, s) for s in (31, 32, 33))
    scale = 1 / math.sqrt(d)
    kbar, vsum = sa.block_means(k), sa.block_sums(v)
    for t in range(0, n, 7):
        for j, (s, e) in enumerate(sa.block_ranges(n)):
            a = q[t] @ kbar[j] * scale
            delta = (k[s:e] - kbar[j]) @ q[t] * scale
            eta = np.abs(delta).max()
            dens = np.exp(k[s:e] @ q[t] * scale).sum()
            den_approx = (e - s) * math.exp(a)
            gap = dens - den_approx
            assert gap >= -1e-12 * dens
            assert gap <= 0.5 * math.exp(a + eta) * (delta ** 2).sum() * (1 + 1e-12)
            num = np.exp(k[s:e] @ q[t] * scale) @ v[s:e]
            num_approx = math.exp(a) * vsum[j]
            bound = math.exp(a + eta) * (np.abs(delta) * np.linalg.norm(v[s:e], axis=1)).sum()
            assert np.linalg.norm(num - num_approx) <= bound * (1 + 1e-12)


def test_approx_correction_beats_exact_only():
    """Accuracy sanity (paper §4.5 "Effect of Approximate Correction"): with identical masks the
    exact+approx output is closer to dense than exact-only.  Statistical, not a hard pin."""
    n, d = 1024, 128
    q, k, v = (_rand_head(n, d, s) for s in (41, 42, 43))
    dense = _sdpa(q, k, v)
    for tau in (0.5, 1.0, 1.5):
        with_approx = sa.sol_attn_head(q, k, v, tau=tau).out
        exact_only = sa.sol_attn_head(q, k, v, tau=tau, approx=False).out
        rows = np.isfinite(exact_only).all(axis=1)     # query blocks with >= 1 exact block
        assert rows.any()
        e1 = np.linalg.norm(with_approx[rows] - dense[rows]) / np.linalg.norm(dense[rows])
        e0 = np.linalg.norm(exact_only[rows] - dense[rows]) / np.linalg.norm(dense[rows])
        assert e1 < e0


# ---------------------------------------------------------------------------
# Routing pins
# ---------------------------------------------------------------------------

def test_proxy_is_column_mean_of_token_to_block_tile():
    """Paper §3.2 (token-to-block tile): Mean over query rows of Q_i K-bar^T equals Q-bar_i K-bar^T."""
    n, d = 333, 32
    q, k = _rand_head(n, d, 51), _rand_head(n, d, 52)
    qbar, kbar = sa.block_means(q), sa.block_means(k)
    s_hat = sa.proxy_scores(qbar, kbar, 1 / math.sqrt(d))
    for i, (s, e) in enumerate(sa.block_ranges(n)):
        tile = q[s:e] @ kbar.T / math.sqrt(d)
        np.testing.assert_allclose(tile.mean(axis=0), s_hat[i], rtol=1e-12, atol=1e-12)


def test_exact_threshold_is_row_mean_and_variance():
    """Paper §3.1 Eq. (5) and appendix "Threshold variance derivation": mu_i and sigma_i^2 equal the
    mean and population variance of the proxy row s_i over the key blocks."""
    n, d = 1024, 64
    q, k = _rand_head(n, d, 61), _rand_head(n, d, 62)
    qbar, kbar = sa.block_means(q), sa.block_means(k)
    scale = 1 / math.sqrt(d)
    s_hat = sa.proxy_scores(qbar, kbar, scale)
    tau_i, mu_i, sigma_i = sa.exact_threshold(qbar, kbar, 0.7, scale)
    np.testing.assert_allclose(mu_i, s_hat.mean(axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sigma_i, s_hat.std(axis=1), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(tau_i, mu_i + 0.7 * sigma_i, rtol=1e-12)


def test_diag_threshold_equals_exact_when_key_covariance_is_diagonal():
    """Paper appendix "Diagonal threshold estimator": with a diagonal covariance of the pooled keys
    the diagonal sigma equals the exact one (the row standard deviation of s_i)."""
    nb, d = 16, 8
    hadamard = np.array([[1.0]])
    while hadamard.shape[0] < nb:
        hadamard = np.block([[hadamard, hadamard], [hadamard, -hadamard]])
    rng = np.random.default_rng(3)
    # zero-mean, mutually orthogonal columns -> diagonal empirical covariance
    kbar = 0.3 + hadamard[:, 1:d + 1] * rng.uniform(0.5, 2.0, size=d)
    qbar = rng.standard_normal((nb, d))
    scale = 1 / math.sqrt(d)
    _, mu_d, sig_d = sa.diag_threshold(qbar, kbar, 1.0, scale)
    s_hat = sa.proxy_scores(qbar, kbar, scale)
    np.testing.assert_allclose(mu_d, s_hat.mean(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sig_d, s_hat.std(axis=1), rtol=1e-12, atol=1e-12)
    # and the diagonal estimator differs once the covariance has off-diagonal terms
    kbar2 = kbar.copy()
    kbar2[:, 1] += kbar2[:, 0]
    _, _, sig_d2 = sa.diag_threshold(qbar, kbar2, 1.0, scale)
    assert not np.allclose(sig_d2, sa.proxy_scores(qbar, kbar2, scale).std(axis=1))


def test_one_hot_routing_selects_the_matching_block():
    """Closed form: K-bar_j = e_j and Q-bar_i = c e_pi(i) give s_ij = c/sqrt(d) [j = pi(i)];
    with tau = 1 only j = pi(i) clears mu_i + sigma_i, which pins the row/column orientation."""
    nb = d = 16
    perm = np.random.default_rng(5).permutation(nb)
    kbar = np.eye(d)
    qbar = 3.0 * np.eye(d)[perm]
    sel, s_hat, tau_i, mu_i, sigma_i = sa.route(qbar, kbar, 1.0, 1 / math.sqrt(d))
    expected = np.zeros((nb, nb), dtype=bool)
    expected[np.arange(nb), perm] = True
    np.testing.assert_array_equal(sel, expected)
    # mu_i = c/(nb sqrt d), sigma_i = c sqrt(1/nb - 1/nb^2)/sqrt d
    np.testing.assert_allclose(mu_i, 3.0 / nb / 4.0)
    np.testing.assert_allclose(sigma_i, 3.0 * math.sqrt(1 / nb - 1 / nb ** 2) / 4.0)


def test_masks_are_nested_and_monotone_in_tau():
    """README: higher tau selects fewer blocks; strict '>' gives nested masks."""
    n, d = 2048, 128
    q, k = _rand_head(n, d, 71), _rand_head(n, d, 72)
    qbar, kbar = sa.block_means(q), sa.block_means(k)
    prev = None
    for tau in (-1.0, 0.0, 0.5, 1.0, 2.0, 3.0):
        sel = sa.route(qbar, kbar, tau, 1 / math.sqrt(d))[0]
        if prev is not None:
            assert not (sel & ~prev).any()
        prev = sel
    assert not sa.route(qbar, kbar, 0.0, 1 / math.sqrt(d))[0].all()   # zero is not dense


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 1.5])
def test_gaussian_calibration_density(beta):
    """Paper §3.1: with Gaussian block proxies the mean selected density is about 1 - Phi(beta).
    Statistical check with i.i.d. Gaussian pooled keys (nb=1024)."""
    nb, d = 1024, 128
    rng = np.random.default_rng(11)
    qbar = rng.standard_normal((nb, d))
    kbar = rng.standard_normal((nb, d))
    sel = sa.route(qbar, kbar, beta, 1 / math.sqrt(d))[0]
    assert abs(sel.mean() - (1 - norm.cdf(beta))) < 0.02


def test_sink_block_ranges():
    """README "Exact KV sink": every 64-token KV block overlapping the range is exact; an omitted
    start places the range at the end; zero tokens means no sink."""
    def blocks(n, s, t):
        return list(np.flatnonzero(sa.sink_block_mask(n, s, t)))
    assert blocks(1000, 0, 512) == list(range(8))
    assert blocks(1000, 0, 513) == list(range(9))
    assert blocks(1000, 100, 50) == [1, 2]
    assert blocks(1000, None, 40) == [15]           # 960..999
    assert blocks(1000, None, 41) == [14, 15]       # 959..999
    assert blocks(1000, 128, 1) == [2]
    assert blocks(1000, 0, 0) == []
    with pytest.raises(ValueError):
        sa.sink_block_mask(1000, 990, 20)
    with pytest.raises(ValueError):
        sa.sink_block_mask(1000, 0, -1)


def test_sink_forces_columns_and_not_rows():
    """Sink blocks are exact for every query; sink query rows are not made dense (README)."""
    n, d = 1024, 128
    q, k, v = (_rand_head(n, d, s) for s in (81, 82, 83))
    r = sa.sol_attn_head(q, k, v, tau=2.0, sink_start=0, sink_tokens=130)
    assert r.sel[:, :3].all()
    assert not r.sel[:3].all()


def test_nonfinite_tau_rejected():
    """GGML docs: the threshold coefficient must be finite."""
    q = _rand_head(128, 16, 1)
    for bad in (math.nan, math.inf, -math.inf):
        with pytest.raises(ValueError):
            sa.sol_attn_head(q, q, q, tau=bad)


# ---------------------------------------------------------------------------
# Brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,d,tau,thresh,sink", [
    (200, 8, 1.0, "diag", (None, 0)),
    (200, 16, 0.3, "diag", (70, 20)),
    (150, 8, 0.8, "exact", (None, 30)),
    (130, 16, -0.2, "exact", (None, 0)),
    (64, 8, 1.0, "diag", (None, 0)),
    (40, 8, 1.0, "diag", (None, 0)),
])
def test_matches_scalar_loop_brute_force(n, d, tau, thresh, sink):
    q, k, v = (_rand_head(n, d, s, offset=1.5) for s in (91, 92, 93))
    ss, st = sink
    r = sa.sol_attn_head(q, k, v, tau=tau, sink_start=ss, sink_tokens=st, thresh=thresh)
    sink_blocks = tuple(np.flatnonzero(sa.sink_block_mask(n, ss, st)))
    sel_b, s_b, tau_b = brute.routing(q.tolist(), k.tolist(), tau, 64, thresh, sink_blocks)
    np.testing.assert_array_equal(r.sel, np.array(sel_b))
    np.testing.assert_allclose(r.s_hat, np.array(s_b), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r.tau_i, np.array(tau_b), rtol=1e-10, atol=1e-12)
    out_b = np.array(brute.sol_attn(q.tolist(), k.tolist(), v.tolist(), tau, 64, thresh, sink_blocks))
    np.testing.assert_allclose(r.out, out_b, rtol=1e-12, atol=1e-12)


def test_realised_sparsity_counts_token_pairs():
    """Token-pair sparsity with a partial block: 1 - sum_{exact} n_i n_j / N^2."""
    n = 200                       # blocks of 64, 64, 64, 8
    sel = np.zeros((4, 4), dtype=bool)
    sel[0, 0] = sel[3, 3] = sel[3, 0] = True
    expected = 1 - (64 * 64 + 8 * 8 + 8 * 64) / n ** 2
    assert abs(sa.realised_sparsity(sel, n) - expected) < 1e-15
