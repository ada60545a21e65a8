"""Planted mistakes in the oracle must trip at least one pin (CPU only).

Each case monkeypatches one plausible mistake into ``oracle`` (a dropped term,
a wrong sign, a transposed operand, a wrong index) and re-runs the pin tests
that should catch it.  A mutation that no pin catches fails this file.
"""
import numpy as np
import pytest

from oracle import sol_attn as sa
from oracle import sol_attn2 as s2
import test_oracle_sol_attn as p1
import test_oracle_sol_attn2 as p2


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError):
        return True
    return False


def _wrap_attend(**override):
    orig = sa.attend_query_block

    def attend(q, k, v, i, sel_row, kbar, vsum, counts, scale, block=64, approx=True):
        kw = dict(q=q, k=k, v=v, i=i, sel_row=sel_row, kbar=kbar, vsum=vsum, counts=counts,
                  scale=scale, block=block, approx=approx)
        kw.update({key: f(kw) for key, f in override.items()})
        return orig(**kw)
    return attend


MUTATIONS_SOL1 = {
    # numerator uses the V mean instead of the V sum
    "vmean_not_vsum": lambda mp: mp.setattr(sa, "block_sums", sa.block_means),
    # denominator drops the block count n_j
    "no_count_in_denominator": lambda mp: mp.setattr(
        sa, "attend_query_block", _wrap_attend(counts=lambda kw: np.ones_like(kw["counts"]))),
    # output logits without the 1/sqrt(d) scale
    "unscaled_logits": lambda mp: mp.setattr(sa, "attend_query_block", _wrap_attend(scale=lambda kw: 1.0)),
    # threshold sign flipped: mu - beta sigma
    "threshold_sign": lambda mp: mp.setattr(
        sa, "diag_threshold",
        (lambda f: (lambda qb, kb, beta, sc: f(qb, kb, -beta, sc)))(sa.diag_threshold)),
    # proxy scores transposed (key block x query block)
    "transposed_proxy": lambda mp: mp.setattr(
        sa, "proxy_scores", (lambda f: (lambda qb, kb, sc: f(qb, kb, sc).T))(sa.proxy_scores)),
    # diagonal estimator forgets to subtract mu_K^2
    "variance_no_centering": lambda mp: mp.setattr(
        sa, "diag_threshold",
        lambda qb, kb, beta, sc: (lambda mu, var: (mu + beta * np.sqrt(var), mu, np.sqrt(var)))(
            (qb @ kb.mean(0)) * sc, ((qb * qb) @ (kb * kb).mean(0)) * sc * sc)),
    # sink block range off by one at the end
    "sink_off_by_one": lambda mp: mp.setattr(
        sa, "sink_block_mask",
        (lambda f: (lambda n, s, t, block=64: np.roll(f(n, s, t, block), 1)))(sa.sink_block_mask)),
}

PINS_SOL1 = [
    (p1.test_whole_sequence_sink_is_dense, (333, 32)),
    (p1.test_mean_key_replacement_identity, (1.0, None)),
    (p1.test_mean_key_replacement_identity, (1.5, (0, 70))),
    (p1.test_one_hot_routing_selects_the_matching_block, ()),
    (p1.test_sink_block_ranges, ()),
    (p1.test_matches_scalar_loop_brute_force, (200, 16, 0.3, "diag", (70, 20))),
    (p1.test_matches_scalar_loop_brute_force, (200, 8, 1.0, "diag", (None, 0))),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS_SOL1))
def test_sol_attn_mutation_is_caught(name, monkeypatch):
    MUTATIONS_SOL1[name](monkeypatch)
    assert any(_fails(fn, *args) for fn, args in PINS_SOL1), f"mutation {name} not caught"


def _tail_mutation(kind):
    orig = s2.tail_stats

    def tail(qbar_a, groups, scale):
        if kind == "no_group_count":
            groups = [(m, 1.0, kb, vb) for (m, n, kb, vb) in groups]
        ln_z, mu, nu = orig(qbar_a, groups, scale)
        if kind == "mu_sign":
            mu = -mu
        if kind == "swap_mu_nu":
            mu, nu = nu, mu
        return ln_z, mu, nu
    return tail


def _split_rule(kind):
    orig = s2.key_groups

    def groups(k_blk, v_blk, qhat, grouping="split2"):
        if grouping != "split2":
            return orig(k_blk, v_blk, qhat, grouping)
        p = k_blk @ qhat
        hi = p >= np.median(p) if kind == "median" else p > p.mean()
        out = []
        for m in (hi, ~hi):
            if m.any():
                out.append((m, float(m.sum()), k_blk[m].mean(axis=0), v_blk[m].mean(axis=0)))
        return out
    return groups


def _per_query_block_direction(mp):
    orig_attend, orig_groups = s2.attend_query_block2, s2.all_key_groups

    def attend(q, k, v, i, sel_row, groups, scale, *args, **kw):
        s, e = i * 64, min(i * 64 + 64, q.shape[0])
        return orig_attend(q, k, v, i, sel_row, orig_groups(k, v, q[s:e].mean(axis=0)), scale, *args, **kw)
    mp.setattr(s2, "attend_query_block2", attend)


def _split_on_unquantized_keys(mp):
    orig_head, orig_groups = s2.sol_attn2_head, s2.all_key_groups

    def head(q, k, v, *args, **kw):
        raw = np.asarray(k, dtype=np.float64)
        mp.setattr(s2, "all_key_groups", lambda kd, vv, qh, grouping="split2", block=64:
                   orig_groups(raw, vv, qh, grouping, block))
        try:
            return orig_head(q, k, v, *args, **kw)
        finally:
            mp.setattr(s2, "all_key_groups", orig_groups)
    mp.setattr(s2, "sol_attn2_head", head)


MUTATIONS_SOL2 = {
    "no_group_count": lambda mp: mp.setattr(s2, "tail_stats", _tail_mutation("no_group_count")),
    "delta_sign": lambda mp: mp.setattr(s2, "tail_stats", _tail_mutation("mu_sign")),
    "swap_mu_nu": lambda mp: mp.setattr(s2, "tail_stats", _tail_mutation("swap_mu_nu")),
    # the group readings pinned by the hand-worked fixture (tests/golden/sol2_groups.txt)
    "median_split": lambda mp: mp.setattr(s2, "key_groups", _split_rule("median")),
    "ties_to_g_lo": lambda mp: mp.setattr(s2, "key_groups", _split_rule("ties_lo")),
    "per_query_block_direction": _per_query_block_direction,
    "split_on_unquantized_keys": _split_on_unquantized_keys,
}

import test_oracle_sol2_groups as p2g  # noqa: E402

PINS_SOL2 = [
    (p2g.test_group_readings_match_the_hand_worked_fixture, ()),
    (p2.test_singleton_groups_and_constant_anchor_queries_are_dense, ()),
    (p2.test_anchor_one_whole_block_groups_reduce_to_sol_attn, (1.0, (None, 0))),
    (p2.test_extra_biased_key_form, (False,)),
    (p2.test_log_partition_gradient_is_mu_over_sqrt_d, ()),
    (p2.test_matches_scalar_loop_brute_force, (200, 8, 1.0, "split2", (None, 0))),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS_SOL2))
def test_sol_attn2_mutation_is_caught(name, monkeypatch):
    MUTATIONS_SOL2[name](monkeypatch)
    assert any(_fails(fn, *args) for fn, args in PINS_SOL2), f"mutation {name} not caught"


import test_oracle_expcast as p3  # noqa: E402
from oracle import e4m3  # noqa: E402


def _code_with_offset(offset):
    def code(u):
        t = (np.float32(8.0) * np.asarray(u, dtype=np.float32) + np.float32(offset)).astype(np.float32)
        return np.clip(np.rint(t), 0.0, 120.0).astype(np.uint8)
    return code


MUTATIONS_EXPCAST = {
    # the plain 56 offset (no centring of the linear mantissa)
    "offset_56": lambda mp: mp.setattr(e4m3, "expcast_code", _code_with_offset(56.0)),
    # the exact tokens use the unquantized V
    "v_not_quantized": lambda mp: mp.setattr(s2, "quantize_head_v", lambda v: (None, np.float32(1.0), v)),
    # the mantissa is read as the next octave (off-by-one exponent)
    "exponent_off_by_one": lambda mp: mp.setattr(
        e4m3, "expcast_weight", lambda u: 2.0 * e4m3.decode(e4m3.expcast_code(u))),
}

PINS_EXPCAST = [
    (p3.test_ratio_to_two_to_the_u_matches_closed_form, ()),
    (p3.test_integer_scores_decode_to_exact_powers_of_two, ()),
    (p3.test_constant_values_come_back_exactly, ()),
    (p3.test_integer_gaps_reduce_to_softmax_over_quantized_v, ()),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS_EXPCAST))
def test_expcast_mutation_is_caught(name, monkeypatch):
    MUTATIONS_EXPCAST[name](monkeypatch)
    assert any(_fails(fn, *args) for fn, args in PINS_EXPCAST), f"mutation {name} not caught"


import test_oracle_backward as p4  # noqa: E402
from oracle import sol_attn_bwd as sb  # noqa: E402

MUTATIONS_BACKWARD = {
    # softmax backward without the D_t = dO . o term
    "no_D_term": lambda mp: mp.setattr(sb, "_logit_grad", lambda p, dp, D: p * dp),
    # the pooled key's gradient reaches every token whole instead of 1/n_j of it
    "mean_chain_rule_dropped": lambda mp: mp.setattr(sb, "_per_token", lambda g, count: g),
    # the pooled keys lose their ln n_j bias (forward weight and chain rule both)
    "no_count_bias": lambda mp: mp.setattr(sb, "block_counts", lambda n, block=64: np.ones((n + block - 1) // block)),
    # pooled values taken as block sums
    "pooled_value_sum": lambda mp: mp.setattr(sb, "block_means", sa.block_sums),
}

PINS_BACKWARD = [
    (p4.test_directional_derivatives_match_central_differences, (130, 32, 4, 0.4)),
    (p4.test_single_coordinates_in_exact_pooled_and_partial_blocks, ()),
    (p4.test_identical_keys_agree_with_dense_gradients, ()),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS_BACKWARD))
def test_backward_mutation_is_caught(name, monkeypatch):
    MUTATIONS_BACKWARD[name](monkeypatch)
    assert any(_fails(fn, *args) for fn, args in PINS_BACKWARD), f"mutation {name} not caught"


import test_oracle_backward2 as p5  # noqa: E402
from oracle import sol_attn2_bwd as b2  # noqa: E402

MUTATIONS_BACKWARD2 = {
    # the group softmax backward forgets mu's dependence on the group logits
    "no_dmu_in_group_grad": lambda mp: mp.setattr(
        b2, "_group_logit_grad", lambda pi, dlnz, kb, mu, dmu, vb, nu, dnu: pi * (dlnz + (vb - nu) @ dnu)),
    # the group softmax backward forgets nu's dependence on the group logits
    "no_dnu_in_group_grad": lambda mp: mp.setattr(
        b2, "_group_logit_grad", lambda pi, dlnz, kb, mu, dmu, vb, nu, dnu: pi * (dlnz + (kb - mu) @ dmu)),
    # the means' chain rule (anchor queries, group keys / values) passes the whole gradient
    "mean_chain_rule_dropped": lambda mp: mp.setattr(b2, "_mean_grad", lambda g, count: g),
}

PINS_BACKWARD2 = [
    (p5.test_directional_derivatives_match_central_differences, (200, 8, 0.5, (None, 0))),
    (p5.test_single_coordinates_through_the_tail, ()),
    (p5.test_singleton_groups_with_constant_anchor_queries_give_the_dense_gradient, ()),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS_BACKWARD2))
def test_backward2_mutation_is_caught(name, monkeypatch):
    MUTATIONS_BACKWARD2[name](monkeypatch)
    assert any(_fails(fn, *args) for fn, args in PINS_BACKWARD2), f"mutation {name} not caught"
