"""Hand-worked pin of the Sol-Attn2 group readings (CPU only).

tests/golden/sol2_groups.txt works one 96-token head out by hand (Sol-Attn2 draft, Method,
Eqs. (1)-(3)): the mean-query direction, the split of each key block at its mean projection
of the dequantized keys with ties in G_hi, the drop of an empty group, the group sizes and
means, the anchors' tail weights, and the outputs with and without an exact sink block.  The
inputs are chosen so that the plausible other readings (median split, ties to G_lo, a
per-query-block direction, a split on the unquantized keys) all give other answers.
"""
import math

import numpy as np

from oracle import sol_attn2 as s2
from sol2_fixture import inputs, load


def _check_groups(r, fx):
    np.testing.assert_array_equal(r.qhat, fx["qhat"])
    g0, g1 = r.groups[0], r.groups[1]
    assert len(g0) == 2, f"block 0 has {len(g0)} groups"
    (m_hi, n_hi, kb_hi, vb_hi), (m_lo, n_lo, kb_lo, vb_lo) = g0
    assert sorted(set((np.flatnonzero(m_hi) % 8).tolist())) == fx["hi_residues"].astype(int).tolist()
    assert not (m_hi & m_lo).any() and (m_hi | m_lo).all()
    assert (n_hi, n_lo) == (fx["n_hi"][0], fx["n_lo"][0])
    np.testing.assert_allclose(kb_hi, fx["kbar_hi"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(vb_hi, fx["vbar_hi"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(kb_lo, fx["kbar_lo"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(vb_lo, fx["vbar_lo"], rtol=0, atol=1e-15)
    assert len(g1) == 1, "an all-equal block must form one group (the empty one dropped)"
    m1, n1, kb1, vb1 = g1[0]
    assert m1.all() and n1 == fx["n_b1"][0]
    np.testing.assert_allclose(kb1, fx["kbar_b1"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(vb1, fx["vbar_b1"], rtol=0, atol=1e-15)


def test_group_readings_match_the_hand_worked_fixture():
    fx = load()
    q, k, v = inputs()
    scale = 1 / math.sqrt(4)
    # case "tail": nothing exact, every row is its anchor's nu_a
    r = s2.sol_attn2_head(q, k, v, tau=100.0)
    assert not r.sel.any()
    _check_groups(r, fx)
    for a, (t0, t1) in enumerate(((0, 32), (32, 64), (64, 96))):
        np.testing.assert_allclose(r.out[t0:t1], np.tile(fx[f"out_tail_a{a}"], (t1 - t0, 1)), rtol=1e-13)
    tail = [g for gl in r.groups for g in gl]
    for a, (t0, t1) in enumerate(((0, 32), (32, 64), (64, 96))):
        ln_z, _, nu = s2.tail_stats(r.q_deq[t0:t1].mean(axis=0), tail, scale)
        assert abs(ln_z - math.log(fx[f"w_tail_a{a}"].sum())) < 1e-12
        np.testing.assert_allclose(nu, fx[f"out_tail_a{a}"], rtol=1e-13)
    # case "sink": block 1 exact for every query block, block 0's two groups in the tail
    r2 = s2.sol_attn2_head(q, k, v, tau=100.0, sink_start=64, sink_tokens=32)
    np.testing.assert_array_equal(r2.sel, np.array([[False, True], [False, True]]))
    _check_groups(r2, fx)
    for name, (t0, t1) in (("out_sink_a0", (0, 32)), ("out_sink_a1", (32, 64)), ("out_sink_a2_hi", (64, 80)),
                           ("out_sink_a2_lo", (80, 96))):
        np.testing.assert_allclose(r2.out[t0:t1], np.tile(fx[name], (t1 - t0, 1)), rtol=1e-13)


def test_fixture_inputs_quantize_as_stated():
    """Every fixture value is an E4M3 value times its block scale except U's 1.046875, which
    rounds to 1 (the fixture's quantization note)."""
    q, k, _ = inputs()
    qc, qs, qd = s2.quantize_head(q)
    kc, ks, kd = s2.quantize_head(k)
    assert list(qs) == [2.0 ** -7, 2.0 ** -7] and list(ks) == [2.0 ** -7, 2.0 ** -8]
    np.testing.assert_array_equal(qd, q)
    diff = np.argwhere(kd != k)
    assert set(map(tuple, diff.tolist())) == {(u, 1) for u in range(7, 64, 8)}
    np.testing.assert_array_equal(kd[7::8][:8, 1], np.ones(8))
