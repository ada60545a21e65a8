"""GPU parity of the Sol-Attn2 HIP path against the CPU oracle (through the C ABI).

Integer / byte work is compared bit for bit: the E4M3 codes and fp32 block
scales (both sides take the rounding decisions in fp32), and the key-group
membership wherever a key's projection is more than a small margin from its
block's mean projection (the decision is taken in fp32 on the GPU, fp64 in the
oracle).  Masks are bit-exact outside the 1e-3 proxy margin.  Outputs: relative
L2 <= 3e-2 against the float64 oracle run on the same dequantized Q/K, with the
kernel's own selection, both over all sampled rows and for every 32-row anchor
on its own (so one anchor with a wrong tail cannot hide in the aggregate).  The
kernel's selected-token-pair counter equals the count of its masks.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from oracle import sol_attn as sa
from oracle import sol_attn2 as s2
from parity import anchor_errors, mask_check, pair_check, say, to_gpu
from workloads import block_offset_tensor, sol2_bench, wan_dit

pytestmark = pytest.mark.gpu
REL_L2_FP8 = 3e-2


def _qkv(B, N, H, seed, offset=1.0):
    return [block_offset_tensor(B, N, H, 128, seed + i, offset) for i in range(3)]


def _head(t, b, h):
    return t[b, :, h, :].to(torch.float64).numpy()


def run_case(q, k, v, tau, sink_start=None, sink_tokens=0, heads=None, sample=None, seed=0, check_prep=True):
    B, N, H, _ = q.shape
    say(f"[sol_attn2] B={B} N={N} H={H} tau={tau} sink=({sink_start},{sink_tokens})")
    qg, kg, vg = to_gpu(q, k, v)
    out = torch.empty_like(qg)
    _, masks, ws, pairs = bsa.debug_routing(2, qg, kg, vg, tau, "diag", sink_start, sink_tokens, out=out,
                                            return_pairs=True)
    out2 = bsa.sol_attn2(qg, kg, vg, tau, "diag", sink_start, sink_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "export and product calls disagree"
    views = bsa.workspace_views(2, ws, B, N, H)
    nb = (N + 63) // 64
    out_c = out.float().cpu().numpy()
    gsel = masks.numpy()
    assert pairs == sa.selected_pairs(gsel, N), "selected-pair counter differs from the kernel's masks"
    rng = np.random.default_rng(seed)
    got, want, want_unq = [], [], []
    worst_anchor = 0.0
    flips = 0
    scale = 1 / math.sqrt(128)
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            qh, kh, vh = _head(q, b, h), _head(k, b, h), _head(v, b, h)
            r = s2.sol_attn2_head(qh, kh, vh, tau, sink_start, sink_tokens, query_blocks=[])
            if check_prep:
                # codes and scales: bit-exact
                q8 = views["q8"][b, h, :N].cpu().numpy()
                k8 = views["k8"][b, h, :N].cpu().numpy()
                assert np.array_equal(q8, r.q_codes), f"Q codes differ at {np.argwhere(q8 != r.q_codes)[:5]}"
                assert np.array_equal(k8, r.k_codes), "K codes differ"
                assert np.array_equal(views["qscale"][b, h, :nb].cpu().numpy(), r.q_scales)
                assert np.array_equal(views["kscale"][b, h, :nb].cpu().numpy(), r.k_scales)
                np.testing.assert_allclose(views["qhat"][b, h].cpu().double().numpy(), r.qhat, rtol=1e-4, atol=1e-6)
                # group membership outside a tie margin; group means
                ghi = views["ghi"][b, h, :nb].cpu().numpy().view(np.uint64)
                for j, (s, e) in enumerate(sa.block_ranges(N)):
                    p = r.k_deq[s:e] @ r.qhat
                    ref_hi = p >= p.mean()
                    gpu_hi = ((np.uint64(ghi[j]) >> np.arange(e - s, dtype=np.uint64)) & np.uint64(1)).astype(bool)
                    tie = np.abs(p - p.mean()) <= 1e-4 * (np.abs(p).max() + 1e-30)
                    assert not ((gpu_hi != ref_hi) & ~tie).any(), f"group split differs in block {j}"
            # masks
            ref_sel = r.sel
            near = np.abs(r.s_hat - r.tau_i[:, None]) <= 1e-3
            forced = np.zeros_like(near)
            forced[:, sa.sink_block_mask(N, sink_start, sink_tokens)] = True
            bad = (gsel[b, h] != ref_sel) & ~(near & ~forced)
            assert not bad.any(), f"{int(bad.sum())} mask bits differ outside the margin"
            flips += int((gsel[b, h] != ref_sel).sum())
            blocks = range(nb) if sample is None else sorted(set(rng.choice(nb, size=min(sample, nb), replace=False)) | {nb - 1})
            groups_unq = s2.all_key_groups(kh, vh, qh.mean(axis=0))
            for i in blocks:
                s, e = i * 64, min(i * 64 + 64, N)
                want.append(s2.attend_query_block2(r.q_deq, r.k_deq, vh, i, gsel[b, h, i], r.groups, scale))
                got.append(out_c[b, s:e, h, :])
                worst_anchor = max([worst_anchor] + anchor_errors(got[-1], want[-1]))
                want_unq.append(s2.attend_query_block2(qh, kh, vh, i, gsel[b, h, i], groups_unq, scale))
    got, want, want_unq = (np.concatenate(x) for x in (got, want, want_unq))
    assert np.isfinite(got).all()
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    err_unq = np.linalg.norm(got - want_unq) / np.linalg.norm(want_unq)
    say(f"   ok: rel L2 {err:.2e} (vs unquantized oracle {err_unq:.2e}), max abs {np.abs(got - want).max():.2e}, "
        f"worst anchor rel L2 {worst_anchor:.2e}, mask flips {flips}, density {gsel.mean():.3f}")
    assert err <= REL_L2_FP8, f"rel L2 {err:.3e} > {REL_L2_FP8}"
    assert worst_anchor <= REL_L2_FP8, f"an anchor's rel L2 {worst_anchor:.3e} > {REL_L2_FP8}"
    return out, masks, views


@pytest.mark.parametrize("tau", [1.0, 0.0, 2.0])
def test_tiny_workload_full(tau):
    q, k, v = _qkv(1, 1024, 2, 1000)
    run_case(q, k, v, tau)


@pytest.mark.parametrize("N", [40, 64, 65, 200, 1000, 4493])
def test_ragged_lengths(N):
    q, k, v = _qkv(1, N, 2, 2100 + N)
    run_case(q, k, v, 0.8)


@pytest.mark.parametrize("sink", [(0, 130), (None, 70), (0, 1000)])
def test_exact_sink(sink):
    q, k, v = _qkv(1, 1000, 2, 2200)
    out, masks, _ = run_case(q, k, v, 1.5, sink_start=sink[0], sink_tokens=sink[1])
    if sink == (0, 1000):
        assert masks.all()


def test_batch_and_odd_heads():
    q, k, v = _qkv(2, 700, 3, 2300)
    run_case(q, k, v, 0.5)


def test_zero_block_uses_unit_scale():
    """An all-zero Q/K block quantizes with scale 1 and all-zero codes."""
    q, k, v = _qkv(1, 300, 2, 2400)
    q[:, 64:128] = 0
    k[:, 128:192] = 0
    out, _, views = run_case(q, k, v, 1.0)
    assert views["qscale"][0, :, 1].eq(1.0).all() and views["kscale"][0, :, 2].eq(1.0).all()


def test_wan21_dit_shape():
    q, k, v = wan_dit().qkv()
    run_case(q, k, v, 1.0, heads=[0, 7, 11], sample=6, seed=5)


def test_sol2_bench_shape():
    """B=1, H=32, N=32768, tau near 90% sparsity: E4M3 codes and scales, the mean-query
    direction, the group split bits and the routing of all 32 heads; 3 sampled query blocks
    per head (the last included) for the outputs."""
    q, k, v = sol2_bench().qkv()
    run_case(q, k, v, 1.28, heads=None, sample=3, seed=6)


def test_single_token():
    """N = 1: one key, so exact and tail branches both return its value (up to the FP8 path)."""
    q, k, v = _qkv(1, 1, 2, 2500)
    out, _, _ = run_case(q, k, v, 1.0)
    np.testing.assert_allclose(out.float().cpu().numpy(), v.float().numpy(), rtol=1e-2, atol=1e-2)


def test_maximum_sequence_length():
    """524288 tokens, the largest length the library accepts: codes, scales, groups and routing of
    the head in full, sampled output rows including the last block."""
    q, k, v = _qkv(1, 524288, 1, 2600)
    run_case(q, k, v, 1.28, sample=2, seed=7)


def test_tail_logit_far_above_the_first_tiles():
    """Key block 40 holds +-300 e_0 in alternate tokens: its block mean is zero, so it stays in
    the tail, while its upper group (the keys along the mean query, e_0) scores about 380 log2
    units above the tail groups of the first tiles for queries with q_0 = 10.  The tail pass's
    fixed reference then overflows and the workgroup is redone with the running maximum; the
    result still matches the oracle."""
    B, N, H = 1, 4096, 1
    q, k, v = _qkv(B, N, H, 3000)
    q[..., 0] = 10.0
    blk = 40
    k[0, blk * 64:(blk + 1) * 64, 0, :] = 0.0
    k[0, blk * 64:(blk + 1) * 64, 0, 0] = 300.0 * torch.tensor([1.0, -1.0]).repeat(32)
    out, masks, _ = run_case(q, k, v, 1.0)
    assert (~masks[0, 0, :, blk]).sum() >= 8, "block 40 is meant to stay in the tail"


def test_exact_logit_far_above_the_first_exact_block():
    """The bf16-V exact pass takes each row's reference from its first exact block (here the
    sink's block 0); key block 40, along the queries' dominant direction at 300 e_0, is
    selected and scores about 380 log2 units higher, so the sums overflow that reference and
    the workgroup is redone with the running maximum.  The result still matches the oracle."""
    B, N, H = 1, 4096, 1
    q, k, v = _qkv(B, N, H, 3100)
    q[..., 0] = 10.0
    blk = 40
    k[0, blk * 64:(blk + 1) * 64, 0, :] = 0.0
    k[0, blk * 64:(blk + 1) * 64, 0, 0] = 300.0
    out, masks, _ = run_case(q, k, v, 1.0, sink_start=0, sink_tokens=64)
    assert masks[0, 0, :, blk].all() and masks[0, 0, :, 0].all()


@pytest.mark.parametrize("case", ["tail", "sink"])
def test_hand_worked_group_fixture(case):
    """The hand-worked head of tests/golden/sol2_groups.txt (d = 4 values embedded in d = 128,
    dims 4.. zero): the kernels' mean-query direction, split bits (the tie included) and group
    counts are exactly the fixture's, and every output row matches its closed form (tau = 100:
    no exact block; with the sink [64, 96): block 1 exact, delta_t nonzero in the last anchor)."""
    from sol2_fixture import inputs, load
    fx = load(128)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).view(1, 96, 1, 128) for x in inputs(128))
    sink = (64, 32) if case == "sink" else (None, 0)
    say(f"[sol_attn2 fixture] case {case}")
    qg, kg, vg = to_gpu(q, k, v)
    out = torch.empty_like(qg)
    _, masks, ws, pairs = bsa.debug_routing(2, qg, kg, vg, 100.0, "diag", sink[0], sink[1], out=out,
                                            return_pairs=True)
    torch.cuda.synchronize()
    want_sel = np.array([[False, True], [False, True]]) if case == "sink" else np.zeros((2, 2), dtype=bool)
    assert np.array_equal(masks[0, 0].numpy(), want_sel)
    assert pairs == (96 * 32 if case == "sink" else 0)
    views = bsa.workspace_views(2, ws, 1, 96, 1)
    qhat = views["qhat"][0, 0].cpu().double().numpy()
    assert np.array_equal(qhat[:4], fx["qhat"]) and not qhat[4:].any()
    ghi = views["ghi"][0, 0, :2].cpu().numpy().view(np.uint64)
    want_hi0 = sum(1 << u for u in range(64) if u % 8 in fx["hi_residues"].astype(int).tolist())
    assert int(ghi[0]) == want_hi0, f"block 0 split {int(ghi[0]):#018x} != {want_hi0:#018x}"
    assert int(ghi[1]) == (1 << 32) - 1, "the all-equal partial block must be one group"
    glogn = views["glogn"][0, 0, :2].cpu().double().numpy()
    np.testing.assert_allclose(glogn[0], np.log([fx["n_hi"][0], fx["n_lo"][0]]), rtol=1e-6)
    assert glogn[1, 0] == pytest.approx(math.log(fx["n_b1"][0]), rel=1e-6) and glogn[1, 1] == -np.inf
    gk = views["gk"][0, 0, :2].cpu().double().numpy()
    np.testing.assert_allclose(gk[0, 0, :4], fx["kbar_hi"], atol=4e-3)
    np.testing.assert_allclose(gk[0, 1, :4], fx["kbar_lo"], atol=4e-3)
    np.testing.assert_allclose(gk[1, 0, :4], fx["kbar_b1"], atol=4e-3)
    got = out[0, :, 0, :].float().cpu().double().numpy()
    assert not got[:, 4:].any()
    if case == "tail":
        rows = [("out_tail_a0", 0, 32), ("out_tail_a1", 32, 64), ("out_tail_a2", 64, 96)]
    else:
        rows = [("out_sink_a0", 0, 32), ("out_sink_a1", 32, 64), ("out_sink_a2_hi", 64, 80),
                ("out_sink_a2_lo", 80, 96)]
    want = np.zeros((96, 4))
    for name, t0, t1 in rows:
        want[t0:t1] = fx[name]
    err = np.linalg.norm(got[:, :4] - want) / np.linalg.norm(want)
    mx = np.abs(got[:, :4] - want).max()
    say(f"   ok: rel L2 {err:.2e}, max abs {mx:.2e}")
    assert err <= REL_L2_FP8 and mx <= 3e-2
