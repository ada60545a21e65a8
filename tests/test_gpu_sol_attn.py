"""GPU parity of the Sol-Attn HIP path against the CPU oracle (through the C ABI).

Masks: bit-exact wherever |s_hat - tau_i| > 1e-3 (scaled-logit units).
Outputs: relative L2 <= 1e-2 and max-abs <= 3e-2 against the float64 oracle, the
oracle evaluated with the selection the kernel made (in-margin flips are both
correct readings).  Small shapes compare every output row; the full-size
workload shapes compare the full routing and a seeded sample of query blocks.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from oracle import sol_attn as sa
from parity import compare_out, mask_check, oracle_rows, order_check, pair_check, say, to_gpu
from workloads import block_offset_tensor, long_sink, operator_bench, wan_dit

pytestmark = pytest.mark.gpu


def _qkv(B, N, H, seed, offset=1.0):
    return [block_offset_tensor(B, N, H, 128, seed + i, offset) for i in range(3)]


def run_case(q, k, v, tau, sink_start=None, sink_tokens=0, thresh="diag", sample=None, seed=0):
    B, N, H, _ = q.shape
    say(f"[sol_attn] B={B} N={N} H={H} tau={tau} sink=({sink_start},{sink_tokens}) thresh={thresh}")
    qg, kg, vg = to_gpu(q, k, v)
    out = torch.empty_like(qg)
    _, masks, ws, pairs = bsa.debug_routing(1, qg, kg, vg, tau, thresh, sink_start, sink_tokens, out=out,
                                            return_pairs=True)
    out2 = bsa.sol_attn(qg, kg, vg, tau, thresh, sink_start, sink_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), (f"export and product calls disagree: max diff "
                                    f"{(out.float() - out2.float()).abs().max().item():.3e} in "
                                    f"{int((out != out2).sum())} elements")
    ref = sa.routing_only(q, k, tau, sink_start, sink_tokens, thresh)
    nb = (N + 63) // 64
    forced = np.zeros((B, H, nb, nb), dtype=bool)
    forced[..., sa.sink_block_mask(N, sink_start, sink_tokens)] = True
    gsel = masks.numpy()
    flips = mask_check(gsel, ref["sel"], ref["s_hat"], ref["tau_i"], forced)
    pair_check(pairs, gsel, ref["sel"], N)
    order_check(1, ws, gsel, B, N, H)
    out_c = out.float().cpu().numpy()
    rng = np.random.default_rng(seed)
    got, want = [], []
    for b in range(B):
        for h in range(H):
            blocks = range(nb) if sample is None else sorted(set(rng.choice(nb, size=min(sample, nb), replace=False)) | {nb - 1})
            for i in blocks:
                s, e = i * 64, min(i * 64 + 64, N)
                want.append(oracle_rows(q, k, v, b, h, i, gsel[b, h, i]))
                got.append(out_c[b, s:e, h, :])
    err, mx = compare_out(np.concatenate(got), np.concatenate(want), what=f"N={N} tau={tau}")
    say(f"   ok: rel L2 {err:.2e} max abs {mx:.2e}, in-margin mask flips {flips}, "
        f"density {gsel.mean():.3f}")
    return out, masks, ws


@pytest.mark.parametrize("tau", [1.0, 0.0, -0.5, 2.5])
def test_tiny_workload_full(tau):
    """B=1, H=2, N=1024 block-offset data: every output row and every mask bit."""
    q, k, v = _qkv(1, 1024, 2, 1000)
    run_case(q, k, v, tau)


@pytest.mark.parametrize("N", [40, 64, 65, 200, 1000, 4493, 8192 + 13])
def test_ragged_lengths(N):
    """Partial last blocks, a sequence shorter than one block, more than one 64-block chunk."""
    q, k, v = _qkv(1, N, 2, 1100 + N)
    run_case(q, k, v, 0.8)


@pytest.mark.parametrize("sink", [(0, 130), (None, 70), (200, 300), (None, 1), (0, 1)])
def test_exact_sink(sink):
    q, k, v = _qkv(1, 1000, 2, 1200)
    run_case(q, k, v, 1.5, sink_start=sink[0], sink_tokens=sink[1])


def test_whole_sequence_sink_is_dense_attention():
    """A sink over [0, N) makes every block exact: textbook attention (fp32 CPU SDPA)."""
    q, k, v = _qkv(1, 777, 3, 1300)
    out, masks, _ = run_case(q, k, v, 1.0, sink_start=0, sink_tokens=777)
    assert masks.all()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.float().transpose(1, 2), k.float().transpose(1, 2), v.float().transpose(1, 2)).transpose(1, 2)
    compare_out(out.float().cpu().numpy(), ref.numpy(), what="dense")


def test_batch_and_odd_heads():
    q, k, v = _qkv(2, 700, 3, 1400)
    run_case(q, k, v, 0.5)


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_exact_covariance_threshold(tau):
    q, k, v = _qkv(1, 2000, 2, 1500)
    run_case(q, k, v, tau, thresh="exact")


def test_identical_keys_are_exact():
    """Keys constant within each block: the proxy branch is exact, so any tau gives dense attention."""
    q, k, v = _qkv(1, 1024, 2, 1600)
    kb = k.float().view(1, 16, 64, 2, 128).mean(dim=2, keepdim=True).expand(1, 16, 64, 2, 128)
    k = kb.reshape(1, 1024, 2, 128).to(torch.bfloat16).contiguous()
    out, _, _ = run_case(q, k, v, 1.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.float().transpose(1, 2), k.float().transpose(1, 2), v.float().transpose(1, 2)).transpose(1, 2)
    compare_out(out.float().cpu().numpy(), ref.numpy(), what="identical keys")


def test_summaries_and_threshold_match_oracle():
    """Workspace block means, V means and tau_i against the oracle's definitions."""
    N, H = 1000, 3
    q, k, v = _qkv(1, N, H, 1700)
    qg, kg, vg = to_gpu(q, k, v)
    ws = bsa.alloc_workspace(1, qg)
    for thresh in ("diag", "exact"):
        bsa.prepare(1, qg, kg, vg, 0.7, ws, thresh)
        torch.cuda.synchronize()
        views = bsa.workspace_views(1, ws, 1, N, H)
        nb = views["nb"]
        for h in range(H):
            qh, kh, vh = (t[0, :, h, :].double().numpy() for t in (q, k, v))
            qbar, kbar = sa.block_means(qh), sa.block_means(kh)
            vbar = sa.block_sums(vh) / sa.block_counts(N)[:, None]
            np.testing.assert_allclose(views["qbar"][0, h, :nb].cpu().double().numpy(), qbar, rtol=1e-5, atol=1e-6)
            kt = views["kbar_t"][0, h, :, :nb, :].cpu().double().permute(1, 0, 2).reshape(nb, 128).numpy()
            np.testing.assert_allclose(kt, kbar, rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(views["kbar_h"][0, h, :nb].cpu().double().numpy(), kbar, rtol=8e-3, atol=1e-6)
            np.testing.assert_allclose(views["vbar_h"][0, h, :nb].cpu().double().numpy(), vbar, rtol=8e-3, atol=1e-6)
            assert not views["kbar_h"][0, h, nb:].float().abs().sum().item()     # zero padding rows
            fn = sa.diag_threshold if thresh == "diag" else sa.exact_threshold
            tau_ref = fn(qbar, kbar, 0.7, 1 / math.sqrt(128))[0]
            np.testing.assert_allclose(views["tau_i"][0, h, :nb].cpu().double().numpy(), tau_ref, rtol=1e-4, atol=2e-5)


@pytest.mark.parametrize("N,H", [(40, 2), (130, 1), (14040, 12), (131584, 2)])
def test_exact_threshold_sizes(N, H):
    """The full-covariance threshold (sliced outer products, reduction, wide tau pass) at one
    block, a few blocks (most slices empty), the Wan-2.1 shape and the longest sequence:
    covariance, mu_K and tau_i against the oracle's definitions (Eq. (5))."""
    q, k, v = _qkv(1, N, H, 1750)
    qg, kg, vg = to_gpu(q, k, v)
    ws = bsa.alloc_workspace(1, qg)
    bsa.prepare(1, qg, kg, vg, 1.3, ws, "exact")
    torch.cuda.synchronize()
    views = bsa.workspace_views(1, ws, 1, N, H)
    nb = views["nb"]
    for h in range(H):
        qh, kh = (t[0, :, h, :].double().numpy() for t in (q, k))
        qbar, kbar = sa.block_means(qh), sa.block_means(kh)
        cov = np.cov(kbar.T, bias=True) if nb > 1 else np.zeros((128, 128))
        np.testing.assert_allclose(views["kcov"][0, h].cpu().double().numpy(), cov, rtol=1e-4,
                                   atol=1e-5 * max(1.0, np.abs(cov).max()))
        np.testing.assert_allclose(views["kstat"][0, h, 0].cpu().double().numpy(), kbar.mean(axis=0), rtol=1e-5,
                                   atol=1e-6)
        tau_ref = sa.exact_threshold(qbar, kbar, 1.3, 1 / math.sqrt(128))[0]
        np.testing.assert_allclose(views["tau_i"][0, h, :nb].cpu().double().numpy(), tau_ref, rtol=1e-4, atol=2e-5)


def test_deterministic_and_stream_ordered():
    q, k, v = _qkv(1, 3000, 2, 1800)
    qg, kg, vg = to_gpu(q, k, v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = bsa.sol_attn(qg, kg, vg, 0.9)
        b = bsa.sol_attn(qg, kg, vg, 0.9)
    s.synchronize()
    assert torch.equal(a, b)


def test_python_binding_rejects_bad_tensors():
    q, k, v = to_gpu(*_qkv(1, 128, 1, 1900))
    with pytest.raises(ValueError):
        bsa.sol_attn(q.float(), k, v)
    with pytest.raises(ValueError):
        bsa.sol_attn(q, k[:, :64].contiguous(), v)
    with pytest.raises(ValueError):
        bsa.sol_attn(q, k, v, tau=float("nan"))
    with pytest.raises(bsa.SolAttnError):
        bsa.sol_attn(q, k, v, sink_start=100, sink_tokens=100)


# ---- workload shapes at full size: full routing, sampled outputs -------------------

@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_wan21_dit_shape(tau):
    """B=1, H=12, N=14040 (9x30x52 raster grid, last block 24 tokens), smooth random field."""
    q, k, v = wan_dit().qkv()
    run_case(q, k, v, tau, sample=6, seed=int(tau * 10))


def test_operator_bench_shape():
    """B=1, H=32, N=32768 block-offset data (the operator benchmark shape)."""
    q, k, v = operator_bench().qkv()
    run_case(q, k, v, 1.28, sample=3, seed=3)


def test_long_sequence_with_text_sink():
    """B=1, H=32, 512 text tokens (exact sink) + 65536 video tokens."""
    w = long_sink(65536)
    q, k, v = w.qkv()
    run_case(q, k, v, 1.3, sink_start=0, sink_tokens=512, sample=2, seed=4)


# The target range's corners (Sol-Attn2 draft, "FP8 Kernel Performance": 32K-128K tokens; the
# Sources page's benchmark scope: 80/85/90% token-pair sparsity).  The tau values were bisected
# on this data with the kernel's own selected-pair counter (bench.py's search) and are kept as
# constants; the realised sparsity is checked from the masks.
@pytest.mark.parametrize("target,tau", [(0.80, 0.8347), (0.85, 1.0306)])
def test_operator_bench_shape_at_80_and_85_percent(target, tau):
    """B=1, H=32, N=32768 at 80% and 85% token-pair sparsity: full routing of every head and
    3 sampled query blocks per head (the last included)."""
    q, k, v = operator_bench().qkv()
    _, masks, _ = run_case(q, k, v, tau, sample=3, seed=int(100 * target))
    sp = sa.realised_sparsity(masks.numpy(), 32768)
    say(f"   realised sparsity {sp:.4f} (target {target})")
    assert abs(sp - target) <= 0.0025


def test_long_sequence_131k_with_text_sink():
    """B=1, H=32, 512 text tokens (exact sink) + 131072 video tokens at ~90% sparsity (the
    automatic four key splits): full routing of every head against the oracle and 4 sampled
    query blocks per head, the last one always among them."""
    w = long_sink(131072)
    q, k, v = w.qkv()
    _, masks, _ = run_case(q, k, v, 1.30, sink_start=0, sink_tokens=512, sample=4, seed=11)
    sp = sa.realised_sparsity(masks.numpy(), q.shape[1])
    say(f"   realised sparsity {sp:.4f}")
    assert 0.88 <= sp <= 0.92


@pytest.mark.parametrize("N", [32768, 32768 + 13])
def test_kv_splits_match_oracle(N):
    """Split-KV (README "Long-sequence tuning": kv_splits): 1, 2, 4 and 8 key-range splits all match
    the oracle, and agree with each other to bf16 rounding."""
    q, k, v = _qkv(1, N, 2, 2500)
    tau = 1.0
    qg, kg, vg = to_gpu(q, k, v)
    _, masks, _ = bsa.debug_routing(1, qg, kg, vg, tau)
    gsel = masks.numpy()
    ref = sa.routing_only(q, k, tau)
    mask_check(gsel, ref["sel"], ref["s_hat"], ref["tau_i"])
    nb = (N + 63) // 64
    want = np.concatenate([oracle_rows(q, k, v, 0, h, i, gsel[0, h, i]) for h in range(2) for i in range(nb)])
    outs = {}
    for kv in (1, 2, 4, 8):
        eff = bsa.kv_splits_for(1, N, 2, kv)
        out = bsa.sol_attn(qg, kg, vg, tau, kv_splits=kv)
        torch.cuda.synchronize()
        oc = out.float().cpu().numpy()
        got = np.concatenate([oc[0, i * 64:min(N, i * 64 + 64), h, :] for h in range(2) for i in range(nb)])
        err, mx = compare_out(got, want, what=f"kv_splits={kv}")
        say(f"   kv_splits {kv} (effective {eff}): rel L2 {err:.2e} max abs {mx:.2e}")
        outs[kv] = out.float()
    for kv in (2, 4, 8):
        d = (outs[kv] - outs[1]).norm() / outs[1].norm()
        assert d < 1e-2, f"kv_splits={kv} vs 1: {d:.3e}"


def test_head_major_copies_are_the_inputs():
    """Stage 1 writes head-major copies of K and V (the tile source of stage 2 and of the
    backward); they are the inputs, bit for bit."""
    B, N, H = 2, 333, 3
    q, k, v = _qkv(B, N, H, 2700)
    qg, kg, vg = to_gpu(q, k, v)
    ws = bsa.alloc_workspace(1, qg)
    bsa.prepare(1, qg, kg, vg, 1.0, ws)
    torch.cuda.synchronize()
    views = bsa.workspace_views(1, ws, B, N, H)
    assert torch.equal(views["kh"], kg.permute(0, 2, 1, 3))
    assert torch.equal(views["vh"], vg.permute(0, 2, 1, 3))


# ---- degenerate inputs and the maximum length ---------------------------------------

@pytest.mark.parametrize("N", [1, 2])
def test_single_block_shorter_than_a_tile(N):
    """One partial block: its proxy equals its threshold (zero spread), a tie that either
    decision satisfies; the oracle comparison uses the kernel's decision.  With one token both
    branches give that token's value."""
    q, k, v = _qkv(1, N, 2, 2600 + N)
    out, _, _ = run_case(q, k, v, 1.0)
    if N == 1:
        compare_out(out.float().cpu().numpy(), v.float().numpy(), what="N=1")


def test_zero_queries_give_the_value_mean():
    """All-zero queries: every logit is 0 and every proxy equals the threshold, so nothing is
    selected and the output is the mean of V over the whole sequence (closed form)."""
    B, N, H = 1, 1000, 2
    _, k, v = _qkv(B, N, H, 2700)
    q = torch.zeros_like(k)
    out, masks, _ = run_case(q, k, v, 0.5)
    assert not masks.any()
    want = v.float().mean(dim=1, keepdim=True).expand(B, N, H, 128)
    compare_out(out.float().cpu().numpy(), want.numpy(), what="zero queries")


def test_maximum_sequence_length():
    """524288 tokens (128 routing chunks, the largest length the library accepts): full routing
    against the oracle and a sample of query blocks including the last."""
    N = 524288
    q, k, v = _qkv(1, N, 1, 2800)
    assert bsa.validate(1, N, 1, 128, 1.28, None, 0) == 0
    assert bsa.validate(1, N + 1, 1, 128, 1.28, None, 0) != 0
    run_case(q, k, v, 1.28, sample=3, seed=5)


def test_exact_logit_far_above_the_pooled_reference():
    """Key block 40 holds +-300 e_0 in alternate tokens and is the sink, so it is exact while its
    pooled logit (the block mean, zero) stays near the first pooled tile's maximum.  For queries
    with q_0 = 10 its exact logits sit about 380 log2 units above that fixed reference, the sums
    overflow, and the workgroup is redone with the running maximum; the result still matches the
    oracle."""
    B, N, H = 1, 4096, 1
    q, k, v = _qkv(B, N, H, 3200)
    q[..., 0] = 10.0
    blk = 40
    k[0, blk * 64:(blk + 1) * 64, 0, :] = 0.0
    k[0, blk * 64:(blk + 1) * 64, 0, 0] = 300.0 * torch.tensor([1.0, -1.0]).repeat(32)
    out, masks, _ = run_case(q, k, v, 1.0, sink_start=blk * 64, sink_tokens=64)
    assert masks[0, 0, :, blk].all()


def test_kv_splits_with_batch_sink_and_ragged_tail():
    """Key splits 1, 2 and 4 over a shape that exercises every edge at once: two batches, three
    heads, 12317 tokens (193 blocks, so the last routing chunk holds one block of 29 tokens) and a
    200-token sink in the middle of the sequence.  Every output row matches the oracle under the
    kernel's own masks, and the splits agree with each other."""
    B, N, H = 2, 12317, 3
    q, k, v = _qkv(B, N, H, 3300)
    tau, s0, st = 0.5, 5000, 200
    qg, kg, vg = to_gpu(q, k, v)
    _, masks, _ = bsa.debug_routing(1, qg, kg, vg, tau, "diag", s0, st)
    gsel = masks.numpy()
    ref = sa.routing_only(q, k, tau, s0, st, "diag")
    nb = (N + 63) // 64
    forced = np.zeros((B, H, nb, nb), dtype=bool)
    forced[..., sa.sink_block_mask(N, s0, st)] = True
    mask_check(gsel, ref["sel"], ref["s_hat"], ref["tau_i"], forced)
    want = np.concatenate([oracle_rows(q, k, v, b, h, i, gsel[b, h, i])
                           for b in range(B) for h in range(H) for i in range(nb)])
    for kv in (2, 4):
        # each (head, split) gets its own order, by the counts within the split's key range
        _, m_kv, ws_kv = bsa.debug_routing(1, qg, kg, vg, tau, "diag", s0, st, kv_splits=kv)
        assert torch.equal(m_kv, masks)
        order_check(1, ws_kv, gsel, B, N, H, kv_splits=kv)
    outs = {}
    for kv in (1, 2, 4):
        out = bsa.sol_attn(qg, kg, vg, tau, "diag", s0, st, kv_splits=kv)
        torch.cuda.synchronize()
        oc = out.float().cpu().numpy()
        got = np.concatenate([oc[b, i * 64:min(N, i * 64 + 64), h, :]
                              for b in range(B) for h in range(H) for i in range(nb)])
        err, mx = compare_out(got, want, what=f"kv_splits={kv}")
        say(f"   kv_splits {kv} (effective {bsa.kv_splits_for(B, N, H, kv)}): rel L2 {err:.2e} max abs {mx:.2e}")
        outs[kv] = out.float()
    for kv in (2, 4):
        d = (outs[kv] - outs[1]).norm() / outs[1].norm()
        assert d < 1e-2, f"kv_splits={kv} vs 1: {d:.3e}"
