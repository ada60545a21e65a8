"""GPU parity of the Sol-Attn2 FP8-PV path (ExpCast P, per-head FP8 V) against the oracle.

Bit for bit: the per-head V scale and the E4M3 V codes (fp32 division and RNE on
both sides), read back from the workspace in the kernel's operand order.  Outputs:
relative L2 <= 3e-2 against the float64 oracle with pv="expcast" on the same
dequantized Q/K and the kernel's own routing, over all sampled rows and for every
32-row anchor on its own.  Both sides take the ExpCast pivot online, one selected
64-token block at a time in ascending order (each block's bytes against the
running row maximum including that block); the bytes can still differ by one
step where fp32 and fp64 round a score differently, which the output bar covers.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from oracle import sol_attn2 as s2
from parity import anchor_errors, say, to_gpu
from workloads import block_offset_tensor, sol2_bench

pytestmark = pytest.mark.gpu
REL_L2_FP8 = 3e-2


def _qkv(B, N, H, seed, offset=1.0):
    return [block_offset_tensor(B, N, H, 128, seed + i, offset) for i in range(3)]


def _head(t, b, h):
    return t[b, :, h, :].to(torch.float64).numpy()


def _operand_order(codes_nd: np.ndarray, tp: int) -> np.ndarray:
    """[N, d] codes -> [d, tp] in the kernel's per-block order (token 32h + 8q + 4g + r
    at position 32g + 16h + 4q + r), zero-padded."""
    n, d = codes_nd.shape
    out = np.zeros((d, tp), dtype=np.uint8)
    p = np.arange(tp)
    blk, pos = p // 64, p % 64
    g, e = pos // 32, pos % 32
    tok = blk * 64 + 32 * (e // 16) + 8 * ((e // 4) % 4) + 4 * g + e % 4
    ok = tok < n
    out[:, p[ok]] = codes_nd[tok[ok]].T
    return out


def run_case(q, k, v, tau, sink_start=None, sink_tokens=0, heads=None, sample=None, seed=0):
    B, N, H, _ = q.shape
    say(f"[sol_attn2_pv8] B={B} N={N} H={H} tau={tau} sink=({sink_start},{sink_tokens})")
    qg, kg, vg = to_gpu(q, k, v)
    _, masks, _ = bsa.debug_routing(2, qg, kg, vg, tau, "diag", sink_start, sink_tokens)
    ws = bsa.alloc_workspace(bsa.SOL_VARIANT_SOL2_PV8, qg)
    out = bsa.sol_attn2_pv8(qg, kg, vg, tau, "diag", sink_start, sink_tokens, workspace=ws)
    torch.cuda.synchronize()
    views = bsa.workspace_views(bsa.SOL_VARIANT_SOL2_PV8, ws, B, N, H)
    nb = (N + 63) // 64
    # The FP8-PV exact pass routes on chip with the same prologue as the exported bf16-V
    # pass (no routing map is kept); a routing difference would show in the rows below,
    # which the oracle evaluates under the exported masks.
    gsel = masks.numpy()
    out_c = out.float().cpu().numpy()
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(128)
    got, want, want_bf16 = [], [], []
    worst_anchor = 0.0
    tp = views["v8t"].shape[-1]
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            qh, kh, vh = _head(q, b, h), _head(k, b, h), _head(v, b, h)
            vc, vs, vd = s2.quantize_head_v(vh)
            assert views["vscale"][b, h].item() == float(vs), "V scale differs"
            v8 = views["v8t"][b, h].cpu().numpy()
            assert np.array_equal(v8, _operand_order(vc, tp)), "V codes differ"
            r = s2.sol_attn2_head(qh, kh, vh, tau, sink_start, sink_tokens, query_blocks=[])
            blocks = range(nb) if sample is None else sorted(set(rng.choice(nb, size=min(sample, nb), replace=False)) | {nb - 1})
            for i in blocks:
                s, e = i * 64, min(i * 64 + 64, N)
                want.append(s2.attend_query_block2(r.q_deq, r.k_deq, vh, i, gsel[b, h, i], r.groups, scale,
                                                   pv="expcast", v_exact=vd))
                want_bf16.append(s2.attend_query_block2(r.q_deq, r.k_deq, vh, i, gsel[b, h, i], r.groups, scale))
                got.append(out_c[b, s:e, h, :])
                worst_anchor = max([worst_anchor] + anchor_errors(got[-1], want[-1]))
    got, want, want_bf16 = (np.concatenate(x) for x in (got, want, want_bf16))
    assert np.isfinite(got).all()
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    err_bf = np.linalg.norm(got - want_bf16) / np.linalg.norm(want_bf16)
    say(f"   ok: rel L2 {err:.2e} (vs bf16-PV oracle {err_bf:.2e}), max abs {np.abs(got - want).max():.2e}, "
        f"worst anchor rel L2 {worst_anchor:.2e}, density {gsel.mean():.3f}")
    assert err <= REL_L2_FP8, f"rel L2 {err:.3e} > {REL_L2_FP8}"
    assert worst_anchor <= REL_L2_FP8, f"an anchor's rel L2 {worst_anchor:.3e} > {REL_L2_FP8}"
    return out


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_tiny_workload_full(tau):
    q, k, v = _qkv(1, 1024, 2, 1000)
    run_case(q, k, v, tau)


@pytest.mark.parametrize("N", [40, 65, 1000, 4493])
def test_ragged_lengths(N):
    q, k, v = _qkv(1, N, 2, 3100 + N)
    run_case(q, k, v, 0.8)


@pytest.mark.parametrize("sink", [(0, 130), (0, 1000)])
def test_exact_sink(sink):
    q, k, v = _qkv(1, 1000, 2, 3200)
    run_case(q, k, v, 1.5, sink_start=sink[0], sink_tokens=sink[1])


def test_constant_values_with_everything_exact():
    """Every block exact and V rows all equal: the output is the per-head-quantized row
    (same decoded weights in numerator and denominator), up to the bf16 output rounding."""
    q, k, _ = _qkv(1, 700, 2, 3300)
    row = torch.randn(128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    v = row.view(1, 1, 1, 128).expand(1, 700, 2, 128).contiguous()
    out = run_case(q, k, v, 1.0, sink_start=0, sink_tokens=700)
    vd = s2.quantize_head_v(v[0, :, 0, :].double().numpy())[2][0]
    np.testing.assert_allclose(out[0, :, 0, :].float().cpu().numpy(), np.tile(vd, (700, 1)), rtol=8e-3, atol=1e-3)


def test_batch_and_odd_heads():
    q, k, v = _qkv(2, 700, 3, 3400)
    run_case(q, k, v, 0.5)


def test_sol2_bench_shape():
    """B=1, H=32, N=32768 near 90% sparsity: codes of 3 heads in full, sampled outputs."""
    q, k, v = sol2_bench().qkv()
    run_case(q, k, v, 1.28, heads=[0, 13, 31], sample=3, seed=7)


def test_maximum_sequence_length():
    """524288 tokens with the FP8 PV path (V codes in their operand order at the largest length)."""
    q, k, v = _qkv(1, 524288, 1, 2700)
    run_case(q, k, v, 1.28, sample=2, seed=8)
