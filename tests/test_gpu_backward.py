"""GPU parity of the Sol-Attn backward (fixed routing) against the float64 oracle, through the C ABI.

The training forward must give the plain forward's output and routing, and store each
row's log-sum-exp; the backward's dq, dk, dv are compared with oracle.sol_attn_bwd
evaluated under the routing the forward kernel made (read back from the workspace).
Bar, per gradient tensor: relative L2 <= 1e-2 and max-abs <= 3e-2 * max(1, max |ref|); the
L2 norm of the reference is floored at an RMS of 1e-4, since some gradients vanish in the
method itself (dq of a query whose every key is one pooled block: dS = P (dP - D) = 0).
The arithmetic behind it: bf16 inputs are exact, P and dS enter the MFMAs rounded to
bf16 (relative 2^-9 each), D uses the bf16 forward output, sums are fp32 and the
gradients are rounded once to bf16 -- a few 1e-3 relative, as in the forward.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from oracle import sol_attn as sa
from oracle import sol_attn_bwd as sb
from parity import bwd_order_check, mask_check, say, to_gpu
from workloads import block_offset_tensor, long_sink, operator_bench, wan_dit

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS = 3e-2


def _qkv(B, N, H, seed, offset=1.0):
    return [block_offset_tensor(B, N, H, 128, seed + i, offset) for i in range(3)]


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _routing_from_workspace(ws, B, N, H):
    views = bsa.workspace_views(bsa.SOL_VARIANT_SOL1_TRAIN, ws, B, N, H)
    nb = views["nb"]
    w = views["mrow"].cpu()
    bits = torch.arange(64, dtype=torch.int64)
    return ((w.unsqueeze(-1) >> bits) & 1).bool().reshape(B, H, nb, -1)[..., :nb].numpy(), views


def _compare(name, got, want):
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-4 * np.sqrt(want.size))
    mx = np.abs(got - want).max()
    bound = MAX_ABS * max(1.0, np.abs(want).max())
    assert err <= REL_L2, f"{name}: rel L2 {err:.3e} > {REL_L2}"
    assert mx <= bound, f"{name}: max abs {mx:.3e} > {bound:.3e}"
    return err, mx


def run_case(q, k, v, tau, sink_start=None, sink_tokens=0, heads=None, seed=0):
    B, N, H, _ = q.shape
    say(f"[backward] B={B} N={N} H={H} tau={tau} sink=({sink_start},{sink_tokens})")
    do = _dout(q.shape, 7000 + seed)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    out, ws = bsa.forward_train(qg, kg, vg, tau, "diag", sink_start, sink_tokens)
    dq, dk, dv = bsa.backward(qg, kg, vg, out, dog, ws)
    plain = bsa.sol_attn(qg, kg, vg, tau, "diag", sink_start, sink_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the training forward changed the output"
    gsel, views = _routing_from_workspace(ws, B, N, H)
    ref = sa.routing_only(q, k, tau, sink_start, sink_tokens)
    nb = (N + 63) // 64
    forced = np.zeros((B, H, nb, nb), dtype=bool)
    forced[..., sa.sink_block_mask(N, sink_start, sink_tokens)] = True
    mask_check(gsel, ref["sel"], ref["s_hat"], ref["tau_i"], forced)
    bwd_order_check(views, gsel)
    lse = views["lse"].cpu().numpy()
    errs = []
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            qh, kh, vh, dh = (x[b, :, h].double().numpy() for x in (q, k, v, do))
            _, lse_ref = sb.forward_with_lse(qh, kh, vh, gsel[b, h])
            # the kernel's lse is base 2 in units of log2(e) q.k/sqrt(d): ln -> log2
            np.testing.assert_allclose(lse[b, h, :N], lse_ref / np.log(2.0), rtol=0, atol=2e-2)
            want = sb.backward_head(qh, kh, vh, dh, gsel[b, h])
            got = [x[b, :, h].float().cpu().numpy() for x in (dq, dk, dv)]
            errs.append([_compare(f"{n} b={b} h={h}", g_, w_) for n, g_, w_ in zip(("dq", "dk", "dv"), got, want)])
    e = np.array(errs)
    say(f"   ok: rel L2 dq/dk/dv max {e[:, 0, 0].max():.2e}/{e[:, 1, 0].max():.2e}/{e[:, 2, 0].max():.2e}, "
        f"density {gsel.mean():.3f}")
    return dq, dk, dv


@pytest.mark.parametrize("tau", [1.0, 0.0, 2.5])
def test_tiny_workload(tau):
    run_case(*_qkv(1, 1024, 2, 1000), tau)


@pytest.mark.parametrize("N", [1, 40, 64, 65, 200, 1000, 4493])
def test_ragged_lengths(N):
    run_case(*_qkv(1, N, 2, 1100 + N), 1.0, seed=N)


@pytest.mark.parametrize("sink", [(0, 130), (None, 70), (0, 1)])
def test_exact_sink(sink):
    run_case(*_qkv(1, 1000, 2, 1200), 1.0, *sink)


def test_batch_and_odd_heads():
    run_case(*_qkv(2, 333, 3, 1300), 0.5)


def test_everything_exact_is_the_sdpa_gradient():
    """A sink over the whole sequence makes every block exact: the gradient is dense
    attention's (torch SDPA autograd in float32 on the CPU)."""
    B, N, H = 1, 700, 2
    q, k, v = _qkv(B, N, H, 1400)
    do = _dout(q.shape, 1401)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    out, ws = bsa.forward_train(qg, kg, vg, 1.0, "diag", 0, N)
    dq, dk, dv = bsa.backward(qg, kg, vg, out, dog, ws)
    torch.cuda.synchronize()
    tq, tk, tv = (x.float().transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    o.backward(do.float().transpose(1, 2).contiguous())
    for name, got, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
        _compare(name, got.float().cpu().numpy(), ref.transpose(1, 2).numpy())


def test_autograd_function_matches_the_entry_points():
    q, k, v = _qkv(1, 1000, 2, 1500)
    do = _dout(q.shape, 1501)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    ql, kl, vl = (x.clone().requires_grad_(True) for x in (qg, kg, vg))
    o = bsa.sol_attn_train(ql, kl, vl, 1.0)
    o.backward(dog)
    out, ws = bsa.forward_train(qg, kg, vg, 1.0)
    dq, dk, dv = bsa.backward(qg, kg, vg, out, dog, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), out)
    assert torch.equal(ql.grad, dq)
    # the pooled-key gradients are summed with fp32 atomics: dk / dv may differ in the last bits
    for a, b in ((kl.grad, dk), (vl.grad, dv)):
        assert (a.float() - b.float()).abs().max().item() <= 1e-2 * max(1.0, b.float().abs().max().item())


def test_wan21_dit_shape():
    wl = wan_dit()
    q, k, v = wl.qkv()
    run_case(q, k, v, 1.0, heads=[0, 11])


def test_operator_bench_shape():
    """The 32K x 32-head shape at 90% sparsity (tau 1.28): two heads compared in full."""
    wl = operator_bench()
    q, k, v = wl.qkv()
    run_case(q, k, v, 1.28, heads=[0, 31])


def test_long_sequence_with_text_sink():
    wl = long_sink(video_tokens=65536)
    q, k, v = wl.qkv()
    run_case(q, k, v, 1.3, 0, 512, heads=[5])
