"""GPU parity of the Sol-Attn2 backward (routing and key groups fixed) against the float64
oracle, through the C ABI.

The training forward must give the plain Sol-Attn2 output and store each row's
log-sum-exp; the backward's dq, dk, dv are compared with oracle.sol_attn2_bwd evaluated on
the oracle's dequantized q', k' (bit-identical to the kernel's, which the forward tests
check), under the routing and the group memberships the forward kernels made (read back
from the workspace), so that a mask bit or a group tie inside the fp32 / fp64 margin
cannot make the two sides differentiate different functions.

Bar, per gradient tensor: relative L2 <= 2e-2 and max-abs <= 5e-2 * max(1, max |ref|),
with the reference's L2 norm floored at an RMS of 1e-4.  The arithmetic behind it: the
exact products run on q', k' rounded to bf16 (relative 2^-9 per operand, where the forward
multiplied the E4M3 codes exactly, so the recomputed probabilities carry a relative error
of about |logit| 2^-8 against the forward's log-sum-exp); P and dS, and the anchors'
q-bar, dmu, dnu, enter the MFMAs rounded to bf16; sums are fp32; the gradients are
rounded once to bf16 -- the Sol-Attn backward's few 1e-3 plus the bf16 q', k'.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from oracle import sol_attn as sa
from oracle import sol_attn2 as s2
from oracle import sol_attn2_bwd as sb2
from parity import bwd_order_check, say, to_gpu
from workloads import block_offset_tensor, long_sink, operator_bench, wan_dit

pytestmark = pytest.mark.gpu

REL_L2 = 2e-2
MAX_ABS = 5e-2


def _qkv(B, N, H, seed, offset=1.0):
    return [block_offset_tensor(B, N, H, 128, seed + i, offset) for i in range(3)]


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _compare(name, got, want):
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-4 * np.sqrt(want.size))
    mx = np.abs(got - want).max()
    bound = MAX_ABS * max(1.0, np.abs(want).max())
    assert np.isfinite(got).all(), f"{name}: non-finite gradient"
    assert err <= REL_L2, f"{name}: rel L2 {err:.3e} > {REL_L2}"
    assert mx <= bound, f"{name}: max abs {mx:.3e} > {bound:.3e}"
    return err, mx


def _state(ws, B, N, H):
    """The routing masks [B, H, nb, nb] and the per-block group member masks the forward used."""
    views = bsa.workspace_views(bsa.SOL_VARIANT_SOL2_TRAIN, ws, B, N, H)
    nb = views["nb"]
    w = views["sel"].cpu()
    bits = torch.arange(64, dtype=torch.int64)
    sel = ((w.unsqueeze(-1) >> bits) & 1).bool().reshape(B, H, nb, -1)[..., :nb].numpy()
    ghi = views["ghi"].cpu().numpy().view(np.uint64)
    masks = []
    for b in range(B):
        mb = []
        for h in range(H):
            mh = []
            for j, (s, e) in enumerate(sa.block_ranges(N)):
                hi = ((ghi[b, h, j] >> np.arange(e - s, dtype=np.uint64)) & np.uint64(1)).astype(bool)
                mh.append([hi, ~hi])
            mb.append(mh)
        masks.append(mb)
    return sel, masks, views


def run_case(q, k, v, tau, sink_start=None, sink_tokens=0, heads=None, seed=0, thresh="diag"):
    B, N, H, _ = q.shape
    say(f"[backward2] B={B} N={N} H={H} tau={tau} sink=({sink_start},{sink_tokens})")
    do = _dout(q.shape, 8000 + seed)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    out, ws = bsa.forward_train2(qg, kg, vg, tau, thresh, sink_start, sink_tokens)
    dq, dk, dv = bsa.backward2(qg, kg, vg, out, dog, ws)
    plain = bsa.sol_attn2(qg, kg, vg, tau, thresh, sink_start, sink_tokens)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the training forward changed the output"
    gsel, gmasks, views = _state(ws, B, N, H)
    bwd_order_check(views, gsel)
    lse = views["lse"].cpu().numpy()
    errs = []
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            qh, kh, vh, dh = (x[b, :, h].double().numpy() for x in (q, k, v, do))
            qd = s2.quantize_head(qh)[2]
            kd = s2.quantize_head(kh)[2]
            _, lse_ref = sb2.forward_fixed(qd, kd, vh, gsel[b, h], gmasks[b][h])
            # the kernel's lse is base 2: ln -> log2
            np.testing.assert_allclose(lse[b, h, :N], lse_ref / np.log(2.0), rtol=0, atol=2e-2)
            want = sb2.backward_head2(qd, kd, vh, dh, gsel[b, h], gmasks[b][h])
            got = [x[b, :, h].float().cpu().numpy() for x in (dq, dk, dv)]
            errs.append([_compare(f"{n} b={b} h={h}", g_, w_) for n, g_, w_ in zip(("dq", "dk", "dv"), got, want)])
    e = np.array(errs)
    say(f"   ok: rel L2 dq/dk/dv max {e[:, 0, 0].max():.2e}/{e[:, 1, 0].max():.2e}/{e[:, 2, 0].max():.2e}, "
        f"density {gsel.mean():.3f}")
    return dq, dk, dv


@pytest.mark.parametrize("tau", [1.0, 0.0, 2.0])
def test_tiny_workload(tau):
    run_case(*_qkv(1, 1024, 2, 1000), tau)


@pytest.mark.parametrize("N", [1, 40, 64, 65, 200, 1000, 4493])
def test_ragged_lengths(N):
    run_case(*_qkv(1, N, 2, 2100 + N), 0.8, seed=N)


@pytest.mark.parametrize("sink", [(0, 130), (None, 70)])
def test_exact_sink(sink):
    run_case(*_qkv(1, 1000, 2, 2200), 1.5, *sink)


def test_batch_and_odd_heads():
    run_case(*_qkv(2, 700, 3, 2300), 0.5)


def test_exact_covariance_threshold():
    run_case(*_qkv(1, 2000, 2, 2350), 1.0, thresh="exact")


def test_everything_exact_is_the_dense_gradient():
    """A sink over the whole sequence makes every block exact and leaves no tail: the
    gradient is dense attention's w.r.t. the dequantized q', k' and v (torch SDPA autograd
    in float32 on the CPU), passed straight through to q, k."""
    B, N, H = 1, 700, 2
    q, k, v = _qkv(B, N, H, 2500)
    do = _dout(q.shape, 2501)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    out, ws = bsa.forward_train2(qg, kg, vg, 1.0, "diag", 0, N)
    dq, dk, dv = bsa.backward2(qg, kg, vg, out, dog, ws)
    torch.cuda.synchronize()
    qd = torch.stack([torch.from_numpy(s2.quantize_head(q[0, :, h].double().numpy())[2]) for h in range(H)], 1)[None]
    kd = torch.stack([torch.from_numpy(s2.quantize_head(k[0, :, h].double().numpy())[2]) for h in range(H)], 1)[None]
    tq, tk, tv = (x.float().transpose(1, 2).contiguous().requires_grad_(True) for x in (qd, kd, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    o.backward(do.float().transpose(1, 2).contiguous())
    for name, got, ref in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
        _compare(name, got.float().cpu().numpy(), ref.transpose(1, 2).numpy())


def test_autograd_function_matches_the_entry_points():
    q, k, v = _qkv(1, 1000, 2, 2600)
    do = _dout(q.shape, 2601)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    ql, kl, vl = (x.clone().requires_grad_(True) for x in (qg, kg, vg))
    o = bsa.sol_attn2_train(ql, kl, vl, 1.0)
    o.backward(dog)
    out, ws = bsa.forward_train2(qg, kg, vg, 1.0)
    dq, dk, dv = bsa.backward2(qg, kg, vg, out, dog, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), out)
    # no atomics anywhere in this backward: bit-identical
    assert torch.equal(ql.grad, dq) and torch.equal(kl.grad, dk) and torch.equal(vl.grad, dv)


def test_wan21_dit_shape():
    q, k, v = wan_dit().qkv()
    run_case(q, k, v, 1.0, heads=[0, 11])


def test_operator_bench_shape():
    """The 32K x 32-head shape: two heads compared in full."""
    q, k, v = operator_bench().qkv()
    run_case(q, k, v, 1.28, heads=[0, 31])


def test_long_sequence_with_text_sink():
    """512 text tokens (exact sink) + 65536 video tokens, 32 heads: one head compared in full."""
    q, k, v = long_sink(video_tokens=65536).qkv()
    run_case(q, k, v, 1.3, 0, 512, heads=[7])
