"""GPU test of sol_attn_noalloc (the entry point that allocates nothing): through the C ABI,
its output equals sol_attn's with a caller workspace on the same inputs, for two calls in a
row on the shared static scratch, the second with a smaller input."""
import numpy as np
import pytest
import torch

import block_sparse_attention_tok_amd as bsa
from parity import compare_out, say
from workloads import block_offset_tensor

pytestmark = pytest.mark.gpu


def test_noalloc_matches_sol_attn_on_two_calls_in_a_row():
    cases = [(1, 4093, 4, 0.9, None, 0, 5100), (1, 1000, 2, 1.2, 0, 130, 5200)]
    for B, N, H, tau, s0, st, seed in cases:
        say(f"[noalloc] B={B} N={N} H={H} tau={tau} sink=({s0},{st})")
        q, k, v = (block_offset_tensor(B, N, H, 128, seed + i).cuda() for i in range(3))
        ref = bsa.sol_attn(q, k, v, tau, "diag", s0, st)
        out = torch.full_like(q, float("nan"))
        got = bsa.sol_attn_noalloc(q, k, v, out, tau, "diag", s0, st)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        err, mx = compare_out(got.float().cpu().numpy(), ref.float().cpu().numpy(), what=f"noalloc N={N}")
        # the same kernels on the same inputs: identical bits
        assert torch.equal(got, ref), f"noalloc differs from sol_attn in {int((got != ref).sum())} elements"
        say(f"   ok: identical to sol_attn (rel L2 {err:.1e})")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    q = torch.zeros(1, 32768, 32, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.SolAttnError) as e:
        bsa.sol_attn_noalloc(q, q, q, torch.empty_like(q))
    assert e.value.status == bsa._lib.SOL_ERR_SCRATCH
