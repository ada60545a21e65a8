"""Shared helpers for the GPU parity tests (test infrastructure: imports the oracle)."""
import math
import sys

import numpy as np
import torch

from oracle import sol_attn as sa

MARGIN = 1e-3          # masks must agree wherever |s_hat - tau_i| > MARGIN (scaled-logit units)
REL_L2_BF16 = 1e-2
MAX_ABS_BF16 = 3e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(*ts):
    return [t.cuda() for t in ts]


def mask_check(gpu_sel: np.ndarray, ref_sel: np.ndarray, s_hat: np.ndarray, tau_i: np.ndarray, forced=None):
    """Masks are bit-exact outside the margin; returns the number of in-margin flips."""
    diff = gpu_sel != ref_sel
    near = np.abs(s_hat - tau_i[..., None]) <= MARGIN
    if forced is not None:
        near = near & ~forced
    bad = diff & ~near
    assert not bad.any(), f"{int(bad.sum())} mask bits differ outside the {MARGIN} margin"
    return int(diff.sum())


def pair_check(gpu_pairs: int, gpu_sel: np.ndarray, ref_sel: np.ndarray, n_tokens: int):
    """The kernel's selected-token-pair counter equals the oracle's count of its own masks
    (integer, exact), and the oracle's masks' count wherever the two mask sets agree."""
    want = sa.selected_pairs(gpu_sel, n_tokens)
    assert gpu_pairs == want, f"selected pairs {gpu_pairs} != {want} counted from the kernel's masks"
    if np.array_equal(gpu_sel, ref_sel):
        assert gpu_pairs == sa.selected_pairs(ref_sel, n_tokens)


def anchor_errors(got: np.ndarray, want: np.ndarray, anchor: int = 32) -> list:
    """Relative L2 error of each 32-row anchor of one query block's rows (rows [0, 32) and
    [32, n)); an anchor whose reference is zero is skipped."""
    errs = []
    for a0 in range(0, want.shape[0], anchor):
        w = np.asarray(want[a0:a0 + anchor], dtype=np.float64)
        g = np.asarray(got[a0:a0 + anchor], dtype=np.float64)
        nw = np.linalg.norm(w)
        if nw > 0:
            errs.append(float(np.linalg.norm(g - w) / nw))
    return errs


def oracle_rows(q, k, v, b, h, i, sel_row):
    """Oracle output rows of query block i for (b, h) under a given selection row."""
    qh = q[b, :, h, :].to(torch.float64).numpy()
    kh = k[b, :, h, :].to(torch.float64).numpy()
    vh = v[b, :, h, :].to(torch.float64).numpy()
    n, d = qh.shape
    kbar, vsum, counts = sa.block_means(kh), sa.block_sums(vh), sa.block_counts(n)
    return sa.attend_query_block(qh, kh, vh, i, sel_row, kbar, vsum, counts, 1 / math.sqrt(d))


def compare_out(gpu: np.ndarray, ref: np.ndarray, rel=REL_L2_BF16, max_abs=MAX_ABS_BF16, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    err = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(gpu - ref).max()
    assert err <= rel, f"{what}: rel L2 {err:.3e} > {rel}"
    assert mx <= max_abs, f"{what}: max abs {mx:.3e} > {max_abs}"
    return err, mx


def order_check(variant, ws, gsel, B, N, H, kv_splits=0):
    """Sol-Attn stage 2's work order: qcount is each query block's number of exact blocks
    within each key split, counted by the same decision procedure as the fused pass, so over
    the splits it sums to the row sums of the masks that pass exported, exactly; each (head,
    split)'s order lists the blocks by descending count (equal counts in any order) and is a
    permutation, so every block is computed once per split."""
    import block_sparse_attention_tok_amd as bsa
    from block_sparse_attention_tok_amd import _lib
    L = _lib.workspace_layout(variant, B, N, H, kv_splits=kv_splits) if kv_splits else None
    views = bsa.workspace_views(variant, ws, B, N, H) if L is None else None
    if views is None:
        nbp, S = L.nbp, L.kv_splits
        qc_t = ws[L.qcount:L.qcount + B * H * S * nbp * 4].view(torch.int32).view(B, H, S, nbp)
        or_t = ws[L.order:L.order + B * H * S * nbp * 4].view(torch.int32).view(B, H, S, nbp)
        nb = L.nb
    else:
        qc_t, or_t, nb = views["qcount"], views["order"], views["nb"]
    qcount = qc_t.cpu().numpy()[..., :nb]
    order = or_t.cpu().numpy()[..., :nb]
    np.testing.assert_array_equal(qcount.sum(2), gsel.sum(-1))
    for b in range(B):
        for h in range(H):
            for sp in range(qcount.shape[2]):
                np.testing.assert_array_equal(np.sort(order[b, h, sp]), np.arange(nb))
                c = qcount[b, h, sp][order[b, h, sp]]
                assert (np.diff(c) <= 0).all(), "order is not by descending count"


def bwd_order_check(views, gsel):
    """The backward's work orders: bqord lists each head's query blocks by descending number
    of exact key blocks (row sums of the forward's masks), bkord its key blocks by descending
    number of query blocks that select them (column sums); both are permutations, so every
    query block's dQ and every key block's dK / dV is computed once."""
    B, H, nb, _ = gsel.shape
    rows, cols = gsel.sum(-1), gsel.sum(-2)
    for name, cnt in (("bqord", rows), ("bkord", cols)):
        order = views[name].cpu().numpy()[..., :nb]
        for b in range(B):
            for h in range(H):
                np.testing.assert_array_equal(np.sort(order[b, h]), np.arange(nb), err_msg=name)
                assert (np.diff(cnt[b, h][order[b, h]]) <= 0).all(), f"{name} is not by descending count"
