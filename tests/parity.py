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
