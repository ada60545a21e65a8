"""C-ABI boundary tests that need no GPU: the library loads, exports every symbol the
header declares, and the host-side validator / workspace sizing behave as documented."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "solattn.h")


@pytest.fixture(scope="module")
def L():
    from block_sparse_attention_tok_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libsolattn.so not built")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(sol_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("sol_attn", "sol_attn2", "sol_attn_validate", "sol_attn_workspace_bytes", "sol_status_string",
              "sol_attn_prepare", "sol_attn_fused", "sol_attn_debug_routing"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    from block_sparse_attention_tok_amd import _lib
    assert sorted(_lib.EXPORTED) == declared_functions()


def test_status_strings(L):
    for s in range(0, 10):
        assert L.sol_status_string(s)
    assert L.sol_status_string(123) == b"unknown status"


@pytest.mark.parametrize("args,status", [
    ((1, 1024, 2, 128, 1.0, -1, 0, 0), 0),
    ((1, 1024, 2, 128, 0.0, 0, 1024, 1), 0),
    ((1, 1024, 2, 64, 1.0, -1, 0, 0), 3),
    ((0, 1024, 2, 128, 1.0, -1, 0, 0), 2),
    ((1, 0, 2, 128, 1.0, -1, 0, 0), 2),
    ((1, 1024, 0, 128, 1.0, -1, 0, 0), 2),
    ((1, 1024, 2, 128, math.nan, -1, 0, 0), 4),
    ((1, 1024, 2, 128, math.inf, -1, 0, 0), 4),
    ((1, 1024, 2, 128, -math.inf, -1, 0, 0), 4),
    ((1, 1024, 2, 128, 1.0, 1000, 100, 0), 5),
    ((1, 1024, 2, 128, 1.0, 0, -1, 0), 5),
    ((1, 1024, 2, 128, 1.0, -1, 1025, 0), 5),
    ((1, 1024, 2, 128, 1.0, -1, 1024, 0), 0),
    ((1, 1024, 2, 128, 1.0, -1, 0, 7), 8),
])
def test_validate(L, args, status):
    assert L.sol_attn_validate(*args) == status


def test_workspace_sizes_and_layout(L):
    from block_sparse_attention_tok_amd import _lib
    for variant in (1, 2, 4, 5):
        for (B, N, H) in ((1, 1024, 2), (1, 14040, 12), (2, 333, 3), (1, 32768, 32)):
            n = L.sol_attn_workspace_bytes(variant, B, N, H, 128)
            lay = _lib.workspace_layout(variant, B, N, H)
            assert n == lay.total_bytes > 0
            nb = (N + 63) // 64
            assert lay.nb == nb and lay.nbp % 64 == 0 and lay.nbp >= nb
            offs = sorted(o for name, _ in _lib.WsLayout._fields_
                          if name not in ("total_bytes", "nb", "nbp", "kv_splits")
                          for o in [getattr(lay, name)] if o >= 0)
            assert all(o % 256 == 0 for o in offs)
            assert offs[-1] < n
            # every fused kernel routes on chip: only the Sol-Attn2 training layout keeps the
            # forward's routing words (for its backward)
            assert (lay.sel >= 0) == (variant == 5)
            if variant in (1, 4):
                assert lay.q8 == -1 and lay.gk == -1
    assert L.sol_attn_workspace_bytes(1, 1, 1024, 2, 64) == 0
    assert L.sol_attn_workspace_bytes(6, 1, 1024, 2, 128) == 0


@pytest.mark.parametrize("B,N,H", [(1, 1024, 2), (1, 14040, 12), (2, 333, 3)])
def test_fp8_pv_layout_extends_the_sol2_layout(L, B, N, H):
    """The FP8-PV workspace is the Sol-Attn2 one with v8t / vbmax / vscale appended, so the
    shared Sol-Attn2 stage calls (tail pass) run on it unchanged."""
    from block_sparse_attention_tok_amd import _lib
    l2 = _lib.workspace_layout(2, B, N, H)
    l3 = _lib.workspace_layout(3, B, N, H)
    for name, _ in _lib.WsLayout._fields_:
        if name in ("total_bytes", "v8t", "vbmax", "vscale"):
            continue
        assert getattr(l2, name) == getattr(l3, name), name
    assert l2.v8t == l2.vbmax == l2.vscale == -1
    assert l3.v8t >= l2.total_bytes and l3.total_bytes > l3.vscale > l3.vbmax > l3.v8t
    assert l3.vbmax - l3.v8t >= B * H * 128 * l3.nbp * 64


@pytest.mark.parametrize("B,N,H", [(1, 1024, 2), (1, 14040, 12), (2, 333, 3), (1, 32768, 32)])
def test_training_layout_extends_the_sol_attn_layout(L, B, N, H):
    """The training workspace is the Sol-Attn one (split partials included) with the forward
    state and backward scratch appended, so the Sol-Attn stage calls run on it unchanged."""
    from block_sparse_attention_tok_amd import _lib
    l1 = _lib.workspace_layout(1, B, N, H)
    l4 = _lib.workspace_layout(4, B, N, H)
    extra = ("lse", "mrow", "mcol", "ld", "dkbar", "dvbar", "bqord", "bkord")
    for name, _ in _lib.WsLayout._fields_:
        if name in ("total_bytes",) + extra:
            continue
        assert getattr(l1, name) == getattr(l4, name), name
    assert all(getattr(l1, n) == -1 for n in extra)
    offs = [getattr(l4, n) for n in extra]
    assert offs == sorted(offs) and offs[0] >= l1.total_bytes and l4.total_bytes > offs[-1]
    tp = l4.nbp * 64
    nbw = l4.nbp // 64
    assert l4.mrow - l4.lse >= B * H * tp * 4
    assert l4.mcol - l4.mrow >= B * H * l4.nb * nbw * 8
    assert l4.dvbar - l4.dkbar >= B * H * l4.nbp * 128 * 4
    assert l4.bqord - l4.dvbar >= B * H * l4.nbp * 128 * 4
    assert l4.bkord - l4.bqord >= B * H * l4.nbp * 4 and l4.total_bytes - l4.bkord >= B * H * l4.nbp * 4


@pytest.mark.parametrize("B,N,H", [(1, 1024, 2), (1, 14040, 12), (2, 333, 3), (1, 32768, 32)])
def test_work_order_arrays(L, B, N, H):
    """Sol-Attn's stage-2 work order (per-chunk counts, per-block counts, the order itself) has
    its documented sizes in both Sol-Attn layouts and exists in no Sol-Attn2 layout."""
    from block_sparse_attention_tok_amd import _lib
    for variant in (1, 4):
        l = _lib.workspace_layout(variant, B, N, H)
        bh, nbp, S = B * H, l.nbp, l.kv_splits
        assert l.wcnt >= 0 and l.qcount - l.wcnt >= bh * (nbp // 64) * nbp
        assert l.order - l.qcount >= bh * S * nbp * 4 and l.total_bytes - l.order >= bh * S * nbp * 4
        assert l.wcnt % 256 == 0 and l.qcount % 256 == 0 and l.order % 256 == 0
    for variant in (2, 3, 5):
        l = _lib.workspace_layout(variant, B, N, H)
        assert l.wcnt == l.qcount == l.order == -1


@pytest.mark.parametrize("B,N,H", [(1, 1024, 2), (1, 14040, 12), (2, 333, 3), (1, 32768, 32)])
def test_sol2_training_layout_extends_the_sol2_layout(L, B, N, H):
    """The Sol-Attn2 training workspace is the Sol-Attn2 one with the forward's row
    log-sum-exp and the backward scratch appended (so every Sol-Attn2 stage call runs on it
    unchanged), each array large enough for its documented shape."""
    from block_sparse_attention_tok_amd import _lib
    l2 = _lib.workspace_layout(2, B, N, H)
    l5 = _lib.workspace_layout(5, B, N, H)
    extra = ("sel", "lse", "ofp", "mcol", "ld", "kh", "vh", "qd", "kd", "dlam", "qab", "dmub", "dnub", "alz",
             "aextra", "gdk", "gdv", "bqord", "bkord")
    for name, _ in _lib.WsLayout._fields_:
        if name in ("total_bytes",) + extra:
            continue
        assert getattr(l2, name) == getattr(l5, name), name
    assert all(getattr(l2, n) == -1 for n in extra)
    assert l5.mrow == l5.dkbar == l5.dvbar == l5.v8t == -1
    assert all(getattr(l1, n) == -1 for l1 in (_lib.workspace_layout(1, B, N, H),) for n in ("ofp", "qd", "gdk"))
    offs = [getattr(l5, n) for n in extra] + [l5.total_bytes]
    assert offs == sorted(offs) and offs[0] >= l2.total_bytes
    bh, nbp, nb = B * H, l5.nbp, l5.nb
    tp = nbp * 64
    need = dict(sel=bh * nb * (nbp // 64) * 8, lse=bh * tp * 4, ofp=bh * tp * 512, mcol=bh * nb * (nbp // 64) * 8, ld=bh * tp * 8, kh=bh * N * 256, vh=bh * N * 256,
                qd=bh * N * 256, kd=bh * N * 256, dlam=bh * tp * 4, qab=bh * 2 * nbp * 256,
                dmub=bh * 2 * nbp * 256, dnub=bh * 2 * nbp * 256, alz=bh * 2 * nbp * 8, aextra=bh * 2 * nbp * 512,
                gdk=bh * 2 * nbp * 512, gdv=bh * 2 * nbp * 512, bqord=bh * nbp * 4, bkord=bh * nbp * 4)
    for a, b in zip(extra, offs[1:]):
        assert b - getattr(l5, a) >= need[a], a


@pytest.mark.parametrize("tokens,req,expect", [
    (1024, 0, 1), (8192, 0, 1), (8193, 0, 1), (14040, 0, 1), (16385, 0, 1), (24577, 0, 1), (32768, 0, 1),
    (32769, 0, 2), (49152, 0, 2), (65536, 0, 3), (66048, 0, 3), (98304, 0, 4), (131072, 0, 4), (131584, 0, 4),
    (524288, 0, 4),
    (32768, 1, 1), (32768, 2, 2), (32768, 3, 3), (32768, 8, 8), (32768, 16, 8), (1024, 4, 1), (131584, 16, 11),
])
def test_kv_split_rule(L, tokens, req, expect):
    """Splits cover whole 64-block routing chunks; automatic = none up to 8 chunks, then one
    split per six chunks (rounded up), at most 4."""
    assert L.sol_attn_kv_splits(1, tokens, 32, req) == expect
    lay = __import__("block_sparse_attention_tok_amd")._lib.workspace_layout(1, 1, tokens, 32, kv_splits=req)
    assert lay.kv_splits == expect
    assert (lay.opart >= 0) == (expect > 1)
    assert L.sol_attn_kv_splits(1, tokens, 32, 17) == 0       # out of range


def test_shape_limits(L):
    assert L.sol_attn_validate(1, 524288, 32, 128, 1.0, -1, 0, 0) == 0
    assert L.sol_attn_validate(1, 524289, 1, 128, 1.0, -1, 0, 0) == 2
    assert L.sol_attn_validate(1, 524288, 64, 128, 1.0, -1, 0, 0) == 2      # a head's rows exceed 4 GiB
    # H = 48: 349526 rows fit 4 GiB, but padded to 349568 (whole 64-row blocks) they do not
    assert L.sol_attn_validate(1, 349526, 48, 128, 1.0, -1, 0, 0) == 2
    assert L.sol_attn_validate(1, 349504, 48, 128, 1.0, -1, 0, 0) == 0


def test_entry_points_reject_bad_arguments_before_any_launch(L):
    """Argument errors return a status without touching the device (NULL and fake pointers)."""
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    # null inputs
    assert L.sol_attn(None, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, 1 << 30, None) == 1
    # non-finite tau
    assert L.sol_attn(fake, fake, fake, fake, 1, 1024, 2, 128, float("nan"), -1, 0, 0, fake, 1 << 30, None) == 4
    # head dim
    assert L.sol_attn(fake, fake, fake, fake, 1, 1024, 2, 64, 1.0, -1, 0, 0, fake, 1 << 30, None) == 3
    # sink out of range
    assert L.sol_attn2(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, 1000, 100, 0, fake, 1 << 30, None) == 5
    # workspace too small
    assert L.sol_attn(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, 16, None) == 6
    # misaligned workspace
    assert L.sol_attn(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 0, vp(0x1010), 1 << 30, None) == 8
    # unknown threshold type
    assert L.sol_attn(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 9, fake, 1 << 30, None) == 8
    # missing mask buffer for the debug export (the selected-pair counter is optional: a NULL
    # counter is not an error, so the non-finite tau is what gets reported)
    assert L.sol_attn_debug_routing(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, 0, fake, 1 << 30,
                                    None, fake, None) == 1
    assert L.sol_attn_debug_routing(fake, fake, fake, None, 1, 1024, 2, 128, float("nan"), -1, 0, 0, 0, fake,
                                    1 << 30, fake, None, None) == 4
    assert L.sol_attn2_debug_routing(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, 0, fake, 1 << 30,
                                     None, None, None) == 1
    assert L.sol_attn2_debug_routing(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, 2, fake, 1 << 30,
                                     fake, None, None) == 8
    # kv_splits out of range
    assert L.sol_attn_fused_kv(fake, fake, fake, fake, 1, 1024, 2, 128, -1, 0, 17, fake, 1 << 30, None) == 8
    # Sol-Attn2 stage 2 parts: sink out of range, missing output, workspace too small
    assert L.sol_attn2_tail(fake, fake, fake, 1, 1024, 2, 128, 1000, 100, fake, 1 << 30, None) == 5
    assert L.sol_attn2_exact(fake, fake, fake, None, 1, 1024, 2, 128, -1, 0, fake, 1 << 30, None) == 1
    assert L.sol_attn2_exact(fake, fake, fake, fake, 1, 1024, 2, 128, -1, 0, fake, 16, None) == 6
    assert L.sol_attn2_exact(fake, fake, fake, fake, 1, 1024, 2, 128, 1000, 100, fake, 1 << 30, None) == 5
    assert L.sol_attn2_pv8_exact(fake, fake, fake, fake, 1, 1024, 2, 128, 0, -3, fake, 1 << 30, None) == 5
    # training forward / backward: missing output or gradient, workspace sized for the plain forward,
    # misaligned gradient
    assert L.sol_attn_forward_train(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, 1 << 30, None) == 1
    small = L.sol_attn_workspace_bytes(1, 1, 1024, 2, 128)
    assert L.sol_attn_forward_train(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, small, None) == 6
    assert L.sol_attn_backward(fake, fake, fake, fake, None, fake, fake, fake, 1, 1024, 2, 128, fake, 1 << 30,
                               None) == 1
    assert L.sol_attn_backward(fake, fake, fake, fake, fake, fake, fake, fake, 1, 1024, 2, 128, fake, small,
                               None) == 6
    assert L.sol_attn_backward(fake, fake, fake, fake, fake, vp(0x1008), fake, fake, 1, 1024, 2, 128, fake,
                               1 << 30, None) == 8
    assert L.sol_attn_backward(fake, fake, fake, fake, fake, fake, fake, fake, 1, 1024, 2, 64, fake, 1 << 30,
                               None) == 3
    # Sol-Attn2 training: a workspace sized for the plain Sol-Attn2 forward is too small
    small2 = L.sol_attn_workspace_bytes(2, 1, 1024, 2, 128)
    assert L.sol_attn2_forward_train(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, 1 << 30,
                                     None) == 1
    assert L.sol_attn2_forward_train(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, -1, 0, 0, fake, small2,
                                     None) == 6
    assert L.sol_attn2_forward_train(fake, fake, fake, fake, 1, 1024, 2, 128, float("inf"), -1, 0, 0, fake,
                                     1 << 30, None) == 4
    assert L.sol_attn2_backward(fake, fake, fake, fake, fake, fake, None, fake, 1, 1024, 2, 128, fake, 1 << 30,
                                None) == 1
    assert L.sol_attn2_backward(fake, fake, fake, fake, fake, fake, fake, fake, 1, 1024, 2, 128, fake, small2,
                                None) == 6
    assert L.sol_attn2_backward(fake, fake, fake, fake, fake, fake, fake, vp(0x1004), 1, 1024, 2, 128, fake,
                                1 << 30, None) == 8


def test_python_validate_wrapper():
    from block_sparse_attention_tok_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libsolattn.so not built")
    assert _lib.validate(1, 1024, 2, 128, 1.0, None, 0) == 0
    assert _lib.validate(1, 1024, 2, 128, 1.0, None, 2000) == 5
    assert _lib.validate(1, 1024, 2, 128, 1.0, None, 0, "bogus") == 8


def test_binding_rejects_bad_outputs_and_workspaces():
    """The binding checks caller-supplied outputs and workspaces before any pointer reaches the
    library: wrong dtype, shape, layout or device for out / dq / dk / dv, a workspace of the
    wrong type or device (host-side checks; no GPU needed)."""
    import torch
    from block_sparse_attention_tok_amd import _lib
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    _lib._check_like(None, q, "out")
    _lib._check_like(torch.empty_like(q), q, "out")
    for bad in (q.float(), q[:, :32].contiguous(), q.transpose(1, 2), torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16),
                torch.empty(64 * 2 * 128, dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            _lib._check_like(bad, q, "out")
    with pytest.raises(ValueError):
        _lib._check_like(torch.empty(1, 64, 2, 128, dtype=torch.bfloat16, device="meta"), q, "dq")
    _lib._check_workspace(torch.empty(4096, dtype=torch.uint8), q)
    with pytest.raises(ValueError):
        _lib._check_workspace(torch.empty(1024, dtype=torch.float32), q)
    with pytest.raises(ValueError):
        _lib._check_workspace(torch.empty(4096, dtype=torch.uint8, device="meta"), q)
    with pytest.raises(ValueError):
        _lib._check_workspace(torch.empty(2, 4096, dtype=torch.uint8)[:, :100], q)


def test_noalloc_rejects_shapes_beyond_its_scratch_before_any_launch(L):
    """sol_attn_noalloc checks the shape's workspace against its static scratch on the host:
    a shape that does not fit returns SOL_ERR_SCRATCH (no device is touched), argument errors
    come first, and the scratch size in the header is the one the binding states."""
    from block_sparse_attention_tok_amd import _lib
    fake = ctypes.c_void_p(0x1000)
    text = open(HEADER).read()
    assert re.search(r"#define SOL_NOALLOC_SCRATCH_BYTES \(128u << 20\)", text)
    assert _lib.NOALLOC_SCRATCH_BYTES == 128 << 20
    # 1 x 32768 x 32 needs ~1059 MiB of workspace: rejected
    assert L.sol_attn_workspace_bytes(1, 1, 32768, 32, 128) > _lib.NOALLOC_SCRATCH_BYTES
    assert L.sol_attn_noalloc(fake, fake, fake, fake, 1, 32768, 32, 128, 1.0, -1, 0, 0, None) == 9
    assert b"scratch" in L.sol_status_string(9)
    # argument errors are reported before the size check
    assert L.sol_attn_noalloc(fake, fake, fake, None, 1, 1024, 2, 128, 1.0, -1, 0, 0, None) == 1
    assert L.sol_attn_noalloc(fake, fake, fake, fake, 1, 1024, 2, 128, float("nan"), -1, 0, 0, None) == 4
    assert L.sol_attn_noalloc(fake, fake, fake, fake, 1, 1024, 2, 64, 1.0, -1, 0, 0, None) == 3
    assert L.sol_attn_noalloc(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0, 1000, 100, 0, None) == 5
    # the Wan-2.1-shaped call (B=1, H=12, 14040 tokens) fits
    assert L.sol_attn_workspace_bytes(1, 1, 14040, 12, 128) <= _lib.NOALLOC_SCRATCH_BYTES
