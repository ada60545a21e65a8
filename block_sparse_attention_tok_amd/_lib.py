"""ctypes binding of libsolattn (argument marshalling only).

Every step of the Sol-Attn path runs in the library's HIP kernels; this module
only turns torch tensors into device pointers, allocates the caller-owned
workspace with torch, and raises on a non-OK status.  It never falls back to
another implementation: if the shared library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsolattn.so")

SOL_OK = 0
SOL_VARIANT_SOL1 = 1
SOL_VARIANT_SOL2 = 2
SOL_VARIANT_SOL2_PV8 = 3
SOL_VARIANT_SOL1_TRAIN = 4
SOL_VARIANT_SOL2_TRAIN = 5
THRESH = {"diag": 0, "exact": 1}

EXPORTED = [
    "sol_status_string", "sol_attn_validate", "sol_attn_workspace_bytes", "sol_attn_workspace_layout",
    "sol_attn_kv_splits", "sol_attn_workspace_bytes_kv", "sol_attn_workspace_layout_kv",
    "sol_attn", "sol_attn_prepare", "sol_attn_fused", "sol_attn_fused_kv", "sol_attn_debug_routing",
    "sol_attn2", "sol_attn2_prepare", "sol_attn2_fused", "sol_attn2_tail", "sol_attn2_exact",
    "sol_attn2_debug_routing", "sol_attn2_pv8", "sol_attn2_pv8_prepare", "sol_attn2_pv8_exact",
    "sol_attn_forward_train", "sol_attn_backward", "sol_attn_noalloc", "sol_attn2_forward_train",
    "sol_attn2_backward",
]
SOL_ERR_SCRATCH = 9
NOALLOC_SCRATCH_BYTES = 128 << 20


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "total_bytes", "nb", "nbp", "qbar", "kbar_t", "kbar_h", "vbar_h", "tau_i", "kstat", "kcov", "kpart",
        "q8", "k8", "qscale", "kscale", "qhat", "gk", "gv", "glogn", "ghi", "qanc", "kv_splits", "opart", "olse",
        "sel", "tmu", "tnu", "tlz", "v8t", "vbmax", "vscale", "lse", "mrow", "mcol", "ld", "dkbar", "dvbar",
        "kh", "vh", "qd", "kd", "dlam", "qab", "dmub", "dnub", "alz", "aextra", "gdk", "gdv", "ofp", "kcovp",
        "wcnt", "qcount", "order", "bqord", "bkord")]


class SolAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib().sol_status_string(status).decode()} (status {status})")
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libsolattn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m block_sparse_attention_tok_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, f32, i32, vp, sz = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.sol_status_string.argtypes = [i32]
    L.sol_status_string.restype = ctypes.c_char_p
    L.sol_attn_validate.argtypes = [i64, i64, i64, i64, f32, i64, i64, i32]
    L.sol_attn_validate.restype = i32
    L.sol_attn_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
    L.sol_attn_workspace_bytes.restype = sz
    L.sol_attn_workspace_layout.argtypes = [i32, i64, i64, i64, i64, ctypes.POINTER(WsLayout)]
    L.sol_attn_workspace_layout.restype = i32
    L.sol_attn_kv_splits.argtypes = [i64, i64, i64, i32]
    L.sol_attn_kv_splits.restype = i32
    L.sol_attn_workspace_bytes_kv.argtypes = [i32, i64, i64, i64, i64, i32]
    L.sol_attn_workspace_bytes_kv.restype = sz
    L.sol_attn_workspace_layout_kv.argtypes = [i32, i64, i64, i64, i64, i32, ctypes.POINTER(WsLayout)]
    L.sol_attn_workspace_layout_kv.restype = i32
    L.sol_attn_fused_kv.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp, sz, vp]
    L.sol_attn_fused_kv.restype = i32
    L.sol_attn2_tail.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, sz, vp]
    L.sol_attn2_tail.restype = i32
    for name in ("sol_attn2_exact", "sol_attn2_pv8_exact"):
        getattr(L, name).argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, sz, vp]
        getattr(L, name).restype = i32
    full = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i64, i64, i32, vp, sz, vp]
    for name in ("sol_attn", "sol_attn2", "sol_attn2_pv8", "sol_attn_forward_train", "sol_attn2_forward_train"):
        getattr(L, name).argtypes = full
        getattr(L, name).restype = i32
    prep = [vp, vp, vp, i64, i64, i64, i64, f32, i32, vp, sz, vp]
    for name in ("sol_attn_prepare", "sol_attn2_prepare", "sol_attn2_pv8_prepare"):
        getattr(L, name).argtypes = prep
        getattr(L, name).restype = i32
    fused = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, sz, vp]
    for name in ("sol_attn_fused", "sol_attn2_fused"):
        getattr(L, name).argtypes = fused
        getattr(L, name).restype = i32
    dbg = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i64, i64, i32, i32, vp, sz, vp, vp, vp]
    for name in ("sol_attn_debug_routing", "sol_attn2_debug_routing"):
        getattr(L, name).argtypes = dbg
        getattr(L, name).restype = i32
    for name in ("sol_attn_backward", "sol_attn2_backward"):
        getattr(L, name).argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        getattr(L, name).restype = i32
    L.sol_attn_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i64, i64, i32, vp]
    L.sol_attn_noalloc.restype = i32
    _LIB = L
    return L


def _check(status: int, where: str):
    if status != SOL_OK:
        raise SolAttnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _sink_start(s: Optional[int]) -> int:
    return -1 if s is None else int(s)


def _check_tensors(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [batch, tokens, heads, 128]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, tokens, heads, 128]")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
    if k.shape != q.shape or v.shape != q.shape or k.device != q.device or v.device != q.device:
        raise ValueError("k and v must have the same shape and device as q")


def _check_like(t: Optional[torch.Tensor], q: torch.Tensor, name: str):
    """A caller-supplied output must be a contiguous bf16 tensor of q's shape on q's device
    (the kernels write it in full through a raw pointer)."""
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_contiguous()
            or t.shape != q.shape or t.device != q.device):
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor of q's shape {tuple(q.shape)} "
                         f"on {q.device}")


def _check_workspace(ws: torch.Tensor, q: torch.Tensor):
    """The workspace is device memory on q's device; its size is passed in bytes."""
    if not isinstance(ws, torch.Tensor) or ws.device != q.device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    if ws.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor (as alloc_workspace returns)")


def kv_splits_for(batch: int, tokens: int, heads: int, kv_splits: int = 0) -> int:
    """Effective key-range split count (0 = automatic)."""
    return int(lib().sol_attn_kv_splits(batch, tokens, heads, kv_splits))


def workspace_bytes(variant: int, batch: int, tokens: int, heads: int, head_dim: int = 128,
                    kv_splits: int = 0) -> int:
    n = lib().sol_attn_workspace_bytes_kv(variant, batch, tokens, heads, head_dim, kv_splits)
    if n == 0:
        st = lib().sol_attn_validate(batch, tokens, heads, head_dim, 1.0, -1, 0, 0)
        _check(st if st != SOL_OK else 2, "sol_attn_workspace_bytes")
    return int(n)


def workspace_layout(variant: int, batch: int, tokens: int, heads: int, head_dim: int = 128,
                     kv_splits: int = 0) -> WsLayout:
    L = WsLayout()
    _check(lib().sol_attn_workspace_layout_kv(variant, batch, tokens, heads, head_dim, kv_splits, ctypes.byref(L)),
           "sol_attn_workspace_layout_kv")
    return L


def alloc_workspace(variant: int, q: torch.Tensor, kv_splits: int = 0) -> torch.Tensor:
    B, N, H, D = q.shape
    return torch.empty(workspace_bytes(variant, B, N, H, D, kv_splits), dtype=torch.uint8, device=q.device)


def validate(batch: int, tokens: int, heads: int, head_dim: int, tau: float, sink_start: Optional[int],
             sink_tokens: int, thresh: str = "diag") -> int:
    """Host-only contract check; returns the status code (0 = ok)."""
    if thresh not in THRESH:
        return 8
    return lib().sol_attn_validate(batch, tokens, heads, head_dim, float(tau), _sink_start(sink_start),
                                   int(sink_tokens), THRESH[thresh])


def _full_call(fn_name: str, variant: int, q, k, v, tau, sink_start, sink_tokens, thresh, out, workspace):
    _check_tensors(q, k, v)
    if thresh not in THRESH:
        raise ValueError("thresh must be 'diag' or 'exact'")
    if not math.isfinite(float(tau)):
        raise ValueError("tau must be finite")
    B, N, H, D = q.shape
    _check_like(out, q, "out")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(variant, q)
    _check_workspace(workspace, q)
    st = getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, float(tau),
                                 _sink_start(sink_start), int(sink_tokens), THRESH[thresh], _ptr(workspace),
                                 workspace.numel(), _stream(q.device))
    _check(st, fn_name)
    return out


def sol_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
             sink_start: Optional[int] = None, sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, kv_splits: int = 0) -> torch.Tensor:
    """Sol-Attn forward on contiguous bf16 [batch, tokens, heads, 128] GPU tensors.

    tau: threshold coefficient (higher selects fewer KV blocks; 0 is not dense).
    sink_start None with sink_tokens > 0 keeps the last sink_tokens tokens exact.
    kv_splits: key-range splits of the fused pass (0 = automatic).
    """
    if kv_splits == 0:
        return _full_call("sol_attn", SOL_VARIANT_SOL1, q, k, v, tau, sink_start, sink_tokens, thresh, out,
                          workspace)
    _check_tensors(q, k, v)
    _check_like(out, q, "out")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(SOL_VARIANT_SOL1, q, kv_splits)
    prepare(SOL_VARIANT_SOL1, q, k, v, tau, workspace, thresh)
    fused(SOL_VARIANT_SOL1, q, k, v, out, workspace, sink_start, sink_tokens, kv_splits)
    return out


def sol_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, tau: float = 1.0,
                     thresh: str = "diag", sink_start: Optional[int] = None, sink_tokens: int = 0) -> torch.Tensor:
    """Sol-Attn on the library's static per-device scratch: the C call allocates nothing.

    The caller passes `out` (a contiguous bf16 tensor of q's shape); shapes whose workspace
    exceeds NOALLOC_SCRATCH_BYTES raise SolAttnError (status SOL_ERR_SCRATCH).  Calls that
    overlap on one device race on the shared scratch."""
    _check_tensors(q, k, v)
    if out is None:
        raise ValueError("out is required (the no-allocation call writes into the caller's tensor)")
    _check_like(out, q, "out")
    if thresh not in THRESH:
        raise ValueError("thresh must be 'diag' or 'exact'")
    if not math.isfinite(float(tau)):
        raise ValueError("tau must be finite")
    B, N, H, D = q.shape
    _check(lib().sol_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, float(tau),
                                  _sink_start(sink_start), int(sink_tokens), THRESH[thresh], _stream(q.device)),
           "sol_attn_noalloc")
    return out


def sol_attn2(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
              sink_start: Optional[int] = None, sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sol-Attn2 forward (FP8 Q/K, complementary tail) on the same tensor contract."""
    return _full_call("sol_attn2", SOL_VARIANT_SOL2, q, k, v, tau, sink_start, sink_tokens, thresh, out, workspace)


def sol_attn2_pv8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
                  sink_start: Optional[int] = None, sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sol-Attn2 with ExpCast P and per-head FP8 V (FP8 PV)."""
    return _full_call("sol_attn2_pv8", SOL_VARIANT_SOL2_PV8, q, k, v, tau, sink_start, sink_tokens, thresh, out,
                      workspace)


def forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
                  sink_start: Optional[int] = None, sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Sol-Attn forward that keeps its routing and row log-sum-exp for `backward`;
    returns (out, workspace)."""
    if workspace is None:
        workspace = alloc_workspace(SOL_VARIANT_SOL1_TRAIN, q)
    out = _full_call("sol_attn_forward_train", SOL_VARIANT_SOL1_TRAIN, q, k, v, tau, sink_start, sink_tokens, thresh,
                     out, workspace)
    return out, workspace


def forward_train2(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
                   sink_start: Optional[int] = None, sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Sol-Attn2 forward that keeps its routing, groups, anchor tails and row log-sum-exp for
    `backward2`; returns (out, workspace)."""
    if workspace is None:
        workspace = alloc_workspace(SOL_VARIANT_SOL2_TRAIN, q)
    out = _full_call("sol_attn2_forward_train", SOL_VARIANT_SOL2_TRAIN, q, k, v, tau, sink_start, sink_tokens,
                     thresh, out, workspace)
    return out, workspace


def _backward_call(fn_name: str, q, k, v, out, dout, workspace, dq, dk, dv):
    _check_tensors(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor of q's shape on q's device")
    B, N, H, D = q.shape
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_like(t, q, name)
    _check_workspace(workspace, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check(getattr(lib(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                   B, N, H, D, _ptr(workspace), workspace.numel(), _stream(q.device)), fn_name)
    return dq, dk, dv


def backward2(q, k, v, out, dout, workspace: torch.Tensor, dq: Optional[torch.Tensor] = None,
              dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(dout * out) with the routing and groups of the
    `forward_train2` call that filled `workspace` held fixed."""
    return _backward_call("sol_attn2_backward", q, k, v, out, dout, workspace, dq, dk, dv)


def backward(q, k, v, out, dout, workspace: torch.Tensor, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(dout * out) with the routing of the `forward_train` call
    that filled `workspace` held fixed."""
    return _backward_call("sol_attn_backward", q, k, v, out, dout, workspace, dq, dk, dv)


class SolAttnFunction(torch.autograd.Function):
    """Sol-Attn as a differentiable op: forward_train, then backward with the routing fixed."""

    @staticmethod
    def forward(ctx, q, k, v, tau, thresh, sink_start, sink_tokens):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, ws = forward_train(q, k, v, tau, thresh, sink_start, sink_tokens)
        ctx.save_for_backward(q, k, v, out, ws)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, ws = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, out, dout.contiguous(), ws)
        return dq, dk, dv, None, None, None, None


def sol_attn_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
                   sink_start: Optional[int] = None, sink_tokens: int = 0) -> torch.Tensor:
    """Differentiable Sol-Attn (autograd): gradients flow through q, k, v with the forward's routing fixed."""
    return SolAttnFunction.apply(q, k, v, tau, thresh, sink_start, sink_tokens)


class SolAttn2Function(torch.autograd.Function):
    """Sol-Attn2 as a differentiable op: forward_train2, then backward2 with routing and groups fixed."""

    @staticmethod
    def forward(ctx, q, k, v, tau, thresh, sink_start, sink_tokens):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, ws = forward_train2(q, k, v, tau, thresh, sink_start, sink_tokens)
        ctx.save_for_backward(q, k, v, out, ws)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, ws = ctx.saved_tensors
        dq, dk, dv = backward2(q, k, v, out, dout.contiguous(), ws)
        return dq, dk, dv, None, None, None, None


def sol_attn2_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float = 1.0, thresh: str = "diag",
                    sink_start: Optional[int] = None, sink_tokens: int = 0) -> torch.Tensor:
    """Differentiable Sol-Attn2 (autograd): gradients flow through q, k, v (the E4M3 quantizer
    passed straight through) with the forward's routing and key groups fixed."""
    return SolAttn2Function.apply(q, k, v, tau, thresh, sink_start, sink_tokens)


def prepare(variant: int, q, k, v, tau: float, workspace: torch.Tensor, thresh: str = "diag"):
    """Stage 1 (summaries + threshold [+ Sol-Attn2 quantization and groups]) into `workspace`."""
    _check_tensors(q, k, v)
    _check_workspace(workspace, q)
    B, N, H, D = q.shape
    name = {SOL_VARIANT_SOL1: "sol_attn_prepare", SOL_VARIANT_SOL2: "sol_attn2_prepare",
            SOL_VARIANT_SOL2_PV8: "sol_attn2_pv8_prepare"}[variant]
    _check(getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), B, N, H, D, float(tau), THRESH[thresh],
                                _ptr(workspace), workspace.numel(), _stream(q.device)), name)


def fused(variant: int, q, k, v, out, workspace: torch.Tensor, sink_start: Optional[int] = None,
          sink_tokens: int = 0, kv_splits: int = 0):
    """Stage 2 (the fused kernel [+ split merge]) reading a workspace prepared for the same inputs."""
    _check_tensors(q, k, v)
    _check_like(out, q, "out")
    _check_workspace(workspace, q)
    B, N, H, D = q.shape
    if variant == SOL_VARIANT_SOL1:
        _check(lib().sol_attn_fused_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, _sink_start(sink_start),
                                       int(sink_tokens), int(kv_splits), _ptr(workspace), workspace.numel(),
                                       _stream(q.device)), "sol_attn_fused_kv")
        return
    if variant == SOL_VARIANT_SOL2_PV8:
        tail2(q, k, v, workspace, sink_start, sink_tokens)
        exact2(q, k, v, out, workspace, pv8=True, sink_start=sink_start, sink_tokens=sink_tokens)
        return
    _check(lib().sol_attn2_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, _sink_start(sink_start),
                                 int(sink_tokens), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "sol_attn2_fused")


def tail2(q, k, v, workspace: torch.Tensor, sink_start: Optional[int] = None, sink_tokens: int = 0):
    """Sol-Attn2 stage 2a: the per-anchor tail (routed on chip), into the workspace."""
    _check_tensors(q, k, v)
    _check_workspace(workspace, q)
    B, N, H, D = q.shape
    _check(lib().sol_attn2_tail(_ptr(q), _ptr(k), _ptr(v), B, N, H, D, _sink_start(sink_start), int(sink_tokens),
                                _ptr(workspace), workspace.numel(), _stream(q.device)), "sol_attn2_tail")


def exact2(q, k, v, out, workspace: torch.Tensor, pv8: bool = False, sink_start: Optional[int] = None,
           sink_tokens: int = 0):
    """Sol-Attn2 stage 2b: the exact FP8 pass (FP8 PV with pv8), routed on chip with the sink
    given to stage 2a, combined with the tail of stage 2a."""
    _check_tensors(q, k, v)
    _check_like(out, q, "out")
    if out is None:
        raise ValueError("out is required")
    _check_workspace(workspace, q)
    B, N, H, D = q.shape
    name = "sol_attn2_pv8_exact" if pv8 else "sol_attn2_exact"
    _check(getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, _sink_start(sink_start),
                                sink_tokens, _ptr(workspace), workspace.numel(), _stream(q.device)), name)


def debug_routing(variant: int, q, k, v, tau: float = 1.0, thresh: str = "diag", sink_start: Optional[int] = None,
                  sink_tokens: int = 0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, kv_splits: int = 0, return_pairs: bool = False):
    """Run the full call and return (out, masks [B, H, nb, nb] bool on the CPU, workspace), plus,
    with return_pairs, the kernel's count of selected token pairs sum n_i n_j (a Python int).

    The masks and the count are what the fused kernel itself decided (test export)."""
    _check_tensors(q, k, v)
    _check_like(out, q, "out")
    B, N, H, D = q.shape
    nb = (N + 63) // 64
    nbw = (nb + 63) // 64
    if workspace is None:
        workspace = alloc_workspace(variant, q, kv_splits)
    _check_workspace(workspace, q)
    words = torch.zeros(B * H * nb * nbw, dtype=torch.int64, device=q.device)
    pairs = torch.zeros(1, dtype=torch.int64, device=q.device)
    name = "sol_attn_debug_routing" if variant == SOL_VARIANT_SOL1 else "sol_attn2_debug_routing"
    _check(getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, H, D, float(tau),
                                _sink_start(sink_start), int(sink_tokens), THRESH[thresh], int(kv_splits),
                                _ptr(workspace), workspace.numel(), _ptr(words), _ptr(pairs), _stream(q.device)),
           name)
    w = words.view(B, H, nb, nbw).cpu()
    bits = torch.arange(64, dtype=torch.int64)
    m = ((w.unsqueeze(-1) >> bits) & 1).bool().reshape(B, H, nb, nbw * 64)[..., :nb]
    if return_pairs:
        return out, m, workspace, int(pairs.item())
    return out, m, workspace


def workspace_views(variant: int, workspace: torch.Tensor, batch: int, tokens: int, heads: int) -> dict:
    """Typed views of the workspace arrays (for tests)."""
    L = workspace_layout(variant, batch, tokens, heads)
    nbp = L.nbp
    bh = batch * heads

    def view(off, dtype, shape):
        if off < 0:
            return None
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype).view(*shape)

    d = dict(
        nb=L.nb, nbp=nbp,
        qbar=view(L.qbar, torch.float32, (batch, heads, nbp, 128)),
        kbar_t=view(L.kbar_t, torch.float32, (batch, heads, 32, nbp, 4)),
        kbar_h=view(L.kbar_h, torch.bfloat16, (batch, heads, nbp, 128)),
        vbar_h=view(L.vbar_h, torch.bfloat16, (batch, heads, nbp, 128)),
        kh=view(L.kh, torch.bfloat16, (batch, heads, tokens, 128)),
        vh=view(L.vh, torch.bfloat16, (batch, heads, tokens, 128)),
        tau_i=view(L.tau_i, torch.float32, (batch, heads, nbp)),
        kstat=view(L.kstat, torch.float32, (batch, heads, 2, 128)),
        kcov=view(L.kcov, torch.float32, (batch, heads, 128, 128)),
        wcnt=view(L.wcnt, torch.uint8, (batch, heads, nbp // 64, nbp)),
        qcount=view(L.qcount, torch.int32, (batch, heads, max(1, L.kv_splits), nbp)),
        order=view(L.order, torch.int32, (batch, heads, max(1, L.kv_splits), nbp)),
    )
    if variant in (SOL_VARIANT_SOL2, SOL_VARIANT_SOL2_PV8, SOL_VARIANT_SOL2_TRAIN):
        tp = nbp * 64
        d.update(
            q8=view(L.q8, torch.uint8, (batch, heads, tp, 128)),
            k8=view(L.k8, torch.uint8, (batch, heads, tp, 128)),
            qscale=view(L.qscale, torch.float32, (batch, heads, nbp)),
            kscale=view(L.kscale, torch.float32, (batch, heads, nbp)),
            qhat=view(L.qhat, torch.float32, (batch, heads, 128)),
            gk=view(L.gk, torch.bfloat16, (batch, heads, nbp, 2, 128)),
            gv=view(L.gv, torch.bfloat16, (batch, heads, nbp, 2, 128)),
            glogn=view(L.glogn, torch.float32, (batch, heads, nbp, 2)),
            ghi=view(L.ghi, torch.int64, (batch, heads, nbp)),
            qanc=view(L.qanc, torch.float32, (batch, heads, nbp, 2, 128)),
            tmu=view(L.tmu, torch.float32, (batch, heads, nbp, 2, 128)),
            tnu=view(L.tnu, torch.float32, (batch, heads, nbp, 2, 128)),
            tlz=view(L.tlz, torch.float32, (batch, heads, nbp, 2)),
        )
    if variant == SOL_VARIANT_SOL1_TRAIN:
        tp = nbp * 64
        d.update(
            lse=view(L.lse, torch.float32, (batch, heads, tp)),
            mrow=view(L.mrow, torch.int64, (batch, heads, L.nb, nbp // 64)),
            mcol=view(L.mcol, torch.int64, (batch, heads, L.nb, nbp // 64)),
            ld=view(L.ld, torch.float32, (batch, heads, tp, 2)),
            dkbar=view(L.dkbar, torch.float32, (batch, heads, nbp, 128)),
            dvbar=view(L.dvbar, torch.float32, (batch, heads, nbp, 128)),
            bqord=view(L.bqord, torch.int32, (batch, heads, nbp)),
            bkord=view(L.bkord, torch.int32, (batch, heads, nbp)),
        )
    if variant == SOL_VARIANT_SOL2_TRAIN:
        tp = nbp * 64
        d.update(
            sel=view(L.sel, torch.int64, (batch, heads, L.nb, nbp // 64)),
            lse=view(L.lse, torch.float32, (batch, heads, tp)),
            ofp=view(L.ofp, torch.float32, (batch, heads, tp, 128)),
            mcol=view(L.mcol, torch.int64, (batch, heads, L.nb, nbp // 64)),
            ld=view(L.ld, torch.float32, (batch, heads, tp, 2)),
            qd=view(L.qd, torch.bfloat16, (batch, tokens, heads, 128)),
            kd=view(L.kd, torch.bfloat16, (batch, tokens, heads, 128)),
            dlam=view(L.dlam, torch.float32, (batch, heads, tp)),
            qab=view(L.qab, torch.bfloat16, (batch, heads, nbp, 2, 128)),
            dmub=view(L.dmub, torch.bfloat16, (batch, heads, nbp, 2, 128)),
            dnub=view(L.dnub, torch.bfloat16, (batch, heads, nbp, 2, 128)),
            alz=view(L.alz, torch.float32, (batch, heads, nbp, 2, 2)),
            aextra=view(L.aextra, torch.float32, (batch, heads, nbp, 2, 128)),
            gdk=view(L.gdk, torch.float32, (batch, heads, nbp, 2, 128)),
            gdv=view(L.gdv, torch.float32, (batch, heads, nbp, 2, 128)),
            bqord=view(L.bqord, torch.int32, (batch, heads, nbp)),
            bkord=view(L.bkord, torch.int32, (batch, heads, nbp)),
        )
    if variant == SOL_VARIANT_SOL2_PV8:
        tp = nbp * 64
        d.update(
            v8t=view(L.v8t, torch.uint8, (batch, heads, 128, tp)),
            vbmax=view(L.vbmax, torch.float32, (batch, heads, nbp)),
            vscale=view(L.vscale, torch.float32, (batch, heads)),
        )
    del bh
    return d
