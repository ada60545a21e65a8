"""Sol-Attn / Sol-Attn2 for AMD Instinct MI355X (gfx950): the forward passes and their
backward passes with the routing (and Sol-Attn2's key groups) fixed.

The compute lives in libsolattn.so (hand-written HIP kernels behind a C ABI,
include/solattn.h); this package is its thin ctypes binding.  Tensors are
contiguous bf16 [batch, tokens, heads, 128] on the GPU (Sol-Attn README,
"Core API").
"""
from ._lib import (SOL_VARIANT_SOL1, SOL_VARIANT_SOL1_TRAIN, SOL_VARIANT_SOL2, SOL_VARIANT_SOL2_PV8,  # noqa: F401
                   SOL_VARIANT_SOL2_TRAIN, SolAttn2Function, SolAttnError, SolAttnFunction, alloc_workspace, backward,
                   backward2, debug_routing, exact2, forward_train, forward_train2, fused, kv_splits_for, lib, prepare,
                   sol_attn, sol_attn2, sol_attn2_pv8, sol_attn2_train, sol_attn_noalloc, sol_attn_train, tail2,
                   validate, workspace_bytes, workspace_layout, workspace_views)

__all__ = ["sol_attn", "sol_attn2", "sol_attn2_pv8", "validate", "workspace_bytes", "workspace_layout", "prepare",
           "fused", "tail2", "exact2", "debug_routing", "alloc_workspace", "kv_splits_for", "workspace_views",
           "SolAttnError", "lib", "SOL_VARIANT_SOL1", "SOL_VARIANT_SOL2", "SOL_VARIANT_SOL2_PV8",
           "SOL_VARIANT_SOL1_TRAIN", "forward_train", "backward", "sol_attn_train", "SolAttnFunction",
           "sol_attn_noalloc", "SOL_VARIANT_SOL2_TRAIN", "forward_train2", "backward2", "sol_attn2_train",
           "SolAttn2Function"]
