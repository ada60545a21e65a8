"""CPU oracle for the Sol-Attn and Sol-Attn2 forward passes -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, float64 restatement of what the Sol-Attn pages
define.  Only the test suite, the smoke check and the bench's CPU-baseline leg
may import it; the library's product path never does, and this package shares
no code, tables or constants with the HIP implementation.

Modules
-------
sol_attn   Sol-Attn (block summaries, diagonal / full-covariance thresholds,
           routing with an exact KV sink, exact + proxy-reuse output).
e4m3       OCP FP8 E4M3FN codec written from the format's definition.
sol_attn2  Sol-Attn2 complementary tail (FP8 Q/K, two key groups per block,
           query anchors, first-order mass correction, shared denominator).
brute      Scalar-loop pure-Python versions of both, for tiny inputs.

Parity status: every function is pinned by tests under ``tests/`` (closed
forms, reductions to textbook attention, brute force, invariants), except the
Sol-Attn2 group-split rule and mean-query direction, which the pages leave
open; those follow a stated reading and are marked "parity unpinned" in
``oracle/sol_attn2.py``.
"""
from . import e4m3, sol_attn, sol_attn2, brute  # noqa: F401
