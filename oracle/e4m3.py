"""OCP FP8 E4M3FN codec from the format's definition (test infrastructure only).

The Sol-Attn2 draft ("FP8 quantization and ExpCast") quantizes Q and K to
E4M3 with a per-block scale s_X = max|X| / 448; 448 is the largest finite
E4M3FN magnitude, so the format is the OCP "FN" variant (no infinities, one
NaN pattern per sign).  Bit layout: sign(1) | exponent(4, bias 7) |
mantissa(3).  Exponent field 0 encodes subnormals m/8 * 2^-6; field 15 with
mantissa 7 is NaN; every other code is (1 + m/8) * 2^(e-7).

Encoding is round-to-nearest, ties to the even code, with saturation to
+/-448 (the reading adopted for values just above 448 after division by a
rounded scale).  It is written as "pick the nearest representable value",
which is the definition of RNE, not as bit manipulation.
"""
from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0


def decode_code(code: int) -> float:
    """Value of one E4M3FN byte."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values in code order 0x00..0x7E (monotonic increasing).
_POS = DECODE[:0x7F].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """Vectorized decode of uint8 codes to float64."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(x) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest value, ties to even, saturating."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_sat = np.minimum(a, MAX_FINITE)
    hi = np.searchsorted(_POS, a_sat, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - _POS[lo]
    d_hi = _POS[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(_POS[hi] == a_sat, hi.astype(np.uint8), code)
    code = code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def quantize_block_fp32(x_block: np.ndarray):
    """One quantization block: s = max|X| / 448 and X8 = E4M3(X / s), both in IEEE fp32.

    Sol-Attn2 draft, "FP8 quantization and ExpCast".  The pages do not say what
    happens to an all-zero block; the reading is s = 1 (every code is then 0).
    Returns (codes uint8, s as np.float32).
    """
    xf = np.asarray(x_block, dtype=np.float32)
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0)
    s = np.float32(amax / np.float32(MAX_FINITE)) if amax > 0 else np.float32(1.0)
    y = (xf / s).astype(np.float32)           # correctly rounded fp32 division
    return encode_rne(y), s


# ----------------------------------------------------------------------------
# ExpCast (Sol-Attn2 draft, "FP8 quantization and ExpCast", after VC-Attention):
# a base-2 score u = (s - m) log2 e maps straight to an E4M3 probability byte,
#     c(u) = clip_[0,120]( RNE(8 u + 55.65) ),   p-hat(u) = decode(c(u)) ~ 2^u.
# For u = k + phi the byte is 8 (k + 7) + j with mantissa j ~ 8 phi, i.e. the
# exponent field carries k and the mantissa a linear stand-in for 2^phi; the
# 55.65 (not 56) offset shifts the rounding points to balance that stand-in.
# The rounding decides an integer, so it is done in IEEE fp32, as the kernel does.
# ----------------------------------------------------------------------------

def expcast_code(u) -> np.ndarray:
    """ExpCast codes of base-2 scores u (float array): uint8 in [0, 120]."""
    uf = np.asarray(u, dtype=np.float32)
    t = (np.float32(8.0) * uf + np.float32(55.65)).astype(np.float32)   # 8 u is exact in fp32
    c = np.rint(t)                                                       # nearest, ties to even
    return np.clip(c, 0.0, 120.0).astype(np.uint8)


def expcast_weight(u) -> np.ndarray:
    """p-hat(u) = decode(c(u)), float64."""
    return decode(expcast_code(u))
