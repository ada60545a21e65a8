"""Pins of the oracle's OCP E4M3FN codec and per-block quantization (CPU only).

References: the OCP 8-bit floating point format (E4M3FN: bias 7, max 448, no
infinities), PyTorch's ``torch.float8_e4m3fn`` CPU conversion as an
independent library routine, and the Sol-Attn2 draft "FP8 quantization and
ExpCast" (s = max|X| / 448).
"""
import math

import numpy as np
import pytest
import torch

from oracle import e4m3


def test_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256))
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    np.testing.assert_array_equal(nan_ref, nan_ours)
    np.testing.assert_array_equal(ref[~nan_ref], ours[~nan_ours])


def test_decode_landmarks():
    assert e4m3.decode_code(0x7E) == 448.0
    assert e4m3.decode_code(0xFE) == -448.0
    assert e4m3.decode_code(0x01) == 2.0 ** -9
    assert e4m3.decode_code(0x07) == 7 * 2.0 ** -9
    assert e4m3.decode_code(0x08) == 2.0 ** -6
    assert e4m3.decode_code(0x38) == 1.0
    assert e4m3.decode_code(0x3C) == 1.5
    assert math.isnan(e4m3.decode_code(0x7F)) and math.isnan(e4m3.decode_code(0xFF))
    assert e4m3.decode_code(0x77) == 240.0 and e4m3.decode_code(0x78) == 256.0


def _torch_encode(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(50000) * 1e-2,
        rng.standard_normal(50000) * 1e-3,
    ]).astype(np.float32)
    np.testing.assert_array_equal(e4m3.encode_rne(x), _torch_encode(x))


def test_encode_ties_go_to_even_code():
    pos = e4m3.DECODE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)       # exact ties (all representable)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)
    codes = e4m3.encode_rne(mids)
    assert np.all(codes % 2 == 0)
    np.testing.assert_array_equal(codes, _torch_encode(mids))
    np.testing.assert_array_equal(e4m3.encode_rne(-mids), _torch_encode(-mids))


def test_encode_saturates_and_keeps_nan():
    assert e4m3.encode_rne(np.float32(1000.0)) == 0x7E
    assert e4m3.encode_rne(np.float32(-1e30)) == 0xFE
    assert e4m3.encode_rne(np.float32(460.0)) == 0x7E
    assert e4m3.encode_rne(np.float32(np.nan)) == 0x7F
    assert e4m3.encode_rne(np.float32(0.0)) == 0x00
    assert e4m3.encode_rne(np.float32(-0.0)) == 0x80
    assert e4m3.encode_rne(np.float32(2.0 ** -11)) == 0x00        # below half the smallest subnormal
    assert e4m3.encode_rne(np.float32(2.0 ** -10 * 1.01)) == 0x01


def test_block_quantization_scale_and_error_bound():
    """s = max|X|/448 in fp32; the largest magnitude maps to 448; |X - s X8| <= s * half-ulp(X8)."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    codes, s = e4m3.quantize_block_fp32(x)
    assert s == np.float32(np.abs(x).max() / np.float32(448))
    dec = e4m3.decode(codes)
    assert np.abs(dec).max() == 448.0
    y = x.astype(np.float32) / s
    np.testing.assert_array_equal(codes, _torch_encode(y))
    # half-ulp bound: spacing of E4M3 at |y| is 2^(floor(log2|y|) - 3), subnormal spacing 2^-9
    ay = np.abs(y.astype(np.float64))
    expo = np.floor(np.log2(np.maximum(ay, 2.0 ** -6)))
    half_ulp = 0.5 * 2.0 ** (expo - 3)
    assert np.all(np.abs(ay - np.abs(dec)) <= half_ulp * (1 + 1e-12))


def test_zero_block_uses_unit_scale():
    codes, s = e4m3.quantize_block_fp32(np.zeros((64, 8), dtype=np.float32))
    assert s == np.float32(1.0) and not codes.any()


@pytest.mark.parametrize("shape", [(64, 128), (13, 128)])
def test_quantize_head_partial_block(shape):
    from oracle.sol_attn2 import quantize_head
    rng = np.random.default_rng(2)
    n = 64 + shape[0]
    x = torch.from_numpy(rng.standard_normal((n, 128)).astype(np.float32)).to(torch.bfloat16)
    x = x.to(torch.float64).numpy()
    codes, scales, deq = quantize_head(x)
    assert scales.shape == (2,)
    for j, (s, e) in enumerate([(0, 64), (64, n)]):
        assert scales[j] == np.float32(np.float32(np.abs(x[s:e]).max()) / np.float32(448))
        np.testing.assert_array_equal(deq[s:e], np.float64(scales[j]) * e4m3.decode(codes[s:e]))
