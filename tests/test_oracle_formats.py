"""Pins for the oracle's bit-format decoders (CPU only).

The E4M3FN landmarks are the OCP FP8 definition of the format that the
FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4`` page calls "per-tensor
FP8 E4M3" and the vLLM listing calls ``torch.float8_e4m3fn``: bias 7,
subnormals at exponent 0, NaN only at S.1111.111, max 448.  torch's own
casts are a second, independent decoder.
"""

import numpy as np
import pytest
import torch

from oracle.formats import (bf16_bits_to_f64, e4m3fn_bits_to_f64,
                            round_to_bf16)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0),
    (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xFE, -448.0),
])
def test_e4m3fn_landmarks(code, value):
    assert e4m3fn_bits_to_f64(np.uint8(code)) == value


def test_e4m3fn_nan_and_negative_zero():
    v = e4m3fn_bits_to_f64(np.array([0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3fn_bits_to_f64(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])


def test_e4m3fn_values_are_exact_bf16():
    # every finite E4M3FN value has <= 4 significant bits, so the BF16
    # pattern (upper half of its binary32) represents it exactly
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3fn_bits_to_f64(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(round_to_bf16(vals[fin]), vals[fin])


@pytest.mark.parametrize("bits,value", [
    (0x0000, 0.0), (0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7),
    (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, 2.0 ** 127 * (2 - 2.0 ** -7)),
])
def test_bf16_landmarks(bits, value):
    assert bf16_bits_to_f64(np.uint16(bits)) == value


def test_bf16_sweep_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    ours = bf16_bits_to_f64(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])


def test_round_to_bf16_ties_to_even():
    x = np.array([1 + 2.0 ** -8,          # tie between 1 and 1+2^-7 -> 1
                  1 + 3 * 2.0 ** -8,      # tie -> 1 + 2^-6 (even mantissa)
                  -(1 + 2.0 ** -8),
                  1 + 2.0 ** -8 + 2.0 ** -30,   # just above the tie -> up
                  2.0 ** -140,            # subnormal region: spacing 2^-133
                  3 * 2.0 ** -134])       # tie at the subnormal spacing
    want = np.array([1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7, 0.0,
                     2 * 2.0 ** -133])
    assert np.array_equal(round_to_bf16(x), want)


def test_round_to_bf16_matches_torch_on_binary32_inputs():
    # torch rounds float32 -> bf16 once; on binary32-exact inputs the result
    # must agree with the direct binary64 rounding
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))
         ).astype(np.float32)
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), theirs)
