"""Bit formats of the inputs, decoded from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages state the element types but not their encodings: the FlashInfer
``trtllm_batch_decode_sparse_mla_dsv4`` page says the query may be BF16 or
per-tensor FP8 E4M3 and the pools use head dim 512; the vLLM
``DeepseekV4FlashInferMLAAttention`` listing names ``torch.float8_e4m3fn``.
The encodings below are the public definitions of those two types:

* BF16: the upper 16 bits of an IEEE-754 binary32 value.
* OCP FP8 E4M3FN ("fn": finite, no infinities): 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; the largest finite
  magnitude is 1.75 * 2^8 = 448.

Pinned by tests/test_oracle_formats.py (closed-form landmark values and all
256 E4M3FN codes / a sweep of BF16 codes against torch's own casts) and, for
the packed block-scaled row, tests/test_oracle_packed.py (every UE8M0 code,
hand-assembled rows, and the decode against the plain definition).
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 BF16 patterns -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


_E4M3FN = _e4m3fn_table()


def e4m3fn_bits_to_f64(bits) -> np.ndarray:
    """uint8 OCP E4M3FN patterns -> exact float64 values (NaN for S.1111.111)."""
    return _E4M3FN[np.asarray(bits, dtype=np.uint8)]


# The packed block-scaled FP8 row.  FlashInfer
# ``trtllm_batch_decode_sparse_mla_dsv4`` (introduction, packed-backend
# paragraph; parameter ``swa_kv_cache``) gives only its size, 584 bytes per
# token of uint8, and vLLM ``DeepseekV4FlashInferMLAAttention`` (the class
# comment on ``use_flashmla_fp8_layout``) its family, UE8M0 block-scaled FP8.
# Reading (the pages leave the byte order open): the row holds the 512 dims
# in the order the query lays them out (448 NoPE, then 64 RoPE, per the Cake
# page's ``q`` parameter), then its scales --
#   bytes [0, 448)   : NoPE dims 0..447 as OCP E4M3FN codes,
#   bytes [448, 576) : RoPE dims 448..511 as BF16, little-endian,
#   bytes [576, 584) : eight UE8M0 scale bytes; byte j scales NoPE dims
#                      [56 j, 56 j + 56) (448 = 8 x 56 uses every byte),
# and NoPE dim d decodes to E4M3FN(byte d) * 2^(scale[d // 56] - 127).
PACKED_ROW_BYTES = 584
PACKED_NOPE_DIMS = 448
PACKED_BLOCK_DIMS = 56
PACKED_ROPE_OFFSET = 448
PACKED_SCALE_OFFSET = 576


def ue8m0_to_f64(codes) -> np.ndarray:
    """UE8M0 scale bytes (an 8-bit biased exponent with no sign and no
    mantissa, bias 127) -> exact float64 powers of two 2^(e - 127); the
    all-ones byte 255 is NaN."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(np.ones(e.shape), e - 127)
    return np.where(e == 255, np.nan, out)


def packed584_to_f64(bits) -> np.ndarray:
    """[..., 584] uint8 packed rows -> [..., 512] exact float64 values."""
    b = np.asarray(bits, dtype=np.uint8)
    if b.shape[-1] != PACKED_ROW_BYTES:
        raise ValueError(f"packed rows have {PACKED_ROW_BYTES} bytes, got {b.shape[-1]}")
    nope = e4m3fn_bits_to_f64(b[..., :PACKED_NOPE_DIMS])
    scale = ue8m0_to_f64(b[..., PACKED_SCALE_OFFSET:PACKED_ROW_BYTES])
    nope = nope * np.repeat(scale, PACKED_BLOCK_DIMS, axis=-1)
    lo = b[..., PACKED_ROPE_OFFSET:PACKED_SCALE_OFFSET:2].astype(np.uint16)
    hi = b[..., PACKED_ROPE_OFFSET + 1:PACKED_SCALE_OFFSET:2].astype(np.uint16)
    rope = bf16_bits_to_f64(lo | (hi << np.uint16(8)))
    return np.concatenate([nope, rope], axis=-1)


def decode_bits(bits, dtype: str) -> np.ndarray:
    """Decode stored patterns of ``dtype`` ("bf16", "fp8_e4m3fn", or
    "packed_fp8_584" for [..., 584]-byte packed rows)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "fp8_e4m3fn":
        return e4m3fn_bits_to_f64(bits)
    if dtype == "packed_fp8_584":
        return packed584_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest BF16 value, ties to even, and
    return them as float64.  The rounding is done on the binary64 value
    directly (no intermediate binary32 step, which would round twice)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    # BF16 keeps 8 significant bits (1 implicit + 7 stored).  For a value
    # with exponent e (|x| in [2^e, 2^(e+1))) the spacing is 2^(e-7), and
    # below the smallest normal 2^-126 the spacing is fixed at 2^-133.
    mag = np.abs(xf)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    # guard the floor(log2) estimate against rounding at exact powers of two
    e = np.where(2.0 ** e > mag, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= mag, e + 1, e)
    e = np.maximum(e, -126.0)
    ulp = 2.0 ** (e - 7)
    q = xf / ulp                      # exact: division by a power of two
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))
    r = r + up
    res = r * ulp
    res = np.where(mag == 0, xf, res)
    # beyond the largest finite BF16 value the result overflows to inf
    big = 2.0 ** 127 * (2.0 - 2.0 ** -7)
    res = np.where(np.abs(res) > big, np.copysign(np.inf, xf), res)
    out[finite] = res
    return out
