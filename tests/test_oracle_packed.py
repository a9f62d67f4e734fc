"""Pins of the oracle's packed block-scaled FP8 row (584 bytes: 448 E4M3FN
NoPE codes, 64 BF16 RoPE dims little-endian, 8 UE8M0 scale bytes of 56 NoPE
dims each -- a reading of the FlashInfer trtllm_batch_decode_sparse_mla_dsv4
page (introduction, packed-backend paragraph; ``swa_kv_cache``) and the vLLM
DeepseekV4FlashInferMLAAttention class comment on ``use_flashmla_fp8_layout``,
which give only the size and the family).

The expected values here are built independently of oracle/formats.py:
scales with math.ldexp, E4M3FN values from the format's definition written
out as a formula, BF16 values through struct (the upper half of a binary32),
bytes assembled with struct.pack in little-endian order.
"""

import math
import struct

import numpy as np
import pytest

import oracle
from oracle.brute import brute_force_decode
from sparse_mla_decode_gather_amd import workloads as W


def e4m3(code):
    """OCP E4M3FN by its definition (bias 7, subnormals m/8 * 2^-6)."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1 + m / 8.0) * 2.0 ** (e - 7)


def bf16_from_float(x):
    """The BF16 bits of a float that BF16 holds exactly."""
    bits = struct.unpack("<I", struct.pack("<f", x))[0]
    assert bits & 0xFFFF == 0, x
    return bits >> 16


def assemble(nope_codes, scale_bytes, rope_values):
    """One 584-byte row from its parts (little-endian BF16 RoPE)."""
    assert len(nope_codes) == 448 and len(scale_bytes) == 8 and len(rope_values) == 64
    raw = bytes(nope_codes) + b"".join(
        struct.pack("<H", bf16_from_float(v)) for v in rope_values) + bytes(scale_bytes)
    assert len(raw) == 584
    return np.frombuffer(raw, dtype=np.uint8)


def test_every_ue8m0_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.ue8m0_to_f64(codes)
    for c in range(255):
        assert got[c] == math.ldexp(1.0, c - 127), c
    assert math.isnan(got[255])
    # landmarks
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5
    assert got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_hand_assembled_row():
    rng = np.random.default_rng(0)
    codes = [int(c) for c in rng.integers(0, 256, 448)]
    codes = [c if (c & 0x7F) != 0x7F else 0x38 for c in codes]     # no NaN codes
    scales = [127, 120, 130, 127 - 20, 127 + 15, 1, 254, 100]
    rope = [float(v) for v in (np.arange(64) - 31.5) / 4.0]          # exact in BF16
    row = assemble(codes, scales, rope)
    got = oracle.packed584_to_f64(row)
    want = [e4m3(codes[d]) * math.ldexp(1.0, scales[d // 56] - 127) for d in range(448)]
    want += rope
    assert got.shape == (512,)
    assert np.array_equal(got, np.array(want)), np.nonzero(got != np.array(want))


def test_block_boundaries_and_byte_order():
    """Dim 55 and dim 56 fall in different blocks; RoPE dim 0 is bytes 448
    (low) and 449 (high); the scales are the last 8 bytes."""
    codes = [0x38] * 448                        # 1.0 everywhere
    scales = [127 + j for j in range(8)]        # block j: 2^j
    rope = [0.0] * 64
    rope[0], rope[63] = 1.5, -3.0
    got = oracle.packed584_to_f64(assemble(codes, scales, rope))
    for d in range(448):
        assert got[d] == 2.0 ** (d // 56), d
    assert got[448] == 1.5 and got[511] == -3.0 and not got[449:511].any()
    raw = assemble(codes, scales, rope)
    assert raw[448] == 0xC0 and raw[449] == 0x3F        # 1.5 = 0x3FC0, low byte first
    assert list(raw[576:]) == scales


def test_batched_decode_matches_row_by_row():
    p = W.packed_rows(37, seed=4).numpy()
    whole = oracle.packed584_to_f64(p)
    for r in range(37):
        assert np.array_equal(whole[r], oracle.packed584_to_f64(p[r]))
    assert oracle.decode_bits(p, "packed_fp8_584").shape == (37, 512)


def test_generated_rows_are_what_the_writer_meant():
    """The pool generator's rows decode to within E4M3 rounding (relative
    2^-4) of the N(0,1) values scaled per block, RoPE exactly BF16 of them,
    and every NoPE value is exactly representable in BF16 (so the decode
    equals a BF16 row: the kernels widen to BF16 without rounding)."""
    import torch
    p = W.packed_rows(64, seed=9).numpy()
    v = oracle.packed584_to_f64(p)
    assert np.isfinite(v).all()
    assert np.array_equal(oracle.round_to_bf16(v), v)
    scales = oracle.ue8m0_to_f64(p[:, 576:])
    assert ((p[:, 576:] >= 1) & (p[:, 576:] <= 254)).all()
    # each block's largest magnitude is within the E4M3 range times its scale
    mags = np.abs(v[:, :448]).reshape(64, 8, 56).max(-1)
    assert (mags <= 448 * scales).all()


def single_slot_case(kv_rows, row, b2):
    q = np.zeros((1, 4, 512), np.uint16)
    idx = np.full((1, 200), -1, np.int32)
    idx[0, 150] = row
    return oracle.sparse_mla_decode(q, "bf16", kv_rows[:1], kv_rows, "packed_fp8_584",
                                    idx, None, None, 0.3, b2, 1.0)


def test_single_slot_returns_the_decoded_row():
    """One active slot, no sink: out = bmm2 * row (closed form), whatever q."""
    p = W.packed_rows(10, seed=2).numpy()
    ref = single_slot_case(p, 7, 0.5)
    want = 0.5 * oracle.packed584_to_f64(p[7])
    for h in range(4):
        assert np.array_equal(ref["out"][0, h], want)
    assert np.all(ref["lse"][0] == 0.0)        # a single logit of q=0: log2(1)


def test_packed_decode_equals_the_bf16_decode_of_the_same_values():
    """The method on packed rows is the method on their decoded values: the
    same call with the rows re-expressed as BF16 bit patterns (exact, as the
    test above shows) gives identical results."""
    rng = np.random.default_rng(5)
    swa = W.packed_rows(300, seed=11).numpy()
    comp = W.packed_rows(400, seed=12).numpy()
    T, H, K = 3, 8, 260
    idx = np.concatenate([rng.integers(0, 300, (T, 128)),
                          rng.integers(0, 400, (T, K - 128))], 1).astype(np.int32)
    idx[1, ::5] = -1
    lens = np.array([260, 200, 129], np.int32)
    q = W.raw_bits(W.normal_rows(T * H, 13).view(T, H, 512))
    sinks = rng.standard_normal(H).astype(np.float32)

    def bits_of(rows):
        v = oracle.packed584_to_f64(rows).astype(np.float32)
        return (v.view(np.uint32) >> 16).astype(np.uint16)
    a = oracle.sparse_mla_decode(q, "bf16", swa, comp, "packed_fp8_584", idx, lens,
                                 sinks, 0.04, 1.0, 1.0)
    b = oracle.sparse_mla_decode(q, "bf16", bits_of(swa), bits_of(comp), "bf16", idx,
                                 lens, sinks, 0.04, 1.0, 1.0)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_packed_decode_matches_the_multiset_brute_force():
    rng = np.random.default_rng(6)
    swa = W.packed_rows(40, seed=21).numpy()
    comp = W.packed_rows(50, seed=22).numpy()
    T, H, K = 2, 2, 140
    idx = np.concatenate([rng.integers(0, 40, (T, 128)),
                          rng.integers(0, 50, (T, K - 128))], 1).astype(np.int32)
    idx[0, 3] = -1
    q = W.raw_bits(W.normal_rows(T * H, 23).view(T, H, 512))
    sinks = np.array([0.3, -1.2], np.float32)
    ref = oracle.sparse_mla_decode(q, "bf16", swa, comp, "packed_fp8_584", idx,
                                   np.array([140, 131], np.int32), sinks, 0.05, 1.0, 1.0)
    bf_out, bf_lse = brute_force_decode(q, "bf16", swa, comp, "packed_fp8_584", idx,
                                        np.array([140, 131], np.int32), sinks, 0.05,
                                        1.0, 1.0)
    assert np.allclose(ref["out"], bf_out, rtol=1e-12, atol=1e-14)
    assert np.allclose(ref["lse"], bf_lse, rtol=0, atol=1e-12)


def test_empty_token_with_packed_rows():
    """A token with no active slot gives out = 0 and lse = the sink's own
    term (or -inf without a sink), with packed pools as with any other."""
    swa = W.packed_rows(8, seed=31).numpy()
    q = np.zeros((2, 3, 512), np.uint16)
    idx = np.full((2, 130), -1, np.int32)
    idx[1, 2] = 5
    sinks = np.array([0.5, -1.0, 2.0], np.float32)
    for sk in (sinks, None):
        ref = oracle.sparse_mla_decode(q, "bf16", swa, swa, "packed_fp8_584", idx,
                                       np.array([0, 130], np.int32), sk, 0.1, 1.0, 1.0)
        assert ref["out"].shape == (2, 3, 512) and not ref["out"][0].any()
        if sk is None:
            assert np.all(np.isneginf(ref["lse"][0]))
        else:
            assert np.allclose(ref["lse"][0], sinks.astype(np.float64) / math.log(2.0))


@pytest.mark.parametrize("mistake", ["block64", "big_endian", "bias128", "scale_first"])
def test_planted_layout_mistakes_fail(mistake):
    """Plausible misreadings of the layout, planted in a copy of the decode,
    are caught by the hand-assembled row."""
    rng = np.random.default_rng(1)
    codes = [int(c) for c in rng.integers(0, 0x70, 448)]
    scales = [127 + j - 3 for j in range(8)]
    rope = [float(v) for v in (np.arange(64) - 20) / 8.0]
    row = assemble(codes, scales, rope)
    want = oracle.packed584_to_f64(row)
    b = row
    nope = oracle.e4m3fn_bits_to_f64(b[:448])
    if mistake == "block64":
        sc = oracle.ue8m0_to_f64(b[576:583])
        bad_nope = nope * np.repeat(sc, 64)
        rope_v = oracle.bf16_bits_to_f64(b[448:576:2].astype(np.uint16)
                                         | (b[449:576:2].astype(np.uint16) << 8))
    else:
        off_r, off_s = (448, 576) if mistake != "scale_first" else (456, 448)
        sc = oracle.ue8m0_to_f64(b[off_s:off_s + 8]) if mistake != "bias128" else \
            np.ldexp(1.0, b[576:584].astype(np.int64) - 128)
        bad_nope = nope * np.repeat(sc, 56)
        lo, hi = b[off_r:off_r + 128:2].astype(np.uint16), b[off_r + 1:off_r + 128:2].astype(np.uint16)
        rope_v = oracle.bf16_bits_to_f64((lo << 8) | hi if mistake == "big_endian" else lo | (hi << 8))
    bad = np.concatenate([bad_nope, rope_v])
    assert not np.array_equal(bad, want)
