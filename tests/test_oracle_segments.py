"""Pins of the oracle's two-segment form (CPU only).

The two-segment form (FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4``:
introduction, packed-backend paragraph, parameters ``swa_topk_lens``,
``extra_sparse_indices``, ``extra_sparse_topk_lens``; the Cake page's
``extra_indices`` / ``extra_topk_length``) names a token's SWA rows in one
table and its compressed rows in another, each with its own length.  What
fixes the expected values here: the multiset brute force in 50-digit
arithmetic, the combined-table form it must reduce to when the SWA table has
128 columns, closed forms for single slots, and invariants (an empty
segment, swapping the tables' roles over one shared pool, split-K).
"""

import math

import numpy as np
import pytest

import oracle
from oracle.formats import decode_bits
from test_oracle_pins import bf16_bits, fp8_bits

D = 512


def seg_case(seed, T=3, H=3, K1=7, K2=45, swa_rows=30, comp_rows=50,
             dtype="bf16", neg=4, sinks=True, lens="random", qscale=0.15):
    rng = np.random.default_rng(seed)
    enc = bf16_bits if dtype == "bf16" else fp8_bits
    ks = 1.0 if dtype == "bf16" else 1 / 0.08
    q = enc(rng.standard_normal((T, H, D)) * qscale * (1 if dtype == "bf16" else 8))
    swa = enc(rng.standard_normal((swa_rows, D)) * ks)
    comp = enc(rng.standard_normal((comp_rows, D)) * ks)
    si = rng.integers(0, swa_rows, (T, K1)).astype(np.int32) if K1 else None
    ei = rng.integers(0, comp_rows, (T, K2)).astype(np.int32) if K2 else None
    for tab, K in ((si, K1), (ei, K2)):
        if tab is not None:
            for t in range(T):
                tab[t, rng.choice(K, min(neg, K), replace=False)] = -1
    if lens == "random":
        sl = rng.integers(0, K1 + 1, T).astype(np.int32) if K1 else None
        el = rng.integers(0, K2 + 1, T).astype(np.int32) if K2 else None
    else:
        sl, el = lens
    sk = rng.standard_normal(H).astype(np.float32) if sinks else None
    return dict(q_bits=q, q_dtype=dtype, swa_bits=swa, comp_bits=comp, kv_dtype=dtype,
                swa_indices=si, extra_indices=ei, swa_topk_lens=sl,
                extra_topk_lens=el, sinks=sk)


def run(case, b1=0.07, b2=1.0, g=1.0):
    return oracle.sparse_mla_decode_segments(bmm1_scale=b1, bmm2_scale=b2,
                                             lse_scale=g, **case)


def close(a, b, tol=1e-12):
    fa, fb = np.isfinite(a["lse"]), np.isfinite(b["lse"])
    assert np.array_equal(fa, fb)
    np.testing.assert_allclose(a["lse"][fa], b["lse"][fb], rtol=tol, atol=tol)
    np.testing.assert_allclose(a["out"], b["out"], rtol=tol, atol=tol)


@pytest.mark.parametrize("seed,dtype,K1,K2,sinks", [
    (10, "bf16", 7, 45, True), (11, "bf16", 0, 40, False), (12, "bf16", 33, 0, True),
    (13, "fp8_e4m3fn", 5, 60, True), (14, "bf16", 130, 20, False),
])
def test_brute_force_multiset(seed, dtype, K1, K2, sinks):
    """Independent formulation: multiset of (pool, row) over both tables,
    evaluated without max subtraction in 50 digits."""
    case = seg_case(seed, dtype=dtype, K1=K1, K2=K2, sinks=sinks,
                    swa_rows=40 if K1 < 130 else 140)
    b1, b2, g = 0.0625, 0.75, 1.5
    ref = run(case, b1, b2, g)
    out, lse = oracle.brute_force_decode_segments(
        case["q_bits"], dtype, case["swa_bits"], case["comp_bits"], dtype,
        case["swa_indices"], case["extra_indices"], case["swa_topk_lens"],
        case["extra_topk_lens"], case["sinks"], b1, b2, g)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(ref["lse"]))
    np.testing.assert_allclose(ref["lse"][fin], lse[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["out"], out, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed", [20, 21, 22])
def test_reduces_to_combined_table(seed):
    """With a 128-column SWA table, the two-segment call equals the combined
    table [SWA columns (masked with -1 from swa_topk_len on) | extra
    columns] with topk_len = 128 + extra_topk_len: the same slots, in the
    same column order."""
    case = seg_case(seed, K1=128, K2=70, swa_rows=150, comp_rows=90)
    T = case["q_bits"].shape[0]
    comb = np.concatenate([case["swa_indices"], case["extra_indices"]], axis=1)
    for t in range(T):
        comb[t, case["swa_topk_lens"][t]:128] = -1
    topk = (128 + case["extra_topk_lens"]).astype(np.int32)
    a = run(case)
    b = oracle.sparse_mla_decode(case["q_bits"], "bf16", case["swa_bits"],
                                 case["comp_bits"], "bf16", comb, topk, case["sinks"],
                                 0.07, 1.0, 1.0)
    assert np.array_equal(a["n_active"], b["n_active"])
    close(a, b, 0.0)


def test_single_extra_slot_closed_form():
    """One active slot, in the extra table, no sink: out = beta2 * row and
    lse = gamma * s * log2(e) with s = beta1 <q, row>."""
    case = seg_case(30, T=1, H=2, K1=6, K2=9, sinks=False,
                    lens=(np.array([0], np.int32), np.array([1], np.int32)))
    case["extra_indices"][0, 0] = 17
    b1, b2, g = 0.05, 0.5, 2.0
    r = run(case, b1, b2, g)
    row = decode_bits(case["comp_bits"][17], "bf16")
    q = decode_bits(case["q_bits"][0], "bf16")
    np.testing.assert_array_equal(r["out"][0], np.broadcast_to(b2 * row, (2, D)))
    s = np.float32(b1).astype(np.float64) * (q @ row)
    np.testing.assert_allclose(r["lse"][0], g * s / math.log(2.0), rtol=1e-14)


def test_empty_segments():
    """A zero length (or an absent table) drops its segment: the result is
    the other segment alone; both empty gives 0 and -inf (or the sink)."""
    case = seg_case(31, K1=9, K2=33)
    T = case["q_bits"].shape[0]
    zero = np.zeros(T, np.int32)
    only_extra = dict(case, swa_topk_lens=zero)
    no_swa = dict(case, swa_indices=None, swa_topk_lens=None)
    a, b = run(only_extra), run(no_swa)
    close(a, b, 0.0)
    none = run(dict(case, swa_topk_lens=zero, extra_topk_lens=zero, sinks=None))
    assert np.all(none["out"] == 0) and np.all(np.isneginf(none["lse"]))
    sink = run(dict(case, swa_topk_lens=zero, extra_topk_lens=zero))
    np.testing.assert_allclose(sink["lse"], np.broadcast_to(
        case["sinks"].astype(np.float64) / math.log(2.0), sink["lse"].shape), rtol=1e-14)


def test_tables_swap_over_one_pool():
    """When both pools are the same array, which table names a row does not
    matter: swapping the tables (and their lengths) permutes the slots only."""
    case = seg_case(32, K1=20, K2=30, swa_rows=50, comp_rows=50)
    case["comp_bits"] = case["swa_bits"]
    sw = dict(case, swa_indices=case["extra_indices"], extra_indices=case["swa_indices"],
              swa_topk_lens=case["extra_topk_lens"], extra_topk_lens=case["swa_topk_lens"])
    close(run(case), run(sw), 1e-13)


def test_split_form_over_virtual_columns():
    """Split-K over the virtual row of K1 + K2 columns: combining the
    partials of every split equals the unsplit result."""
    case = seg_case(33, T=2, K1=70, K2=200, swa_rows=80, comp_rows=220, lens="random")
    ref = run(case)
    K = 270
    for S in (1, 2, 3, 5):
        ranges = oracle.split_columns(K, S, 64)
        for t in range(2):
            slots = oracle.active_slots_segments(
                case["swa_indices"][t], case["swa_topk_lens"][t],
                case["extra_indices"][t], case["extra_topk_lens"][t])
            rows = oracle.sparse_mla.gather_rows(slots, case["swa_bits"],
                                                 case["comp_bits"], "bf16")
            q_t = decode_bits(case["q_bits"][t], "bf16")
            b1 = float(np.float32(0.07))   # scales cross the boundary as binary32
            mo, ml = oracle.split_partials(q_t, slots, rows, ranges, b1, 1.0)
            out, lse = oracle.combine(mo, ml, case["sinks"], 1.0)
            np.testing.assert_allclose(out, ref["out"][t], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, ref["lse"][t], rtol=1e-12, atol=1e-12)


def test_columns_are_virtual():
    """Extra slot j sits at column K1 + j, after every SWA slot."""
    slots = oracle.active_slots_segments(np.array([3, -1, 5], np.int32), 3,
                                         np.array([7, 8, -1, 9], np.int32), 2)
    assert slots == [(0, 0, 3), (2, 0, 5), (3, 1, 7), (4, 1, 8)]
