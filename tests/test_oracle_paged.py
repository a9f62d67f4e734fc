"""Pins of the oracle's page-table form (CPU only).

The page-table form (FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4``:
the HCA paragraph of the introduction and the parameters
``hca_swa_indices``, ``swa_topk_lens``, ``hca_compressed_block_tables``,
``sparse_topk_lens``, ``hca_sparse_indices_format``) names a token's window
rows directly and its compressed rows by pages: slot j of the compressed
stream is row page[j / page_size] * page_size + j % page_size.  What fixes
the expected values here: the multiset brute force with its own page
expansion (50 digits), the two-segment form fed the expanded table, closed
forms, page-order invariance, and split-K over the virtual columns.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.formats import decode_bits
from test_oracle_pins import bf16_bits, fp8_bits

D = 512


def paged_case(seed, T=3, H=3, K1=16, pages=5, ps=8, swa_rows=40, n_pages=30,
               dtype="bf16", sinks=True, lens="random"):
    rng = np.random.default_rng(seed)
    enc = bf16_bits if dtype == "bf16" else fp8_bits
    ks = 1.0 if dtype == "bf16" else 1 / 0.08
    q = enc(rng.standard_normal((T, H, D)) * 0.15 * (1 if dtype == "bf16" else 8))
    swa = enc(rng.standard_normal((swa_rows, D)) * ks)
    comp = enc(rng.standard_normal((n_pages * ps, D)) * ks)
    si = rng.integers(0, swa_rows, (T, K1)).astype(np.int32) if K1 else None
    bt = np.stack([rng.permutation(n_pages)[:pages] for _ in range(T)]).astype(np.int32) \
        if pages else None
    if lens == "random":
        sl = rng.integers(0, K1 + 1, T).astype(np.int32)
        tot = (sl + rng.integers(0, pages * ps + 1, T)).astype(np.int32)
    else:
        sl, tot = lens
    sk = rng.standard_normal(H).astype(np.float32) if sinks else None
    return dict(q_bits=q, q_dtype=dtype, swa_bits=swa, comp_bits=comp, kv_dtype=dtype,
                swa_indices=si, block_tables=bt, page_size=ps, swa_topk_lens=sl,
                topk_lens=tot, sinks=sk)


def run(case, b1=0.07, b2=1.0, g=1.0):
    return oracle.sparse_mla_decode_paged(bmm1_scale=b1, bmm2_scale=b2, lse_scale=g,
                                          **case)


def close(a, b, tol=1e-12):
    fa, fb = np.isfinite(a["lse"]), np.isfinite(b["lse"])
    assert np.array_equal(fa, fb)
    np.testing.assert_allclose(a["lse"][fa], b["lse"][fb], rtol=tol, atol=tol)
    np.testing.assert_allclose(a["out"], b["out"], rtol=tol, atol=tol)


def expand(bt, ps):
    """The canonical expansion written out with numpy (independent of the
    oracle's loop): row = page * ps + offset, pages in table order."""
    return (bt[:, :, None] * ps + np.arange(ps)[None, None, :]).reshape(bt.shape[0], -1)


@pytest.mark.parametrize("seed,dtype,K1,pages,ps,sinks", [
    (40, "bf16", 16, 5, 8, True), (41, "bf16", 0, 3, 16, False),
    (42, "fp8_e4m3fn", 9, 4, 4, True), (43, "bf16", 128, 2, 8, True),
    (44, "bf16", 12, 0, 8, False),
])
def test_brute_force_multiset(seed, dtype, K1, pages, ps, sinks):
    case = paged_case(seed, dtype=dtype, K1=K1, pages=pages, ps=ps, sinks=sinks,
                      swa_rows=40 if K1 < 128 else 140)
    b1, b2, g = 0.0625, 0.75, 1.5
    ref = run(case, b1, b2, g)
    out, lse = oracle.brute_force_decode_paged(
        case["q_bits"], dtype, case["swa_bits"], case["comp_bits"], dtype,
        case["swa_indices"], case["block_tables"], ps, case["swa_topk_lens"],
        case["topk_lens"], case["sinks"], b1, b2, g)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(ref["lse"]))
    np.testing.assert_allclose(ref["lse"][fin], lse[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["out"], out, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed", [50, 51])
def test_equals_the_expanded_two_segment_form(seed):
    """The page table is a compact spelling of an extra table: expanding
    it (numpy, above) and giving the extra length total - window reproduces
    the result exactly."""
    case = paged_case(seed, K1=20, pages=6, ps=8)
    ext = expand(case["block_tables"], 8).astype(np.int32)
    el = np.clip(case["topk_lens"] - case["swa_topk_lens"], 0, ext.shape[1]).astype(np.int32)
    a = run(case)
    b = oracle.sparse_mla_decode_segments(
        case["q_bits"], "bf16", case["swa_bits"], case["comp_bits"], "bf16",
        case["swa_indices"], ext, case["swa_topk_lens"], el, case["sinks"], 0.07, 1.0, 1.0)
    assert np.array_equal(a["n_active"], b["n_active"])
    close(a, b, 0.0)


def test_single_compressed_slot_closed_form():
    """No window, one visible compressed slot: it is slot 0 of the first
    page, row page0 * ps; out = beta2 * row, lse = gamma * s * log2(e)."""
    case = paged_case(60, T=1, H=2, K1=4, pages=3, ps=8, sinks=False,
                      lens=(np.array([0], np.int32), np.array([1], np.int32)))
    case["block_tables"][0] = [7, 2, 5]
    b1, b2, g = 0.05, 0.5, 2.0
    r = run(case, b1, b2, g)
    row = decode_bits(case["comp_bits"][7 * 8], "bf16")
    q = decode_bits(case["q_bits"][0], "bf16")
    np.testing.assert_array_equal(r["out"][0], np.broadcast_to(b2 * row, (2, D)))
    s = np.float32(b1).astype(np.float64) * (q @ row)
    np.testing.assert_allclose(r["lse"][0], g * s / math.log(2.0), rtol=1e-14)
    assert oracle.active_slots_paged(np.zeros(4, np.int32), 0, np.array([7, 2, 5]), 8, 10)[-1] \
        == (4 + 9, 1, 2 * 8 + 1)


def test_whole_pages_in_any_order():
    """With every slot of every page visible, the order of the pages in the
    table only permutes the slots."""
    case = paged_case(61, K1=10, pages=4, ps=8, lens="random")
    case["topk_lens"] = (case["swa_topk_lens"] + 32).astype(np.int32)
    perm = dict(case, block_tables=case["block_tables"][:, ::-1].copy())
    close(run(case), run(perm), 1e-13)


def test_window_and_total_lengths():
    """Window length 0 and total = window give the compressed stream alone
    and the window alone; a total below the window clamps to no compressed
    slot; both empty give 0 and -inf."""
    case = paged_case(62, K1=16, pages=3, ps=8, sinks=False)
    T = 3
    w0 = run(dict(case, swa_topk_lens=np.zeros(T, np.int32), topk_lens=np.full(T, 24, np.int32)))
    only_c = oracle.sparse_mla_decode_paged(
        case["q_bits"], "bf16", case["swa_bits"], case["comp_bits"], "bf16", None,
        case["block_tables"], 8, None, np.full(T, 24, np.int32), None, 0.07, 1.0, 1.0)
    close(w0, only_c, 0.0)
    sl = np.array([16, 5, 9], np.int32)
    a = run(dict(case, swa_topk_lens=sl, topk_lens=sl))
    b = run(dict(case, swa_topk_lens=sl, topk_lens=np.array([0, 1, 2], np.int32)))
    assert np.array_equal(a["n_active"], sl) and np.array_equal(b["n_active"], sl)
    close(a, b, 0.0)
    e = run(dict(case, swa_topk_lens=np.zeros(T, np.int32), topk_lens=np.zeros(T, np.int32)))
    assert np.all(e["out"] == 0) and np.all(np.isneginf(e["lse"]))


def test_split_form_over_virtual_columns():
    case = paged_case(63, T=2, K1=70, pages=5, ps=64, n_pages=12, swa_rows=80)
    ref = run(case)
    K = 70 + 5 * 64
    b1 = float(np.float32(0.07))
    for S in (2, 3, 6):
        ranges = oracle.split_columns(K, S, 64)
        for t in range(2):
            slots = oracle.active_slots_paged(case["swa_indices"][t], case["swa_topk_lens"][t],
                                              case["block_tables"][t], 64, case["topk_lens"][t])
            rows = oracle.sparse_mla.gather_rows(slots, case["swa_bits"], case["comp_bits"], "bf16")
            q_t = decode_bits(case["q_bits"][t], "bf16")
            mo, ml = oracle.split_partials(q_t, slots, rows, ranges, b1, 1.0)
            out, lse = oracle.combine(mo, ml, case["sinks"], 1.0)
            np.testing.assert_allclose(out, ref["out"][t], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse, ref["lse"][t], rtol=1e-12, atol=1e-12)
