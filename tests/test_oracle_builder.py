"""Pins of the oracle's combined-table builder (CPU only).

The builder (vLLM ``DeepseekV4FlashInferMLAAttention._build_sparse_index_metadata``
feeding FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4``'s
``sparse_indices`` / ``sparse_topk_lens``) translates local compressed
positions through a block table with the canonical page expansion of the
FlashInfer page (``hca_sparse_indices_format``).  What fixes the expected
values here: the page-table form's own, independently written expansion
(a token whose local positions are 0..n-1 in order must give exactly the
page-table form's slots, and decoding both gives the same result), a
worked example, invariants (bijection per request, permutation
equivariance), and the special cases the readings name.
"""

import numpy as np

import oracle
from oracle.index_builder import build_combined_indices
from test_oracle_pins import bf16_bits

D = 512


def test_worked_example():
    # page_size 4, request 0 owns pages [7, 2]: position 0 -> 7*4+0,
    # 5 -> page 2, offset 1 -> 9, 3 -> 31, -1 stays, 6 -> 2*4+2 = 10
    idx, lens, bad = build_combined_indices(
        np.array([[11]]), np.array([[0, 5, 3, -1, 6]]), local=True, page_size=4,
        block_tables=np.array([[7, 2]]))
    assert idx.tolist() == [[11, 28, 9, 31, -1, 10]]
    assert lens.tolist() == [6] and bad == []


def test_in_order_positions_equal_the_page_table_form():
    rng = np.random.default_rng(3)
    T, W, pages, ps = 4, 128, 6, 16
    swa = rng.integers(-1, 500, (T, W))
    bt = np.stack([rng.permutation(40)[:pages] for _ in range(T)]).astype(np.int32)
    n = pages * ps
    comp = np.tile(np.arange(n), (T, 1))
    n2 = rng.integers(0, n + 1, T)
    idx, lens, bad = build_combined_indices(swa, comp, local=True, page_size=ps,
                                            block_tables=bt, comp_topk_lens=n2)
    assert bad == []
    for t in range(T):
        ref = oracle.active_slots_paged(swa[t], None, bt[t], ps, W + int(n2[t]))
        comp_ref = [r for (c, pool, r) in ref if pool == 1]
        assert idx[t, W:W + n2[t]].tolist() == comp_ref
        assert (idx[t, W + n2[t]:] == -1).all()
        assert idx[t, :W].tolist() == swa[t].tolist()
        assert lens[t] == W + n2[t]


def test_decoding_the_built_table_equals_the_page_table_decode():
    rng = np.random.default_rng(5)
    T, H, W, pages, ps, n_pages = 3, 4, 128, 3, 16, 12
    swa_rows = 300
    q = bf16_bits(rng.standard_normal((T, H, D)) * 0.15)
    swa_bits = bf16_bits(rng.standard_normal((swa_rows, D)))
    comp_bits = bf16_bits(rng.standard_normal((n_pages * ps, D)))
    swa = np.stack([rng.choice(swa_rows, W, replace=False) for _ in range(T)])
    swa[0, 5] = -1
    bt = np.stack([rng.permutation(n_pages)[:pages] for _ in range(T)]).astype(np.int32)
    n2 = np.array([pages * ps, 17, 0])
    comp = np.tile(np.arange(pages * ps), (T, 1))
    idx, lens, _ = build_combined_indices(swa, comp, local=True, page_size=ps,
                                          block_tables=bt, comp_topk_lens=n2)
    sinks = rng.standard_normal(H).astype(np.float32)
    common = dict(q_bits=q, q_dtype="bf16", swa_bits=swa_bits, comp_bits=comp_bits,
                  kv_dtype="bf16", sinks=sinks, bmm1_scale=0.05, bmm2_scale=1.0,
                  lse_scale=1.0)
    a = oracle.sparse_mla_decode(indices=idx, topk_lens=lens, **common)
    b = oracle.sparse_mla_decode_paged(swa_indices=swa.astype(np.int32),
                                       block_tables=bt, page_size=ps,
                                       swa_topk_lens=None,
                                       topk_lens=(W + n2).astype(np.int32), **common)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13, atol=1e-13)


def test_global_entries_pass_through_with_their_lengths():
    rng = np.random.default_rng(7)
    swa = rng.integers(0, 99, (3, 5))
    comp = rng.integers(-1, 1000, (3, 9))
    n2 = np.array([9, 4, 12])          # the last one is clamped to K2 = 9
    idx, lens, bad = build_combined_indices(swa, comp, local=False, comp_topk_lens=n2)
    assert bad == []
    assert lens.tolist() == [14, 9, 14]
    for t in range(3):
        m = min(n2[t], 9)
        assert idx[t, 5:5 + m].tolist() == np.where(comp[t, :m] < 0, -1, comp[t, :m]).tolist()
        assert (idx[t, 5 + m:] == -1).all()


def test_positions_of_one_request_map_one_to_one_onto_its_pages():
    rng = np.random.default_rng(9)
    ps, pages = 8, 5
    bt = np.array([rng.permutation(50)[:pages]], dtype=np.int32)
    perm = rng.permutation(pages * ps)
    idx, _, _ = build_combined_indices(np.zeros((1, 0), np.int64), perm[None, :],
                                       local=True, page_size=ps, block_tables=bt)
    rows = idx[0].tolist()
    assert len(set(rows)) == pages * ps
    assert set(rows) == {int(p) * ps + o for p in bt[0] for o in range(ps)}
    # permuting the positions permutes the rows the same way
    idx2, _, _ = build_combined_indices(np.zeros((1, 0), np.int64),
                                        np.arange(pages * ps)[None, :], local=True,
                                        page_size=ps, block_tables=bt)
    assert rows == idx2[0][perm].tolist()


def test_tokens_share_their_request_block_table():
    bt = np.array([[3, 1], [0, 2]], dtype=np.int32)
    comp = np.array([[0, 5], [0, 5], [7, 2]])
    idx, _, _ = build_combined_indices(np.zeros((3, 0), np.int64), comp, local=True,
                                       page_size=4, block_tables=bt,
                                       token_to_req=np.array([0, 0, 1]))
    assert idx.tolist() == [[12, 5], [12, 5], [11, 2]]


def test_untranslatable_positions_are_masked_and_reported():
    bt = np.array([[4, -3]], dtype=np.int32)
    comp = np.array([[1, 5, 9, -7]])     # page 0 ok, page 1 negative, page 2 past
    idx, lens, bad = build_combined_indices(np.array([[2]]), comp, local=True,
                                            page_size=4, block_tables=bt)
    assert idx.tolist() == [[2, 17, -1, -1, -1]]
    assert lens.tolist() == [5]
    assert bad == [(0, 2), (0, 3)]
    big = np.array([[0x7FFFFFFF // 4 + 1]], dtype=np.int32)
    idx, _, bad = build_combined_indices(np.zeros((1, 0), np.int64), np.array([[0]]),
                                         local=True, page_size=4, block_tables=big)
    assert idx.tolist() == [[-1]] and bad == [(0, 0)]


def test_invalid_tokens_are_empty_and_decode_to_the_sink_only_result():
    idx, lens, _ = build_combined_indices(
        np.array([[3, 4], [5, 6]]), np.array([[0], [1]]), local=True, page_size=2,
        block_tables=np.array([[1], [2]]), valid_tokens=np.array([1, 0]))
    assert idx.tolist() == [[3, 4, 2], [-1, -1, -1]]
    assert lens.tolist() == [3, 0]
    rng = np.random.default_rng(1)
    H = 2
    q = bf16_bits(rng.standard_normal((2, H, D)))
    pool = bf16_bits(rng.standard_normal((8, D)))
    sinks = np.array([0.5, -1.0], np.float32)
    r = oracle.sparse_mla_decode(q, "bf16", pool, pool, "bf16", idx, lens, sinks,
                                 0.05, 1.0, 1.0)
    assert (r["out"][1] == 0).all()
    np.testing.assert_allclose(r["lse"][1], sinks.astype(np.float64) / np.log(2),
                               rtol=1e-6)


def test_tokens_of_requests_outside_the_block_table_are_empty_and_reported():
    bt = np.array([[1, 2]], dtype=np.int32)
    idx, lens, bad = build_combined_indices(
        np.array([[4], [5], [6]]), np.array([[0], [1], [2]]), local=True, page_size=2,
        block_tables=bt, token_to_req=np.array([0, 1, -1]))
    assert idx.tolist() == [[4, 2], [-1, -1], [-1, -1]]
    assert lens.tolist() == [2, 0, 0]
    assert bad == [(1, -1), (2, -1)]
