"""The C-ABI library on the host (CPU only, no kernel is ever launched).

Covers: the library loads and exports every function include/sparsemla.h
declares; status strings; the split planner's bounds and determinism;
workspace sizing; and every host-side argument check of sparse_mla_decode /
sparse_mla_combine.  The argument checks use non-null dummy pointer values
with exactly one violation each, so every call is rejected before anything
would be launched.
"""

import ctypes
import json
import os

import pytest

from sparse_mla_decode_gather_amd import lib as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "pages_constants.json")


@pytest.fixture(scope="module")
def so():
    return L.load()


def test_every_declared_symbol_is_exported(so):
    names = L.header_functions()
    assert set(names) == {
        "sparse_mla_plan_splits", "sparse_mla_workspace_size",
        "sparse_mla_workspace_layout", "sparse_mla_decode",
        "sparse_mla_gather_only", "sparse_mla_decode_segments",
        "sparse_mla_decode_paged", "sparse_mla_build_indices",
        "sparse_mla_combine", "sparse_mla_get_device_error",
        "sparse_mla_status_string", "sparse_mla_decode_noalloc"}
    for n in names:
        assert hasattr(so, n), n


def test_status_strings(so):
    for code in range(9):
        assert L.status_string(code) not in ("", "unknown status")
    assert L.status_string(99) == "unknown status"


def test_pages_constants_match_header():
    with open(os.path.join(L.INCLUDE, "sparsemla.h")) as f:
        hdr = f.read()
    c = json.load(open(GOLDEN))
    assert f"SMLA_SWA_COLUMNS  {c['swa_columns']['value']}" in hdr
    assert f"SMLA_HEAD_DIM     {c['head_dim']['value']}" in hdr


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------

def plan(T, H=128, K=2048, q=0, kv=0, max_splits=0, override=0, cus=256):
    return L.plan_splits(T, H, K, q, kv, max_splits, override, cus)


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 64, 100, 256, 300, 512, 4096])
@pytest.mark.parametrize("H,K", [(128, 2048), (64, 1024), (128, 512), (64, 256),
                                 (128, 100), (64, 5000)])
def test_plan_bounds(T, H, K):
    p = plan(T, H, K)
    assert 1 <= p.num_splits <= 16 and p.num_splits <= p.num_chunks
    assert p.head_tiles in ((1, 2) if H == 128 else (1,)) and p.K == K
    assert p.num_chunks == -(-K // p.chunk_cols)
    assert p.num_splits * p.chunks_per_split * p.chunk_cols >= K
    # no split is entirely past the table
    assert (p.num_splits - 1) * p.chunks_per_split * p.chunk_cols < K
    q = plan(T, H, K)
    assert p.as_dict() == q.as_dict()


def test_plan_adapts_to_batch():
    # one chunk per block at low batch, a single chunk at high batch
    assert plan(1).num_splits == 16
    assert plan(8).num_splits >= 11      # 11 with head tiles (16 workgroups per half)
    assert plan(512).num_splits == 1
    assert plan(4096).num_splits == 1
    assert plan(1, max_splits=4).num_splits == 4


def test_plan_override_and_clamp():
    assert plan(512, override=3).num_splits == 3
    assert plan(512, K=100, override=16).num_splits == 2   # only 2 chunks
    assert plan(1, K=64 * 64, override=1000).num_splits == 64


@pytest.mark.parametrize("args,code", [
    ((-1, 128, 2048), 1), ((4, 128, 0), 1), ((4, 96, 2048), 3),
    ((4, 256, 2048), 3),
])
def test_plan_rejects(args, code, so):
    p = L.Plan()
    assert so.sparse_mla_plan_splits(*args, 0, 0, 0, 0, 256,
                                     ctypes.byref(p)) == code
    assert so.sparse_mla_plan_splits(4, 128, 2048, 1, 0, 0, 0, 256,
                                     ctypes.byref(p)) == 2   # FP8 q, BF16 KV


def test_workspace_sizes():
    p1 = plan(512)
    assert L.workspace_size(p1, 512, 128) == 0
    assert L.workspace_size(p1, 512, 128, L.FLAG_VALIDATE_INDICES) == 256
    p = plan(8)
    S = p.num_splits
    lse_off, out_off = L.workspace_layout(p, 8, 128)
    assert lse_off == 256 and out_off % 256 == 0
    assert out_off >= lse_off + 8 * 128 * S * 4
    assert L.workspace_size(p, 8, 128) == out_off + 8 * 128 * S * 512 * 2


# ---------------------------------------------------------------------------
# argument validation of sparse_mla_decode (rejected before any launch)
# ---------------------------------------------------------------------------

DUMMY = 0x7f0000000000      # 256-B aligned, never dereferenced


def good_args(T=4, H=128, K=256):
    a = L.DecodeArgs()
    a.T, a.H, a.K = T, H, K
    a.q_dtype = a.kv_dtype = 0
    a.q = a.swa_pool = a.compressed_pool = a.out = DUMMY
    a.indices = DUMMY
    a.swa_rows, a.compressed_rows = 1024, 4096
    a.bmm1_scale, a.bmm2_scale, a.lse_scale = 0.04, 1.0, 1.0
    return a


def call(so, a, p=None, T=None):
    if p is None:
        p = plan(max(a.T if T is None else T, 1),
                 a.H if a.H in (64, 128) else 128, max(a.K, 1))
    return so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None)


@pytest.mark.parametrize("field,value,code", [
    ("T", -1, 1), ("K", 0, 1), ("H", 96, 3), ("H", 256, 3),
    ("q", None, 1), ("swa_pool", None, 1), ("indices", None, 1),
    ("out", None, 1), ("compressed_pool", None, 1),
    ("swa_rows", -5, 1), ("q_dtype", 1, 2), ("kv_dtype", 3, 2),
    ("q", DUMMY + 8, 5), ("out", DUMMY + 2, 5), ("swa_pool", DUMMY + 4, 5),
    ("compressed_pool", DUMMY + 8, 5), ("indices", DUMMY + 2, 5),
    ("pool_row_stride", 500, 1), ("pool_row_stride", 516, 5),
    ("index_row_stride", 100, 1), ("cum_seq_lens_q", DUMMY, 1),
])
def test_decode_rejects(so, field, value, code):
    a = good_args()
    setattr(a, field, value)
    assert call(so, a) == code


@pytest.mark.parametrize("field,value", [
    ("bmm1_scale", 0.0), ("bmm1_scale", -0.04), ("bmm1_scale", float("nan")),
    ("bmm1_scale", float("inf")), ("bmm1_scale", 3.0e38),
    ("bmm2_scale", float("nan")), ("bmm2_scale", float("-inf")),
    ("lse_scale", float("inf")), ("lse_scale", float("nan")),
])
def test_decode_rejects_bad_scales(so, field, value):
    """The QK scale must be positive and finite (the kernels scale the raw
    tile max, which needs a positive scale; times log2(e) it must stay a
    finite float); the other two must be finite.  Every table form checks
    them before anything is launched."""
    a = good_args()
    setattr(a, field, value)
    assert call(so, a) == 1
    a = seg_args()
    setattr(a, field, value)
    assert call_seg(so, a, good_segments()) == 1
    a = paged_args()
    setattr(a, field, value)
    assert call_paged(so, a, good_paged()) == 1


def test_decode_accepts_small_and_negative_free_scales(so):
    """Scales that are allowed reach the plan check (forced to fail here so
    that nothing is launched): a tiny positive bmm1, negative bmm2 and
    lse_scale."""
    a = good_args()
    a.bmm1_scale, a.bmm2_scale, a.lse_scale = 1e-30, -2.0, -0.5
    p = plan(4, 128, 256)
    p.K = 999
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 6


def test_noalloc_host_checks(so):
    """sparse_mla_decode_noalloc refuses a workspace and the validate flag,
    and a call whose partials exceed its scratch, before any device work;
    zero tokens do nothing."""
    assert so.sparse_mla_decode_noalloc(None, None, None) == 1
    a = good_args(T=512, K=2048)
    p = plan(512, 128, 2048, override=16)
    assert L.workspace_size(p, 512, 128) > L.NOALLOC_SCRATCH_BYTES
    assert so.sparse_mla_decode_noalloc(ctypes.byref(a), ctypes.byref(p), None) == 8
    a.workspace, a.workspace_bytes = DUMMY, 1 << 30
    assert so.sparse_mla_decode_noalloc(ctypes.byref(a), ctypes.byref(p), None) == 1
    a.workspace, a.workspace_bytes = None, 0
    a.flags = L.FLAG_VALIDATE_INDICES
    assert so.sparse_mla_decode_noalloc(ctypes.byref(a), ctypes.byref(p), None) == 1
    a = good_args(T=0)
    assert so.sparse_mla_decode_noalloc(ctypes.byref(a), ctypes.byref(plan(1, 128, 256)),
                                        None) == 0
    a = good_args()
    a.bmm1_scale = 0.0
    assert so.sparse_mla_decode_noalloc(ctypes.byref(a), ctypes.byref(plan(4, 128, 256)),
                                        None) == 1


def test_packed_rows_argument_checks(so):
    """Packed 584-byte rows: only with BF16 q; the row stride is in bytes,
    0 meaning 584, at least 584 and a multiple of 8.  Calls that pass the
    checks are stopped at a forced plan mismatch (nothing is launched)."""
    pk = L.DTYPE_PACKED_FP8_584
    a = good_args()
    a.kv_dtype = pk
    p = plan(4, 128, 256, kv=pk)
    p.K = 999
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 6
    for stride, code in ((584, 6), (592, 6), (583, 1), (512, 1), (588, 5)):
        a.pool_row_stride = stride
        assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == code, stride
    a.pool_row_stride = 0
    a.q_dtype = L.DTYPE_FP8_E4M3FN
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 2
    # the planner takes the pair too, and rejects FP8 q with packed rows
    assert L.plan_splits(512, 128, 2048, 0, pk, num_cus=256).num_splits >= 1
    q = L.Plan()
    assert so.sparse_mla_plan_splits(4, 128, 256, 1, pk, 0, 0, 256, ctypes.byref(q)) == 2
    # gather_only serves BF16 rows only
    a = good_args()
    a.kv_dtype = pk
    assert call_gather(so, a) == 2


def test_decode_null_args_and_empty_batch(so):
    assert so.sparse_mla_decode(None, None, None) == 1
    a = good_args(T=0)
    a.q = a.out = None         # nothing is touched for T = 0
    p = plan(1, 128, 256)
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 0


def test_decode_swa_only_allows_null_compressed_pool(so):
    a = good_args(K=128)
    a.compressed_pool = None
    a.workspace = None
    p = plan(4, 128, 128)
    # the only thing left to fail is a plan mismatch, which we force here
    p.K = 64
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 6


def test_decode_workspace_checks(so):
    a = good_args(T=8, K=2048)
    p = plan(8, 128, 2048)
    assert p.num_splits > 1
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 4
    a.workspace = DUMMY
    a.workspace_bytes = L.workspace_size(p, 8, 128) - 1
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 4
    a.workspace_bytes += 1
    a.workspace = DUMMY + 128
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 5
    # validation needs the error block even without splits
    a = good_args(T=512, K=2048)
    a.flags = L.FLAG_VALIDATE_INDICES
    p = plan(512, 128, 2048)
    assert p.num_splits == 1
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 4


@pytest.mark.parametrize("mutate", [
    lambda p: setattr(p, "num_splits", 0),
    lambda p: setattr(p, "num_splits", 65),
    lambda p: setattr(p, "chunk_cols", 0),
    lambda p: setattr(p, "K", 999),
    lambda p: setattr(p, "chunks_per_split", 1),   # no longer covers K
    # spans that would overflow the kernels' 32-bit column numbers
    lambda p: (setattr(p, "num_splits", 4), setattr(p, "chunk_cols", 1 << 29),
               setattr(p, "chunks_per_split", 2)),
    lambda p: (setattr(p, "num_splits", 64), setattr(p, "chunk_cols", 1 << 25),
               setattr(p, "chunks_per_split", 1)),
    lambda p: (setattr(p, "num_splits", 1), setattr(p, "chunk_cols", 2),
               setattr(p, "chunks_per_split", (1 << 29) + 1)),
    lambda p: setattr(p, "head_tiles", 0),
    lambda p: setattr(p, "head_tiles", 3),
])
def test_decode_rejects_bad_plan(so, mutate):
    a = good_args(T=4, K=2048)
    p = plan(512, 128, 2048)
    mutate(p)
    assert so.sparse_mla_decode(ctypes.byref(a), ctypes.byref(p), None) == 6


@pytest.mark.parametrize("args,code", [
    ((4, 128, 0, 4), 1), ((4, 128, 65, 65), 1), ((4, 128, 4, 3), 1),
    ((4, 96, 4, 4), 3), ((-1, 128, 4, 4), 1),
])
def test_combine_rejects(so, args, code):
    T, H, S, stride = args
    assert so.sparse_mla_combine(DUMMY, DUMMY, T, H, S, stride, None, 1.0,
                                 DUMMY, None, None) == code


def test_combine_rejects_non_finite_lse_scale(so):
    for v in (float("nan"), float("inf")):
        assert so.sparse_mla_combine(DUMMY, DUMMY, 4, 128, 4, 4, None, v,
                                     DUMMY, None, None) == 1


def test_plan_rejects_too_wide_tables(so):
    p = L.Plan()
    assert so.sparse_mla_plan_splits(4, 128, (1 << 30) + 1, 0, 0, 0, 0, 256,
                                     ctypes.byref(p)) == 1
    assert so.sparse_mla_plan_splits(4, 128, 1 << 30, 0, 0, 0, 0, 256,
                                     ctypes.byref(p)) == 0


def test_combine_rejects_null_and_misaligned(so):
    assert so.sparse_mla_combine(None, DUMMY, 4, 128, 2, 2, None, 1.0, DUMMY,
                                 None, None) == 1
    assert so.sparse_mla_combine(DUMMY + 8, DUMMY, 4, 128, 2, 2, None, 1.0,
                                 DUMMY, None, None) == 5
    assert so.sparse_mla_combine(DUMMY, DUMMY, 0, 128, 2, 2, None, 1.0, None,
                                 None, None) == 0


def test_get_device_error_rejects_null(so):
    assert so.sparse_mla_get_device_error(None, None, None, None, None) == 1


# ---------------------------------------------------------------------------
# sparse_mla_gather_only: decode's checks, no outputs, H=128 BF16 only
# ---------------------------------------------------------------------------

def call_gather(so, a, p=None):
    if p is None:
        p = plan(max(a.T, 1), a.H if a.H in (64, 128) else 128, max(a.K, 1))
    return so.sparse_mla_gather_only(ctypes.byref(a), ctypes.byref(p), None)


@pytest.mark.parametrize("field,value,code", [
    ("T", -1, 1), ("K", 0, 1), ("H", 96, 3), ("q", None, 1), ("indices", None, 1),
    ("compressed_pool", None, 1), ("q", DUMMY + 8, 5), ("indices", DUMMY + 2, 5),
    ("pool_row_stride", 500, 1), ("index_row_stride", 100, 1),
    ("H", 64, 3), ("q_dtype", 1, 2), ("kv_dtype", 1, 2),
])
def test_gather_only_rejects(so, field, value, code):
    a = good_args()
    setattr(a, field, value)
    if field == "q_dtype":
        a.kv_dtype = 1        # FP8/FP8 is a valid decode pair, not a gather-only one
    assert call_gather(so, a) == code


def test_gather_only_needs_no_outputs_and_checks_the_plan(so):
    assert so.sparse_mla_gather_only(None, None, None) == 1
    a = good_args(T=0)
    a.out = None
    assert call_gather(so, a) == 0
    a = good_args(T=4, K=2048)
    a.out = a.workspace = None
    p = plan(4, 128, 2048)
    p.K = 1024
    assert call_gather(so, a, p) == 6


# ---------------------------------------------------------------------------
# sparse_mla_decode_segments: the two-segment tables
# ---------------------------------------------------------------------------

def good_segments(K1=128, K2=1920):
    g = L.Segments()
    g.swa_indices = DUMMY if K1 else None
    g.extra_indices = DUMMY + 4096 if K2 else None
    g.swa_width, g.extra_width = K1, K2
    return g


def seg_args(T=4, K1=128, K2=1920):
    a = good_args(T=T, K=K1 + K2)
    a.indices = None
    return a


def call_seg(so, a, g, p=None):
    if p is None:
        p = plan(max(a.T, 1), a.H if a.H in (64, 128) else 128, max(a.K, 1))
    return so.sparse_mla_decode_segments(ctypes.byref(a), ctypes.byref(g),
                                         ctypes.byref(p), None)


def bad_plan(a):
    p = plan(max(a.T, 1), 128, max(a.K, 1))
    p.K += 64      # rejected after every argument check
    return p


@pytest.mark.parametrize("K1,K2", [(128, 1920), (0, 300), (77, 0), (5, 61), (200, 5000)])
def test_segments_pass_the_argument_checks(so, K1, K2):
    a, g = seg_args(K1=K1, K2=K2), good_segments(K1, K2)
    if K1 == 0:
        a.swa_pool = None          # not needed without an SWA table
    if K2 == 0:
        a.compressed_pool = None   # nor the compressed pool without extras
    assert call_seg(so, a, g, bad_plan(a)) == 6


@pytest.mark.parametrize("change,code", [
    ("null_seg", 1), ("widths", 1), ("neg_width", 1), ("indices_set", 1),
    ("topk_set", 1), ("no_swa_table", 1), ("no_extra_table", 1),
    ("no_swa_pool", 1), ("no_comp_pool", 1), ("swa_stride", 1),
    ("extra_stride", 1), ("swa_misaligned", 5), ("extra_misaligned", 5),
])
def test_segments_rejects(so, change, code):
    a, g = seg_args(), good_segments()
    if change == "null_seg":
        p = plan(4, 128, a.K)
        assert so.sparse_mla_decode_segments(ctypes.byref(a), None, ctypes.byref(p),
                                             None) == code
        return
    if change == "widths":
        g.extra_width = 1900
    elif change == "neg_width":
        g.swa_width, g.extra_width = -1, 2049
    elif change == "indices_set":
        a.indices = DUMMY
    elif change == "topk_set":
        a.topk_lens = DUMMY
    elif change == "no_swa_table":
        g.swa_indices = None
    elif change == "no_extra_table":
        g.extra_indices = None
    elif change == "no_swa_pool":
        a.swa_pool = None
    elif change == "no_comp_pool":
        a.compressed_pool = None
    elif change == "swa_stride":
        g.swa_row_stride = 100
    elif change == "extra_stride":
        g.extra_row_stride = 1000
    elif change == "swa_misaligned":
        g.swa_indices = DUMMY + 2
    elif change == "extra_misaligned":
        g.extra_indices = DUMMY + 6
    assert call_seg(so, a, g) == code


def test_segments_zero_tokens_and_null_args(so):
    g = good_segments()
    assert so.sparse_mla_decode_segments(None, ctypes.byref(g), None, None) == 1
    a = seg_args(T=0)
    assert call_seg(so, a, g) == 0


# ---------------------------------------------------------------------------
# sparse_mla_decode_paged: window rows + compressed page table
# ---------------------------------------------------------------------------

def good_paged(K1=128, pages=30, ps=64):
    g = L.Paged()
    g.swa_indices = DUMMY if K1 else None
    g.block_tables = DUMMY + 8192 if pages else None
    g.swa_width, g.max_pages, g.page_size = K1, pages, ps
    return g


def paged_args(T=4, K1=128, pages=30, ps=64):
    a = good_args(T=T, K=K1 + pages * ps)
    a.indices = None
    return a


def call_paged(so, a, g, p=None):
    if p is None:
        p = plan(max(a.T, 1), a.H if a.H in (64, 128) else 128, max(a.K, 1))
    return so.sparse_mla_decode_paged(ctypes.byref(a), ctypes.byref(g), ctypes.byref(p), None)


@pytest.mark.parametrize("K1,pages,ps", [(128, 30, 64), (0, 5, 64), (128, 0, 64), (7, 3, 1),
                                         (100, 9, 37)])
def test_paged_pass_the_argument_checks(so, K1, pages, ps):
    a, g = paged_args(K1=K1, pages=pages, ps=ps), good_paged(K1, pages, ps)
    if K1 == 0:
        a.swa_pool = None
    if pages == 0:
        a.compressed_pool = None
    a.topk_lens = DUMMY            # the window + compressed count is allowed here
    assert call_paged(so, a, g, bad_plan(a)) == 6


@pytest.mark.parametrize("change,code", [
    ("null", 1), ("K", 1), ("page_size", 1), ("neg_pages", 1), ("neg_width", 1),
    ("indices_set", 1), ("no_swa_table", 1), ("no_block_table", 1), ("no_comp_pool", 1),
    ("swa_stride", 1), ("block_stride", 1), ("huge", 1), ("block_misaligned", 5),
])
def test_paged_rejects(so, change, code):
    a, g = paged_args(), good_paged()
    if change == "null":
        p = plan(4, 128, a.K)
        assert so.sparse_mla_decode_paged(ctypes.byref(a), None, ctypes.byref(p), None) == code
        return
    if change == "K":
        a.K += 1
    elif change == "page_size":
        g.page_size = 0
    elif change == "neg_pages":
        g.max_pages = -1
    elif change == "neg_width":
        g.swa_width = -3
    elif change == "indices_set":
        a.indices = DUMMY
    elif change == "no_swa_table":
        g.swa_indices = None
    elif change == "no_block_table":
        g.block_tables = None
    elif change == "no_comp_pool":
        a.compressed_pool = None
    elif change == "swa_stride":
        g.swa_row_stride = 127
    elif change == "block_stride":
        g.block_table_stride = 29
    elif change == "huge":
        g.max_pages, g.page_size = 1 << 20, 1 << 12
        a.K = 128
    elif change == "block_misaligned":
        g.block_tables = DUMMY + 2
    assert call_paged(so, a, g) == code


# ---------------------------------------------------------------------------
# sparse_mla_build_indices
# ---------------------------------------------------------------------------

def good_build(T=4, W=128, K2=64, local=True):
    b = L.BuildArgs()
    b.T, b.swa_width, b.comp_width, b.comp_local = T, W, K2, 1 if local else 0
    b.swa_indices = DUMMY if W else None
    b.comp_indices = DUMMY + 4096 if K2 else None
    b.block_tables = DUMMY + 8192 if local else None
    b.max_blocks, b.page_size, b.num_requests = 8, 16, T
    b.out_indices = DUMMY + 16384
    b.out_topk_lens = DUMMY + 32768
    return b


def test_build_null_args_and_empty_batch(so):
    assert so.sparse_mla_build_indices(None, None) == 1
    b = good_build(T=0)
    b.out_indices = b.out_topk_lens = None     # never touched for T = 0
    b.swa_indices = b.comp_indices = b.block_tables = None
    assert so.sparse_mla_build_indices(ctypes.byref(b), None) == 0


@pytest.mark.parametrize("change,code", [
    ("neg_T", 1), ("neg_width", 1), ("neg_comp", 1), ("zero_width", 1),
    ("no_swa", 1), ("no_comp", 1), ("no_out", 1), ("no_lens", 1),
    ("swa_stride", 1), ("comp_stride", 1), ("out_stride", 1),
    ("no_block_table", 1), ("max_blocks", 1), ("page_size", 1), ("num_requests", 1),
    ("block_stride", 1), ("misaligned_out", 5), ("misaligned_err", 5),
    ("misaligned_req", 5),
])
def test_build_rejects(so, change, code):
    b = good_build()
    if change == "neg_T":
        b.T = -1
    elif change == "neg_width":
        b.swa_width = -1
    elif change == "neg_comp":
        b.comp_width = -2
    elif change == "zero_width":
        b.swa_width = b.comp_width = 0
    elif change == "no_swa":
        b.swa_indices = None
    elif change == "no_comp":
        b.comp_indices = None
    elif change == "no_out":
        b.out_indices = None
    elif change == "no_lens":
        b.out_topk_lens = None
    elif change == "swa_stride":
        b.swa_row_stride = 127
    elif change == "comp_stride":
        b.comp_row_stride = 63
    elif change == "out_stride":
        b.out_row_stride = 191
    elif change == "no_block_table":
        b.block_tables = None
    elif change == "max_blocks":
        b.max_blocks = 0
    elif change == "page_size":
        b.page_size = 0
    elif change == "num_requests":
        b.num_requests = 0
    elif change == "block_stride":
        b.block_table_stride = 7
    elif change == "misaligned_out":
        b.out_indices = DUMMY + 2
    elif change == "misaligned_err":
        b.err = DUMMY + 1
    elif change == "misaligned_req":
        b.token_to_req = DUMMY + 3
    assert so.sparse_mla_build_indices(ctypes.byref(b), None) == code


# ---------------------------------------------------------------------------
# flags
# ---------------------------------------------------------------------------

def test_flags_unknown_bits_and_serial_pipeline_forms(so):
    """Flag bits other than the defined ones are rejected; the serialized
    tile pipeline (an LDS-race check) is offered on the combined-table
    decode only, not with the two-segment or page-table forms or the
    gather-only call."""
    a = good_args()
    a.flags = 4
    assert call(so, a) == 1
    a.flags = L.FLAG_SERIAL_PIPELINE | L.FLAG_VALIDATE_INDICES
    assert call(so, a, bad_plan(a)) == 6          # every argument check passed
    s, g = seg_args(), good_segments()
    s.flags = L.FLAG_SERIAL_PIPELINE
    assert call_seg(so, s, g, bad_plan(s)) == 1
    pa, pg = paged_args(), good_paged(128, 30, 64)
    pa.topk_lens = DUMMY
    pa.flags = L.FLAG_SERIAL_PIPELINE
    assert call_paged(so, pa, pg, bad_plan(pa)) == 1
    ga = good_args()
    ga.flags = L.FLAG_SERIAL_PIPELINE
    assert call_gather(so, ga) == 1


@pytest.mark.parametrize("T,H,K,kv,S,HT", [
    (4, 64, 256, 0, 4, 1),        # tiny
    (64, 128, 512, 0, 1, 2),      # batched with sinks: head tiles, no split
    (128, 64, 1024, 1, 2, 1),     # FP8 q and rows
    (1, 128, 2048, 0, 16, 2), (4, 128, 2048, 0, 16, 2), (8, 128, 2048, 0, 11, 2),
    (16, 128, 2048, 0, 8, 2), (32, 128, 2048, 0, 4, 2), (64, 128, 2048, 0, 4, 1),
    (96, 128, 2048, 0, 2, 1), (128, 128, 2048, 0, 1, 2), (512, 128, 2048, 0, 1, 1),
    (512, 128, 2048, 1, 1, 1),    # speculative decode (FP8 rows, BF16 q)
    (16, 128, 512, 1, 4, 2),      # FP8 rows plan by row count, not bytes
    (64, 128, 2048, 1, 4, 1), (16, 128, 2048, 1, 8, 2),
    # H=64, BF16 q and rows: one four-wave workgroup per CU
    (16, 64, 2048, 0, 11, 1), (64, 64, 512, 0, 2, 1), (128, 64, 1024, 0, 2, 1),
    (512, 64, 2048, 0, 1, 1),
])
def test_plan_picks_on_a_256_cu_device(T, H, K, kv, S, HT):
    """The planner's picks for the benchmarked shapes on a 256-CU device
    (each the fastest or within ~2% of the fastest forced plan measured on
    MI355X; the cost model is deterministic, so these are exact)."""
    q = 1 if (kv == 1 and H == 64) else 0
    p = plan(T, H, K, q=q, kv=kv, cus=256)
    assert (p.num_splits, p.head_tiles) == (S, HT)


@pytest.mark.parametrize("kv", [0, 1, 2])
def test_plan_large_batches_keep_one_workgroup_per_token(kv):
    """From T=192 on (measured: head tiles lose there, their second row read
    and twice the workgroups outweigh the shorter MFMA chains) every format
    and width keeps head_tiles = 1 at H=128."""
    for K in (512, 1024, 2048, 4096):
        for T in (192, 256, 384, 512, 1024, 4096):
            assert plan(T, 128, K, q=0, kv=kv, cus=256).head_tiles == 1, (T, K)


def test_plan_head_tiles_only_at_h128_and_not_when_forced():
    """Head tiles are an H=128 choice of the planner; a forced split count
    keeps one workgroup per token and split."""
    for T in (1, 4, 16, 64, 128):
        assert plan(T, 64, 2048, cus=256).head_tiles == 1
        assert plan(T, 128, 2048, override=4, cus=256).head_tiles == 1
    assert plan(64, 128, 512, cus=256).head_tiles == 2


def test_plan_h64_depends_on_the_row_format():
    """At H=64 a BF16 row (LDS-DMA) costs half a row staged through
    registers (FP8, packed), so the same shape can get fewer splits; at
    H=128 the format does not change the plan (head tiles weigh every
    row format alike)."""
    assert plan(64, 64, 512, q=0, kv=0, cus=256).num_splits == 2
    assert plan(64, 64, 512, q=0, kv=1, cus=256).num_splits == 4
    assert plan(64, 64, 512, q=1, kv=1, cus=256).num_splits == 4
    assert plan(64, 64, 512, q=0, kv=2, cus=256).num_splits == 4
    for kv in (0, 1, 2):       # head tiles for every row format alike
        p = plan(128, 128, 1024, q=0, kv=kv, cus=256)
        assert (p.num_splits, p.head_tiles) == (1, 2)
    for kv in (0, 1, 2):
        p = plan(512, 128, 2048, q=0, kv=kv, cus=256)
        assert (p.num_splits, p.head_tiles) == (1, 1)
