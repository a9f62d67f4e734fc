"""Sparse MLA decode: the plain definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages state it
-----------------------------------------------
FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4`` (introduction): each query
token has heads of dimension 512; the first 128 columns of the combined
sparse table index the SWA pool and the remaining columns index the
compressed pool; ``sparse_topk_lens`` counts a token's active columns,
including the 128 SWA ones.  ``bmm1_scale`` is the fused scale of the QK
product and softmax, ``bmm2_scale`` the fused scale of the VO product,
``sinks`` are per-head attention-sink logits.

FlashInfer ``cake_sparse_mla_sm120_dsv4_nvfp4_decode`` (parameters
``indices``, ``topk_length``, ``attn_sink``, ``out_lse``, ``lse_scale``,
``mid_out``/``mid_lse``): -1 masks a slot; an omitted length means every slot
is valid; the sink joins the softmax normalisation; ``out_lse`` is the base-2
log-sum-exp times ``lse_scale``; split partials are a BF16 output and an
fp32 LSE per split.

vLLM ``DeepseekV4FlashInferMLAAttention`` (``__init__``/``_forward``): the
latent row is one plain BF16 or per-tensor FP8 row per KV token; with FP8,
bmm1 = softmax scale * q scale * kv scale and bmm2 = kv scale.

Definition used here, per token t and head h:

  A_t   = { c : c < len_t and idx[t, c] != -1 }          (len_t = K if None)
  row_c = SWA[idx[t,c]] if c < 128 else COMP[idx[t,c]]   (exact decoded values)
  s_c   = beta1 * <q[t,h,:], row_c>                      (natural-log units)
  Z     = sum_{c in A_t} e^{s_c} + e^{sink_h}            (sink term if given)
  out   = beta2 * sum_{c in A_t} e^{s_c} row_c / Z
  lse   = lse_scale * log2(Z)

Readings of points the pages leave open (each also listed in the design
notes): the whole 512-d row is both K and V; log2(e) is not folded into
bmm1_scale; the sink is a natural-log logit not multiplied by bmm1_scale and
carries no value row; ``out_lse`` includes the sink term; an empty A_t gives
out = 0 and lse = -inf (or the sink's own term); duplicate indices count once
per slot; ``seq_lens`` does not change the result.

Two-segment form (``sparse_mla_decode_segments``): the same definition
with A_t = the active slots of an SWA table (length swa_topk_lens[t]) and of
an extra compressed table (length extra_topk_lens[t]) together.

Page-table form (``sparse_mla_decode_paged``): the window entries of an SWA
row plus the canonical page expansion of a block-table row of the
compressed pool.

Parity status: pinned (tests/test_oracle_pins.py, and for the two-segment
and page-table forms tests/test_oracle_segments.py and
tests/test_oracle_paged.py) by an independent
multiset brute force in arbitrary precision, closed forms, invariants and
torch's float64 scaled_dot_product_attention, except that "out_lse includes
the sink" is a reading the pages do not settle (parity unpinned for that
choice; ``lse_nosink`` is returned alongside so it can be flipped).
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .formats import decode_bits

SWA_COLUMNS = 128
LN2 = math.log(2.0)


def _fp32(x: float) -> float:
    """Scalar scales cross the C boundary as binary32 values."""
    return float(np.float32(x))


def active_slots(idx_row: np.ndarray, topk_len: Optional[int]):
    """Active slots of one token, in column order, as (column, pool, row)
    with pool 0 = SWA, 1 = compressed."""
    K = int(idx_row.shape[0])
    n = K if topk_len is None else int(topk_len)
    out = []
    for c in range(min(n, K)):
        r = int(idx_row[c])
        if r == -1:
            continue
        out.append((c, 0 if c < SWA_COLUMNS else 1, r))
    return out


def active_slots_segments(swa_row, swa_len: Optional[int], extra_row,
                          extra_len: Optional[int]):
    """Active slots of one token in the two-segment form, as
    (column, pool, row): FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4``
    (introduction, packed-backend paragraph, and parameters
    ``swa_topk_lens``, ``extra_sparse_indices``, ``extra_sparse_topk_lens``)
    and the Cake page (``indices``/``topk_length`` with
    ``extra_indices``/``extra_topk_length``): the SWA table and its length
    describe the SWA segment, the extra table and its length the compressed
    segment, and the softmax runs over both.  SWA slot c keeps column c;
    extra slot j gets column K1 + j (K1 = the SWA table's width), so the
    split form cuts one row of K1 + K2 columns.  A length counts its own
    table only (None = the whole table); -1 masks a slot in either table."""
    K1 = 0 if swa_row is None else int(np.asarray(swa_row).shape[0])
    K2 = 0 if extra_row is None else int(np.asarray(extra_row).shape[0])
    n1 = K1 if swa_len is None else int(swa_len)
    n2 = K2 if extra_len is None else int(extra_len)
    out = []
    for c in range(min(n1, K1)):
        r = int(swa_row[c])
        if r != -1:
            out.append((c, 0, r))
    for j in range(min(n2, K2)):
        r = int(extra_row[j])
        if r != -1:
            out.append((K1 + j, 1, r))
    return out


def active_slots_paged(swa_row, swa_len: Optional[int], block_row,
                       page_size: int, total_len: Optional[int]):
    """Active slots of one token in the page-table form, as (column, pool,
    row): FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4`` (introduction,
    the HCA paragraph: the SWA stream takes physical token rows, the
    compressed stream physical page IDs; parameters ``hca_swa_indices``,
    ``swa_topk_lens``, ``hca_compressed_block_tables``, ``sparse_topk_lens``
    and, under ``hca_sparse_indices_format``, the canonical expansion
    page_id * page_size + page_offset).  Reading: the first ``swa_len``
    entries of the SWA row are the visible window (None = all); the token's
    compressed slots are the canonical expansion of its block-table row, in
    order, and the first ``total_len - swa_len`` of them are visible
    (``sparse_topk_lens`` counts window plus compressed slots; None = every
    slot of the table).  A -1 SWA entry masks its slot.  Compressed slot j
    has column K1 + j (K1 = the SWA row's width)."""
    K1 = 0 if swa_row is None else int(np.asarray(swa_row).shape[0])
    P = 0 if block_row is None else int(np.asarray(block_row).shape[0])
    K2 = P * int(page_size)
    n1 = K1 if swa_len is None else int(swa_len)
    n1 = max(0, min(n1, K1))
    tot = K1 + K2 if total_len is None else int(total_len)
    n2 = max(0, min(tot - n1, K2))
    out = []
    for c in range(n1):
        r = int(swa_row[c])
        if r != -1:
            out.append((c, 0, r))
    for j in range(n2):
        page = int(block_row[j // page_size])
        out.append((K1 + j, 1, page * int(page_size) + j % int(page_size)))
    return out


def gather_rows(slots, swa_bits, comp_bits, kv_dtype: str) -> np.ndarray:
    """Decoded float64 rows [n, 512] for the given active slots."""
    if not slots:
        # no rows: the decoded width (512 for every row format)
        return decode_bits(np.asarray(swa_bits)[:0], kv_dtype)
    rows = []
    for _, pool, r in slots:
        src = swa_bits if pool == 0 else comp_bits
        rows.append(src[r])
    return decode_bits(np.stack(rows), kv_dtype)


def decode_token(q_t: np.ndarray, rows: np.ndarray, sinks: Optional[np.ndarray],
                 beta1: float, beta2: float, gamma: float):
    """One token, all heads.  q_t [H,512], rows [n,512] float64.
    Returns (out [H,512], lse [H], lse_nosink [H])."""
    H = q_t.shape[0]
    n = rows.shape[0]
    s = beta1 * (q_t @ rows.T) if n else np.zeros((H, 0))
    if sinks is not None:
        sk = np.asarray(sinks, dtype=np.float64).reshape(H, 1)
        m = np.max(np.concatenate([s, sk], axis=1), axis=1, keepdims=True)
    elif n:
        m = np.max(s, axis=1, keepdims=True)
    else:
        return (np.zeros((H, q_t.shape[1])), np.full(H, -np.inf),
                np.full(H, -np.inf))
    w = np.exp(s - m)
    zs = w.sum(axis=1)
    z = zs + (np.exp(sk[:, 0] - m[:, 0]) if sinks is not None else 0.0)
    out = beta2 * (w @ rows) / z[:, None]
    lse = gamma * (m[:, 0] + np.log(z)) / LN2
    with np.errstate(divide="ignore"):
        lse_ns = gamma * (m[:, 0] + np.log(zs)) / LN2
    return out, lse, lse_ns


def sparse_mla_decode(q_bits, q_dtype: str, swa_bits, comp_bits, kv_dtype: str,
                      indices, topk_lens=None, sinks=None,
                      bmm1_scale: float = 1.0, bmm2_scale: float = 1.0,
                      lse_scale: float = 1.0,
                      tokens: Optional[Sequence[int]] = None):
    """Decode the given tokens (default: all).

    q_bits [T,H,512], swa_bits / comp_bits [rows,512] hold stored bit
    patterns (uint16 for "bf16", uint8 for "fp8_e4m3fn"); indices [T,K]
    int32; topk_lens [T] or None; sinks [H] float32 or None.  Scales are
    taken as binary32 values, as they cross the library boundary.

    Returns a dict of float64 arrays over the selected tokens:
    ``out`` [n_tok,H,512] (unrounded), ``lse`` and ``lse_nosink`` [n_tok,H],
    and ``n_active`` [n_tok].
    """
    T = q_bits.shape[0]
    tokens = range(T) if tokens is None else list(tokens)
    b1, b2, g = _fp32(bmm1_scale), _fp32(bmm2_scale), _fp32(lse_scale)
    sk = None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64)
    outs, lses, lses_ns, nact = [], [], [], []
    for t in tokens:
        ln = None if topk_lens is None else int(topk_lens[t])
        slots = active_slots(np.asarray(indices[t]), ln)
        rows = gather_rows(slots, swa_bits, comp_bits, kv_dtype)
        q_t = decode_bits(q_bits[t], q_dtype)
        o, l, lns = decode_token(q_t, rows, sk, b1, b2, g)
        outs.append(o)
        lses.append(l)
        lses_ns.append(lns)
        nact.append(len(slots))
    return {"out": np.stack(outs), "lse": np.stack(lses),
            "lse_nosink": np.stack(lses_ns), "n_active": np.array(nact)}


def sparse_mla_decode_segments(q_bits, q_dtype: str, swa_bits, comp_bits,
                               kv_dtype: str, swa_indices, extra_indices,
                               swa_topk_lens=None, extra_topk_lens=None,
                               sinks=None, bmm1_scale: float = 1.0,
                               bmm2_scale: float = 1.0, lse_scale: float = 1.0,
                               tokens: Optional[Sequence[int]] = None):
    """The two-segment form (see ``active_slots_segments``): swa_indices
    [T,K1] into the SWA pool with swa_topk_lens [T], extra_indices [T,K2]
    into the compressed pool with extra_topk_lens [T]; either table may be
    None (width 0).  Everything after the selection is ``decode_token``.
    Returns the same dict as ``sparse_mla_decode``."""
    T = q_bits.shape[0]
    tokens = range(T) if tokens is None else list(tokens)
    b1, b2, g = _fp32(bmm1_scale), _fp32(bmm2_scale), _fp32(lse_scale)
    sk = None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64)
    outs, lses, lses_ns, nact = [], [], [], []
    for t in tokens:
        slots = active_slots_segments(
            None if swa_indices is None else np.asarray(swa_indices[t]),
            None if swa_topk_lens is None else int(swa_topk_lens[t]),
            None if extra_indices is None else np.asarray(extra_indices[t]),
            None if extra_topk_lens is None else int(extra_topk_lens[t]))
        rows = gather_rows(slots, swa_bits, comp_bits, kv_dtype)
        q_t = decode_bits(q_bits[t], q_dtype)
        o, l, lns = decode_token(q_t, rows, sk, b1, b2, g)
        outs.append(o)
        lses.append(l)
        lses_ns.append(lns)
        nact.append(len(slots))
    return {"out": np.stack(outs), "lse": np.stack(lses),
            "lse_nosink": np.stack(lses_ns), "n_active": np.array(nact)}


def sparse_mla_decode_paged(q_bits, q_dtype: str, swa_bits, comp_bits,
                            kv_dtype: str, swa_indices, block_tables,
                            page_size: int, swa_topk_lens=None, topk_lens=None,
                            sinks=None, bmm1_scale: float = 1.0,
                            bmm2_scale: float = 1.0, lse_scale: float = 1.0,
                            tokens: Optional[Sequence[int]] = None):
    """The page-table form (see ``active_slots_paged``): swa_indices [T,K1]
    with swa_topk_lens [T] (visible window), block_tables [T,max_pages] of
    compressed-pool page IDs with ``page_size`` rows per page, and
    topk_lens [T] = visible window + compressed slots.  Everything after the
    selection is ``decode_token``.  Returns the same dict as
    ``sparse_mla_decode``."""
    T = q_bits.shape[0]
    tokens = range(T) if tokens is None else list(tokens)
    b1, b2, g = _fp32(bmm1_scale), _fp32(bmm2_scale), _fp32(lse_scale)
    sk = None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64)
    outs, lses, lses_ns, nact = [], [], [], []
    for t in tokens:
        slots = active_slots_paged(
            None if swa_indices is None else np.asarray(swa_indices[t]),
            None if swa_topk_lens is None else int(swa_topk_lens[t]),
            None if block_tables is None else np.asarray(block_tables[t]),
            page_size, None if topk_lens is None else int(topk_lens[t]))
        rows = gather_rows(slots, swa_bits, comp_bits, kv_dtype)
        q_t = decode_bits(q_bits[t], q_dtype)
        o, l, lns = decode_token(q_t, rows, sk, b1, b2, g)
        outs.append(o)
        lses.append(l)
        lses_ns.append(lns)
        nact.append(len(slots))
    return {"out": np.stack(outs), "lse": np.stack(lses),
            "lse_nosink": np.stack(lses_ns), "n_active": np.array(nact)}


def split_columns(K: int, num_splits: int, chunk_cols: int):
    """Column ranges of the split form: fixed-size chunks
    [j*chunk, (j+1)*chunk) with split s taking ``chunks_per_split``
    consecutive chunks (the plan the Cake page returns names
    ``num_splits`` and ``chunks_per_block``).  A split may be empty."""
    n_chunks = -(-K // chunk_cols)
    cps = -(-n_chunks // num_splits)
    ranges = []
    for s in range(num_splits):
        c0 = min(K, s * cps * chunk_cols)
        c1 = min(K, (s + 1) * cps * chunk_cols)
        ranges.append((c0, c1))
    return ranges


def split_partials(q_t: np.ndarray, slots, rows: np.ndarray, ranges,
                   beta1: float, beta2: float):
    """Split form of one token: for each column range, the partial output
    beta2 * sum e^{s_c} row_c / sum e^{s_c} and the partial base-2 LSE
    log2 sum e^{s_c}, with no sink and no lse_scale (the Cake page's
    ``mid_out`` / ``mid_lse``).  An empty range gives 0 and -inf.
    Returns (mid_out [H,S,512], mid_lse [H,S])."""
    H, D = q_t.shape
    S = len(ranges)
    mid_out = np.zeros((H, S, D))
    mid_lse = np.full((H, S), -np.inf)
    cols = np.array([c for c, _, _ in slots], dtype=np.int64)
    for s, (c0, c1) in enumerate(ranges):
        sel = np.nonzero((cols >= c0) & (cols < c1))[0] if len(cols) else []
        if len(sel) == 0:
            continue
        o, l, _ = decode_token(q_t, rows[sel], None, beta1, beta2, 1.0)
        mid_out[:, s, :] = o
        mid_lse[:, s] = l
    return mid_out, mid_lse


def combine(mid_out: np.ndarray, mid_lse: np.ndarray, sinks=None,
            lse_scale: float = 1.0):
    """Merge split partials (the combine step of the split-K path that the
    Cake and MSA pages describe): with L the largest of the partial LSEs and
    the sink's base-2 logit, w_s = 2^(lse_s - L),
    W = sum w_s + 2^(sink*log2(e) - L), out = sum w_s o_s / W and
    lse = lse_scale * (L + log2 W).  mid_out [...,S,512], mid_lse [...,S];
    sinks broadcast over the leading dims' last axis (heads)."""
    mid_out = np.asarray(mid_out, np.float64)
    mid_lse = np.asarray(mid_lse, np.float64)
    g = _fp32(lse_scale)
    terms = mid_lse
    if sinks is not None:
        sk = np.asarray(sinks, np.float32).astype(np.float64) / LN2
        sk = np.broadcast_to(sk, mid_lse.shape[:-1])[..., None]
        terms = np.concatenate([mid_lse, sk], axis=-1)
    L = np.max(terms, axis=-1, keepdims=True)
    finite = np.isfinite(L)
    Ls = np.where(finite, L, 0.0)
    with np.errstate(invalid="ignore"):
        w_all = np.where(np.isfinite(terms), np.exp2(terms - Ls), 0.0)
    w = w_all[..., : mid_lse.shape[-1]]
    W = w_all.sum(axis=-1)
    num = np.einsum("...s,...sd->...d", w, mid_out)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(W[..., None] > 0, num / np.where(W > 0, W, 1.0)[..., None],
                       0.0)
        lse = np.where(W > 0, g * (Ls[..., 0] + np.log2(np.where(W > 0, W, 1.0))),
                       -np.inf)
    return out, lse
