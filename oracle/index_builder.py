"""Combined index table from decode metadata (CPU oracle; TEST INFRASTRUCTURE
ONLY, like the rest of this package).

The step before the decode: vLLM's DeepSeek-V4 FlashInfer attention
(``DeepseekV4FlashInferMLAAttention._build_sparse_index_metadata``) turns a
decode token's SWA window rows and its compressed top-k positions into the
combined table and per-token lengths that FlashInfer's
``trtllm_batch_decode_sparse_mla_dsv4`` consumes (``sparse_indices``,
``sparse_topk_lens``: the first columns index the SWA pool, the rest the
compressed pool, -1 masks a slot, the length counts the SWA columns).  For
compress ratio 4 the compressed positions are local to the request
(``decode_compressed_indices_are_local``) and are translated through the
request's compressed block table, whose pages hold
``block_size // compress_ratio`` compressed rows; for ratio 128 they are
global rows with their own lengths (``c128a_decode_topk_lens``).  The
translation of a local position is the canonical page expansion the
FlashInfer page states for ``hca_sparse_indices_format``:
``page_id * page_size + page_offset``.

The pages give the builder's arguments, not its code.  Readings (the
plainest the rest supports):
  * The SWA columns are copied as they come (decode SWA indices are rows of
    the SWA pool; -1 stays -1).
  * A negative compressed entry gives -1.  A local position p maps to row
    ``block_tables[req][p // page_size] * page_size + p % page_size``; a
    position whose page index is past the table's width, a negative page
    id, or a row that does not fit an int32 gives -1 and is reported.
  * Compressed columns at or past the token's compressed length are -1; the
    token's length is ``W + n2`` with ``n2`` the compressed length clamped to
    [0, K2] (``K2`` when no lengths are given), ``W`` the SWA width.
  * A token marked invalid (padding) gets an all -1 row and length 0, and so
    does (local form) a token whose request index lies outside the block
    table; the latter is reported with column -1.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def build_combined_indices(swa_indices: np.ndarray, comp_indices: np.ndarray, *,
                           local: bool, page_size: Optional[int] = None,
                           block_tables: Optional[np.ndarray] = None,
                           token_to_req: Optional[np.ndarray] = None,
                           comp_topk_lens: Optional[np.ndarray] = None,
                           valid_tokens: Optional[np.ndarray] = None):
    """Returns (indices int32 [T, W + K2], topk_lens int32 [T], bad) where
    ``bad`` lists the (token, column) pairs whose local position could not be
    translated (they hold -1).

    swa_indices [T, W] and comp_indices [T, K2] are int32 (W or K2 may be 0);
    block_tables [B, max_pages] int32; token_to_req [T] (None: token t uses
    request t); comp_topk_lens [T] (None: K2); valid_tokens [T] (None: all).
    """
    swa = np.asarray(swa_indices, dtype=np.int64)
    comp = np.asarray(comp_indices, dtype=np.int64)
    T, W = swa.shape
    K2 = comp.shape[1]
    assert comp.shape[0] == T
    out = np.full((T, W + K2), -1, dtype=np.int64)
    lens = np.zeros(T, dtype=np.int64)
    bad = []
    for t in range(T):
        if valid_tokens is not None and not valid_tokens[t]:
            continue
        req = t if token_to_req is None else int(token_to_req[t])
        if local and K2 > 0 and not 0 <= req < block_tables.shape[0]:
            bad.append((t, -1))
            continue
        n2 = K2 if comp_topk_lens is None else int(comp_topk_lens[t])
        n2 = max(0, min(n2, K2))
        lens[t] = W + n2
        out[t, :W] = swa[t]
        for j in range(n2):
            p = int(comp[t, j])
            if p < 0:
                continue
            if not local:
                out[t, W + j] = p
                continue
            blk = p // page_size
            if blk >= block_tables.shape[1]:
                bad.append((t, W + j))
                continue
            page = int(block_tables[req, blk])
            row = page * page_size + p % page_size
            if page < 0 or row > 0x7FFFFFFF:
                bad.append((t, W + j))
                continue
            out[t, W + j] = row
    return out.astype(np.int32), lens.astype(np.int32), bad
