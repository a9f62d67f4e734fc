"""An independent second formulation, for pinning the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Instead of walking the table slot by slot, this version first turns a
token's active slots into a multiset of pool rows: k_r = how many active
slots name row r of a given pool.  Each distinct row then contributes
k_r * e^{s_r} to the normaliser and k_r * e^{s_r} * row_r to the numerator,
with no max-subtraction, evaluated in mpmath at 50 significant digits
(mpmath's exponent range does not overflow).  Dot products of decoded inputs
are computed exactly: every product of two BF16/E4M3 values is exact in
binary64, and math.fsum returns the correctly rounded sum.

It is slow, pure-Python, and only meant for tiny inputs (a handful of
tokens and heads, pools of a few dozen rows).
"""

from __future__ import annotations

import math
from collections import Counter

import mpmath
import numpy as np

from .formats import decode_bits

_SWA = 128


def _combined_multiset(indices, topk_lens, t):
    """Multiset of (pool, row) named by token t's active slots of a combined
    table (columns < 128 name SWA rows)."""
    K = indices.shape[1]
    n = K if topk_lens is None else int(topk_lens[t])
    mult = Counter()
    for c in range(K):
        if c >= n:
            break
        r = int(indices[t][c])
        if r != -1:
            mult[(0 if c < _SWA else 1, r)] += 1
    return mult


def _segments_multiset(swa_indices, swa_lens, extra_indices, extra_lens, t):
    """Multiset of (pool, row) named by token t's active slots of an SWA
    table and an extra (compressed) table, each with its own length."""
    mult = Counter()
    for pool, tab, lens in ((0, swa_indices, swa_lens), (1, extra_indices, extra_lens)):
        if tab is None:
            continue
        n = tab.shape[1] if lens is None else int(lens[t])
        for c in range(min(n, tab.shape[1])):
            r = int(tab[t][c])
            if r != -1:
                mult[(pool, r)] += 1
    return mult


def _paged_multiset(swa_indices, swa_lens, block_tables, page_size, total_lens, t):
    """Multiset of (pool, row) of token t in the page-table form: its
    visible window rows, then compressed rows numbered page by page."""
    mult = Counter()
    k1 = 0 if swa_indices is None else swa_indices.shape[1]
    w = k1 if swa_lens is None else max(0, min(int(swa_lens[t]), k1))
    for c in range(w):
        r = int(swa_indices[t][c])
        if r != -1:
            mult[(0, r)] += 1
    if block_tables is None:
        return mult
    pages = [int(x) for x in block_tables[t]]
    cap = len(pages) * page_size
    n = cap if total_lens is None else max(0, min(int(total_lens[t]) - w, cap))
    done = 0
    for pg in pages:
        for off in range(page_size):
            if done == n:
                return mult
            mult[(1, pg * page_size + off)] += 1
            done += 1
    return mult


def brute_force_decode_paged(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                             swa_indices, block_tables, page_size, swa_lens,
                             total_lens, sinks, bmm1_scale, bmm2_scale,
                             lse_scale, dps: int = 50):
    """The page-table form by the same multiset evaluation.  Returns
    (out, lse)."""
    return _brute(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                  lambda t: _paged_multiset(swa_indices, swa_lens, block_tables,
                                            page_size, total_lens, t),
                  sinks, bmm1_scale, bmm2_scale, lse_scale, dps)


def brute_force_decode(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                       indices, topk_lens, sinks, bmm1_scale, bmm2_scale,
                       lse_scale, dps: int = 50):
    """Returns (out [T,H,D] float64, lse [T,H] float64)."""
    return _brute(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                  lambda t: _combined_multiset(indices, topk_lens, t),
                  sinks, bmm1_scale, bmm2_scale, lse_scale, dps)


def brute_force_decode_segments(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                                swa_indices, extra_indices, swa_lens, extra_lens,
                                sinks, bmm1_scale, bmm2_scale, lse_scale,
                                dps: int = 50):
    """The two-segment form (SWA table + extra compressed table, one length
    each) by the same multiset evaluation.  Returns (out, lse)."""
    return _brute(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype,
                  lambda t: _segments_multiset(swa_indices, swa_lens,
                                               extra_indices, extra_lens, t),
                  sinks, bmm1_scale, bmm2_scale, lse_scale, dps)


def _brute(q_bits, q_dtype, swa_bits, comp_bits, kv_dtype, multiset_of,
           sinks, bmm1_scale, bmm2_scale, lse_scale, dps):
    b1 = mpmath.mpf(float(np.float32(bmm1_scale)))
    b2 = mpmath.mpf(float(np.float32(bmm2_scale)))
    g = mpmath.mpf(float(np.float32(lse_scale)))
    T, H, D = q_bits.shape
    q = decode_bits(q_bits, q_dtype)
    out = np.zeros((T, H, D))
    lse = np.zeros((T, H))
    with mpmath.workdps(dps):
        for t in range(T):
            mult = multiset_of(t)
            rows = {}
            for (pool, r) in mult:
                src = swa_bits if pool == 0 else comp_bits
                rows[(pool, r)] = [float(v) for v in decode_bits(src[r], kv_dtype)]
            for h in range(H):
                qh = [float(v) for v in q[t, h]]
                z = mpmath.mpf(0)
                num = [mpmath.mpf(0)] * D
                for key, k in mult.items():
                    row = rows[key]
                    dot = math.fsum(a * b for a, b in zip(qh, row))
                    wgt = k * mpmath.exp(b1 * mpmath.mpf(dot))
                    z += wgt
                    num = [acc + wgt * mpmath.mpf(v) for acc, v in zip(num, row)]
                if sinks is not None:
                    z += mpmath.exp(mpmath.mpf(float(np.float32(sinks[h]))))
                if z == 0:
                    out[t, h] = 0.0
                    lse[t, h] = -math.inf
                    continue
                out[t, h] = [float(b2 * v / z) for v in num]
                lse[t, h] = float(g * mpmath.log(z, 2))
    return out, lse
