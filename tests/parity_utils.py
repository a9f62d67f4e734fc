"""Helpers shared by the GPU parity tests: moving the rows a set of tokens
touches to the host for the oracle, and comparing GPU results with it."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

# tolerances stated for the decode: |out - ref| <= atol + rtol*|ref|, and an
# absolute bound on the base-2 LSE
TOL_BF16 = (1e-2, 1e-2)
TOL_FP8 = (3e-2, 3e-2)
LSE_ATOL = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    L.load()      # fails loudly if the HIP library is missing


def host_case(w: W.Workload, tokens):
    """The oracle's inputs for ``tokens`` of a GPU-resident workload: q,
    and compact host pools holding only the rows those tokens name, with
    the table re-indexed into them (-1 and out-of-range stay untouched)."""
    tok = torch.as_tensor(list(tokens), dtype=torch.long)
    idx = w.indices.cpu()[tok].numpy().astype(np.int64)
    lens = None if w.topk_lens is None else w.topk_lens.cpu()[tok].numpy()
    out_idx = idx.copy()
    pools = []
    for sl, pool in ((slice(0, 128), w.swa_pool), (slice(128, None), w.comp_pool)):
        part = idx[:, sl]
        ok = (part >= 0) & (part < (0 if pool is None else pool.shape[0]))
        uniq = np.unique(part[ok])
        if pool is None or len(uniq) == 0:
            # a stand-in row in the workload's row format (never indexed)
            if w.kv_dtype == W.PACKED:
                dt, width = torch.uint8, W.PACKED_ROW_BYTES
            else:
                dt, width = (torch.bfloat16 if w.kv_dtype == W.BF16
                             else torch.float8_e4m3fn), 512
            pools.append(W.raw_bits(torch.zeros((1, width), dtype=dt)))
            continue
        rows = pool[torch.as_tensor(uniq, device=pool.device)]
        pools.append(W.raw_bits(rows))
        remapped = part.copy()
        remapped[ok] = np.searchsorted(uniq, part[ok])
        out_idx[:, sl] = remapped
    return dict(q_bits=W.raw_bits(w.q[tok.to(w.q.device)]), q_dtype=w.q_dtype,
                swa_bits=pools[0], comp_bits=pools[1], kv_dtype=w.kv_dtype,
                indices=out_idx.astype(np.int32), topk_lens=lens,
                sinks=None if w.sinks is None else w.sinks.cpu().numpy())


def oracle_for(w: W.Workload, tokens):
    case = host_case(w, tokens)
    return oracle.sparse_mla_decode(bmm1_scale=w.bmm1_scale,
                                    bmm2_scale=w.bmm2_scale,
                                    lse_scale=w.lse_scale, **case)


def compare(out, lse, ref, tol, tokens=None, what=""):
    """Element-wise check of GPU out/out_lse against the oracle."""
    atol, rtol = tol
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy().astype(np.float64)
    if tokens is not None:
        o, l = o[list(tokens)], l[list(tokens)]
    ro, rl = ref["out"], ref["lse"]
    assert o.shape == ro.shape and l.shape == rl.shape, \
        f"{what}: shapes {o.shape}/{l.shape} vs oracle {ro.shape}/{rl.shape}"
    # The oracle's outputs are finite; a NaN or an infinity on the GPU side
    # (an element never written into a NaN-filled buffer, a head that came
    # out NaN) must fail, so the test is "not within the bound" rather than
    # "beyond the bound" (every comparison with NaN is false).
    assert np.all(np.isfinite(ro)), f"{what}: oracle output not finite"
    err = np.abs(o - ro)
    bound = atol + rtol * np.abs(ro)
    bad = ~(err <= bound)
    if bad.any():
        score = np.where(bad, np.where(np.isfinite(err), err - bound, np.inf), -np.inf)
        i = np.unravel_index(np.argmax(score), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance or not "
            f"finite; worst at {i}: gpu {o[i]!r} oracle {ro[i]!r}")
    assert not np.isnan(l).any(), f"{what}: NaN in the GPU LSE"
    assert np.array_equal(np.isneginf(l), np.isneginf(rl)), f"{what}: -inf LSE mismatch"
    assert np.array_equal(np.isposinf(l), np.isposinf(rl)), f"{what}: +inf LSE mismatch"
    fin = np.isfinite(rl)
    lerr = np.abs(l[fin] - rl[fin])
    lbad = ~(lerr <= LSE_ATOL)
    assert not lbad.any(), \
        f"{what}: {lbad.sum()} LSEs off by more than {LSE_ATOL} (or not finite)"
    return float(err.max()), float(lerr.max()) if lerr.size else 0.0


def same_bits(a: torch.Tensor, b: torch.Tensor, what=""):
    """a and b hold identical bits, and a holds no NaN.  Outputs start out
    NaN-filled, so an element no kernel wrote is NaN and must not pass as
    equal to another unwritten element (-inf, an empty token's LSE, is a
    value and is allowed)."""
    assert a.shape == b.shape, f"{what}: shapes {tuple(a.shape)} vs {tuple(b.shape)}"
    assert not torch.isnan(a.float()).any(), f"{what}: NaN (unwritten or invalid) output"
    iv = {2: torch.int16, 4: torch.int32}[a.element_size()]
    assert torch.equal(a.view(iv), b.view(iv)), f"{what}: bits differ"


def run_decode(w, plan=None, flags=0, workspace=None, out_lse=True):
    out = torch.full((w.T, w.H, 512), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((w.T, w.H), float("nan"), dtype=torch.float32,
                     device="cuda") if out_lse else None
    L.decode(w.q, w.swa_pool, w.comp_pool, w.indices, out, out_lse=lse,
             topk_lens=w.topk_lens, seq_lens=w.seq_lens,
             cum_seq_lens_q=w.cum_seq_lens_q, sinks=w.sinks,
             bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
             lse_scale=w.lse_scale, plan=plan, flags=flags,
             workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def log(msg):
    print(msg, flush=True)


LOG2E = 1.0 / math.log(2.0)
