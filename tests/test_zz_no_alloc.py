"""sparse_mla_decode_noalloc through the C ABI: the allocation-free decode
(split partials in the library's static device scratch) against
sparse_mla_decode with a caller workspace, on two calls in a row, the second
with a smaller input, both with split plans that use the scratch, then an
unsplit call, then a call too large for the scratch (rejected on the host).
The outputs must be bit-identical to the workspace call's (same kernels),
and within the stated tolerance of the oracle."""

import ctypes

import pytest
import torch

from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import TOL_BF16, TOL_FP8, compare, log, need_gpu, oracle_for, same_bits

pytestmark = pytest.mark.gpu


def both(w, plan, what):
    """Run w through the allocation-free call and through the workspace
    call; compare bits with each other and values with the oracle."""
    log(f"[noalloc] {what}: T={w.T} H={w.H} K={w.K} plan={plan.as_dict()}")
    out = torch.full((w.T, w.H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.T, w.H), float("nan"), dtype=torch.float32, device="cuda")
    L.decode_noalloc(w.q, w.swa_pool, w.comp_pool, w.indices, out, out_lse=lse,
                     topk_lens=w.topk_lens, seq_lens=w.seq_lens, sinks=w.sinks,
                     bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                     lse_scale=w.lse_scale, plan=plan)
    torch.cuda.synchronize()
    ref_out = torch.full_like(out, float("nan"))
    ref_lse = torch.full_like(lse, float("nan"))
    ws = L.alloc_workspace(plan, w.T, w.H)
    L.decode(w.q, w.swa_pool, w.comp_pool, w.indices, ref_out, out_lse=ref_lse,
             topk_lens=w.topk_lens, seq_lens=w.seq_lens, sinks=w.sinks,
             bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
             lse_scale=w.lse_scale, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    same_bits(out, ref_out, f"{what}: out")
    same_bits(lse, ref_lse, f"{what}: lse")
    tol = TOL_FP8 if W.FP8 in (w.kv_dtype, w.q_dtype) else TOL_BF16
    e, le = compare(out, lse, oracle_for(w, range(w.T)), tol, what=what)
    log(f"[noalloc] {what}: bit-identical to the workspace call; "
        f"max|out err| {e:.3g} max|lse err| {le:.3g}")


def test_noalloc_matches_the_workspace_call():
    need_gpu()
    # first call: 8 tokens x 128 heads x 16 splits (16 MB of partials)
    big = W.make_long_context(8, "cuda")
    p1 = L.plan_splits(8, 128, 2048)
    assert p1.num_splits > 1
    assert L.workspace_size(p1, 8, 128) <= L.NOALLOC_SCRATCH_BYTES
    both(big, p1, "long-context T=8, planner split")
    # second call, smaller: tiny (4 tokens, 64 heads) at 3 splits, so the
    # scratch still holds the first call's larger partials around it
    small = W.make_tiny("cuda")
    p2 = L.plan_splits(small.T, small.H, small.K, num_splits=3)
    assert p2.num_splits == 3
    both(small, p2, "tiny, 3 splits")
    # an unsplit call needs no scratch at all
    both(small, L.plan_splits(small.T, small.H, small.K, num_splits=1), "tiny, unsplit")
    # FP8 rows (H=128, BF16 q), split again after the smaller calls
    spec = W.make_spec_decode("cuda")
    sub = W.Workload(name="spec16", T=16, H=spec.H, K=spec.K, q=spec.q[:16].contiguous(),
                     q_dtype=spec.q_dtype, swa_pool=spec.swa_pool, comp_pool=spec.comp_pool,
                     kv_dtype=spec.kv_dtype, indices=spec.indices[:16].contiguous(),
                     topk_lens=spec.topk_lens[:16].contiguous(),
                     seq_lens=spec.seq_lens, cum_seq_lens_q=None, sinks=spec.sinks,
                     bmm1_scale=spec.bmm1_scale, bmm2_scale=spec.bmm2_scale,
                     lse_scale=spec.lse_scale)
    p3 = L.plan_splits(16, 128, spec.K, L.DTYPE_BF16, L.DTYPE_FP8_E4M3FN, num_splits=4)
    both(sub, p3, "spec-decode rows 0..15, FP8 rows, 4 splits")


def test_noalloc_rejects_what_it_cannot_hold():
    """Host checks only: nothing is launched for these calls (the buffers
    are still sized and filled for the call they describe, every index
    naming row 0 of a one-row pool)."""
    need_gpu()
    so = L.load()
    T, H, K = 512, 128, 2048
    q = torch.zeros((T, H, 512), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    args = L.make_args(q, pool, pool, idx, out, bmm1_scale=0.04)
    # partials of 512 tokens x 16 splits exceed the scratch
    p = L.plan_splits(T, H, K, num_splits=16)
    assert L.workspace_size(p, T, H) > L.NOALLOC_SCRATCH_BYTES
    assert so.sparse_mla_decode_noalloc(ctypes.byref(args), ctypes.byref(p), None) == 8
    # a workspace or the validate flag is refused
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), 1024
    assert so.sparse_mla_decode_noalloc(ctypes.byref(args), ctypes.byref(p), None) == 1
    args.workspace, args.workspace_bytes = None, 0
    args.flags = L.FLAG_VALIDATE_INDICES
    assert so.sparse_mla_decode_noalloc(ctypes.byref(args), ctypes.byref(p), None) == 1
    torch.cuda.synchronize()
