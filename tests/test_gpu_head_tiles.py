"""Head tiles (a plan with head_tiles = 2, H=128 only): each token runs as
two 64-head halves on the H=64 kernel, each half gathering the token's rows.
Through the C ABI: every format pair, unsplit and split, with sinks (each
half takes its own 64 sinks) against the oracle; bitwise against the H=64
kernel run on the two halves as tokens of their own (same arithmetic); the
two-segment and page-table forms; the serialized pipeline; index
validation (errors name the real token); and the planner's own pick of head
tiles on the batched configuration."""

import numpy as np
import pytest
import torch

from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import (TOL_BF16, TOL_FP8, compare, log, need_gpu, oracle_for,
                          run_decode, same_bits)
from test_gpu_parity import custom

pytestmark = pytest.mark.gpu

PAIRS = [(W.BF16, W.BF16), (W.BF16, W.FP8), (W.FP8, W.FP8), (W.BF16, W.PACKED)]


def ht_plan(T, K, q, kv, S):
    p = L.plan_splits(T, 128, K, L.DTYPE_FP8_E4M3FN if q == W.FP8 else L.DTYPE_BF16,
                      {W.BF16: L.DTYPE_BF16, W.FP8: L.DTYPE_FP8_E4M3FN,
                       W.PACKED: L.DTYPE_PACKED_FP8_584}[kv], num_splits=S)
    p.head_tiles = 2
    return p


def ragged(T, K, seed):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 900, (T, K - 128))], 1).astype(np.int32)
    idx[rng.random((T, K)) < 0.05] = -1
    lens = rng.integers(0, K + 1, T).astype(np.int32)
    lens[0], lens[1] = K, 0
    return idx, lens


def packed_case(idx, lens, seed):
    """custom() with packed 584-byte rows in both pools."""
    w = custom(idx, lens, H=128, seed=seed)
    return W.Workload(
        name="packed", T=w.T, H=128, K=w.K, q=w.q, q_dtype=W.BF16,
        swa_pool=W.packed_rows(600, seed + 2, "cuda"),
        comp_pool=W.packed_rows(900, seed + 3, "cuda"), kv_dtype=W.PACKED,
        indices=w.indices, topk_lens=w.topk_lens, seq_lens=w.seq_lens,
        cum_seq_lens_q=None, sinks=w.sinks, bmm1_scale=w.bmm1_scale,
        bmm2_scale=1.0, lse_scale=w.lse_scale)


@pytest.mark.parametrize("q,kv", PAIRS)
@pytest.mark.parametrize("S", [1, 3])
def test_head_tiles_match_oracle(q, kv, S):
    need_gpu()
    T, K = 7, 700
    idx, lens = ragged(T, K, seed=31 + S)
    if kv == W.PACKED:
        w = packed_case(idx, lens, seed=5)
    else:
        w = custom(idx, lens, H=128, kv=kv, q=q, seed=5)
    plan = ht_plan(T, K, q, kv, S)
    log(f"[head tiles] q={q} kv={kv} T={T} K={K} plan={plan.as_dict()}")
    out, lse = run_decode(w, plan=plan)
    tol = TOL_BF16 if kv == W.BF16 else TOL_FP8
    e, le = compare(out, lse, oracle_for(w, range(T)), tol, what=f"head tiles {q}/{kv} S={S}")
    log(f"[head tiles] max|out err| {e:.3g} max|lse err| {le:.3g}")


@pytest.mark.parametrize("S", [1, 4])
def test_head_tiles_equal_the_halves_as_tokens_bitwise(S):
    """Without sinks the two halves of token t are exactly H=64 tokens 2t
    and 2t+1 with q = the halves and t's table row: same bits."""
    need_gpu()
    T, K = 9, 900
    idx, lens = ragged(T, K, seed=8)
    w = custom(idx, lens, H=128, sinks=False, seed=2)
    log(f"[head tiles] bitwise vs halves T={T} K={K} S={S}")
    a, la = run_decode(w, plan=ht_plan(T, K, W.BF16, W.BF16, S))
    halves = W.Workload(
        name="halves", T=2 * T, H=64, K=K, q=w.q.view(2 * T, 64, 512), q_dtype=W.BF16,
        swa_pool=w.swa_pool, comp_pool=w.comp_pool, kv_dtype=W.BF16,
        indices=w.indices.repeat_interleave(2, dim=0).contiguous(),
        topk_lens=w.topk_lens.repeat_interleave(2).contiguous(),
        seq_lens=w.seq_lens.repeat_interleave(2).contiguous(), cum_seq_lens_q=None,
        sinks=None, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
        lse_scale=w.lse_scale)
    b, lb = run_decode(halves, plan=L.plan_splits(2 * T, 64, K, num_splits=S))
    same_bits(a.view(2 * T, 64, 512), b, f"S={S} out")
    assert torch.equal(la.view(2 * T, 64), lb), f"S={S}: LSE bits differ"


def test_head_tiles_serial_pipeline_gives_the_same_bits():
    need_gpu()
    T, K = 6, 640
    idx, lens = ragged(T, K, seed=4)
    for q, kv in ((W.BF16, W.BF16), (W.FP8, W.FP8)):
        w = custom(idx, lens, H=128, kv=kv, q=q, seed=3)
        for S in (1, 2):
            plan = ht_plan(T, K, q, kv, S)
            log(f"[head tiles] serial pipeline q={q} kv={kv} S={S}")
            a, la = run_decode(w, plan=plan)
            b, lb = run_decode(w, plan=plan, flags=L.FLAG_SERIAL_PIPELINE)
            same_bits(a, b, f"{q}/{kv} S={S}")
            assert torch.equal(la, lb)


def test_head_tiles_validation_names_the_token():
    need_gpu()
    T, K = 5, 400
    idx, _ = ragged(T, K, seed=12)
    idx[3, 250] = 5000                     # past the compressed pool (900 rows)
    w = custom(idx, None, H=128, seed=1)
    plan = ht_plan(T, K, W.BF16, W.BF16, 2)
    ws = L.alloc_workspace(plan, T, 128, L.FLAG_VALIDATE_INDICES)
    log("[head tiles] validation")
    out, lse = run_decode(w, plan=plan, flags=L.FLAG_VALIDATE_INDICES, workspace=ws)
    assert L.get_device_error(ws) == (1, 3, 250)
    ok = [0, 1, 2, 4]
    compare(out, lse, oracle_for(w, ok), TOL_BF16, ok, "other tokens unaffected")


def test_head_tiles_segments_and_paged_forms():
    need_gpu()
    import test_gpu_paged as pg
    import test_gpu_segments as sg
    for kv, q in ((W.BF16, W.BF16), (W.FP8, W.BF16)):
        c = sg.make(6, 100, 500, kv=kv, q=q, seed=21)
        for S in (1, 3):
            sg.check(c, f"segments head tiles kv={kv} S={S}", plan=ht_plan(6, 600, q, kv, S))
        c = pg.make(5, 64, 7, 37, kv=kv, q=q, seed=22)
        for S in (1, 2):
            pg.check(c, f"paged head tiles kv={kv} S={S}",
                     plan=ht_plan(5, 64 + 7 * 37, q, kv, S))


def test_planner_picks_head_tiles_for_the_batched_configuration():
    need_gpu()
    w = W.make_batched_sinks("cuda")
    plan = L.plan_splits(w.T, w.H, w.K)
    log(f"[head tiles] batched_sinks default plan {plan.as_dict()}")
    assert plan.head_tiles == 2
    out, lse = run_decode(w, plan=plan)
    toks = list(range(0, w.T, 3))
    compare(out, lse, oracle_for(w, toks), TOL_BF16, toks, "batched_sinks head tiles")
