"""GPU parity of the two-segment form (sparse_mla_decode_segments) with the
oracle, element by element, and bitwise agreement with the combined-table
call where the two describe the same slots in the same column order."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W
from parity_utils import (same_bits, LSE_ATOL, TOL_BF16, TOL_FP8, compare, log, need_gpu)

pytestmark = pytest.mark.gpu


def make(T, K1, K2, H=128, kv=W.BF16, q=W.BF16, swa_rows=600, comp_rows=900,
         seed=0, neg=0.05, lens=True, sinks=True, stride_pad=0):
    """Pools and two tables on the GPU (tables optionally with padded rows)."""
    rng = np.random.default_rng(seed)
    qq = W.normal_rows(T * H, seed + 1, "cuda", q, scale=0.05).view(T, H, 512)
    swa = W.normal_rows(swa_rows, seed + 2, "cuda", kv, scale=0.08)
    comp = W.normal_rows(comp_rows, seed + 3, "cuda", kv, scale=0.08)
    def table(K, rows):
        if K == 0:
            return None
        t = rng.integers(0, rows, (T, K + stride_pad)).astype(np.int32)
        t[rng.random((T, K + stride_pad)) < neg] = -1
        return torch.as_tensor(t).cuda()[:, :K]
    si, ei = table(K1, swa_rows), table(K2, comp_rows)
    sl = el = None
    if lens:
        sl = torch.as_tensor(rng.integers(0, K1 + 1, T).astype(np.int32)).cuda() if K1 else None
        el = torch.as_tensor(rng.integers(0, K2 + 1, T).astype(np.int32)).cuda() if K2 else None
        if T > 2:           # the ends of both ranges
            if sl is not None:
                sl[0], sl[1] = K1, 0
            if el is not None:
                el[0], el[1] = K2, 0
    g = torch.Generator().manual_seed(seed + 7)
    qs = 0.05 if q == W.FP8 else 1.0
    ks = 0.08 if kv == W.FP8 else 1.0
    return dict(q=qq, swa=swa, comp=comp, si=si, ei=ei, sl=sl, el=el, H=H, T=T,
                sinks=torch.randn(H, generator=g).cuda() if sinks else None,
                b1=qs * ks / math.sqrt(512), b2=ks, kv=kv, qd=q)


def run(c, plan=None, flags=0, workspace=None):
    out = torch.full((c["T"], c["H"], 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c["T"], c["H"]), float("nan"), device="cuda")
    L.decode_segments(c["q"], c["swa"] if c["si"] is not None else None,
                      c["comp"] if c["ei"] is not None else None, c["si"], c["ei"], out,
                      swa_topk_lens=c["sl"], extra_topk_lens=c["el"], out_lse=lse,
                      sinks=c["sinks"], bmm1_scale=c["b1"], bmm2_scale=c["b2"],
                      plan=plan, flags=flags, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def oracle_of(c, tokens):
    tok = list(tokens)
    cpu = lambda x: None if x is None else x.cpu().numpy()
    pick = lambda x: None if x is None else cpu(x)[tok]
    return oracle.sparse_mla_decode_segments(
        W.raw_bits(c["q"][tok]), c["qd"], W.raw_bits(c["swa"]), W.raw_bits(c["comp"]),
        c["kv"], pick(c["si"]), pick(c["ei"]), pick(c["sl"]), pick(c["el"]),
        cpu(c["sinks"]), c["b1"], c["b2"], 1.0)


def check(c, what, plan=None, tokens=None):
    tokens = list(range(c["T"])) if tokens is None else list(tokens)
    tol = TOL_FP8 if W.FP8 in (c["kv"], c["qd"]) else TOL_BF16
    log(f"[segments] {what}: T={c['T']} H={c['H']} K1={0 if c['si'] is None else c['si'].shape[1]} "
        f"K2={0 if c['ei'] is None else c['ei'].shape[1]} kv={c['kv']} q={c['qd']} "
        f"plan={None if plan is None else plan.as_dict()}")
    out, lse = run(c, plan)
    e, le = compare(out, lse, oracle_of(c, tokens), tol, tokens, what)
    log(f"[segments] {what}: max|out err| {e:.3g}  max|lse err| {le:.3g}")
    return out, lse


@pytest.mark.parametrize("H,kv,q", [(128, W.BF16, W.BF16), (64, W.BF16, W.BF16),
                                    (128, W.FP8, W.BF16), (64, W.FP8, W.FP8),
                                    (128, W.FP8, W.FP8)])
@pytest.mark.parametrize("K1,K2", [(128, 700), (7, 61), (0, 300), (200, 0), (33, 1500)])
def test_segments_match_oracle(H, kv, q, K1, K2):
    need_gpu()
    c = make(10, K1, K2, H=H, kv=kv, q=q, seed=K1 * 7 + K2)
    check(c, f"H={H} kv={kv} K1={K1} K2={K2}")
    qc = L.DTYPE_FP8_E4M3FN if q == W.FP8 else L.DTYPE_BF16
    kc = L.DTYPE_FP8_E4M3FN if kv == W.FP8 else L.DTYPE_BF16
    S = min(5, -(-(K1 + K2) // 64))
    check(c, f"H={H} kv={kv} K1={K1} K2={K2} S={S}",
          plan=L.plan_splits(10, H, K1 + K2, qc, kc, num_splits=S))


def test_segments_without_lengths_and_with_strided_tables():
    need_gpu()
    c = make(6, 90, 400, seed=3, lens=False, stride_pad=37)
    assert c["si"].stride(0) == 127 and c["ei"].stride(0) == 437
    check(c, "no lengths, strided tables")


def test_segments_equal_the_combined_table_bitwise():
    """A 128-column SWA table plus extras is the combined table
    [SWA (masked from swa_topk_len on) | extras] with topk_len = 128 + extra
    length: the same slots in the same column order, so the same bits."""
    need_gpu()
    for T, K2, H, kv, S in ((12, 700, 128, W.BF16, 1), (12, 700, 64, W.BF16, 3),
                            (8, 1920, 128, W.FP8, 1), (4, 1920, 128, W.BF16, 16)):
        c = make(T, 128, K2, H=H, kv=kv, seed=T + K2)
        comb = torch.cat([c["si"], c["ei"]], 1).clone()
        sl = c["sl"].cpu()
        for t in range(T):
            comb[t, int(sl[t]):128] = -1
        topk = (128 + c["el"]).int()
        kc = L.DTYPE_FP8_E4M3FN if kv == W.FP8 else L.DTYPE_BF16
        plan = L.plan_splits(T, H, 128 + K2, L.DTYPE_BF16, kc, num_splits=S)
        a_out, a_lse = run(c, plan)
        b_out = torch.full_like(a_out, float("nan"))
        b_lse = torch.full_like(a_lse, float("nan"))
        L.decode(c["q"], c["swa"], c["comp"], comb, b_out, out_lse=b_lse, topk_lens=topk,
                 sinks=c["sinks"], bmm1_scale=c["b1"], bmm2_scale=c["b2"], plan=plan)
        torch.cuda.synchronize()
        log(f"[segments] combined-form equality T={T} K2={K2} H={H} kv={kv} S={S}")
        same_bits(a_out, b_out)
        assert torch.equal(a_lse, b_lse)


def test_segments_full_size_matches_combined_and_sampled_oracle():
    """The headline shape: T=512, H=128, 128 SWA + 1920 extra columns,
    every slot active.  Bitwise equal to the combined call; sampled tokens
    against the oracle."""
    need_gpu()
    c = make(512, 128, 1920, seed=11, neg=0.0, lens=False,
             swa_rows=40000, comp_rows=200000)
    plan = L.plan_splits(512, 128, 2048)
    out, lse = run(c, plan)
    b_out = torch.empty_like(out)
    b_lse = torch.empty_like(lse)
    L.decode(c["q"], c["swa"], c["comp"], torch.cat([c["si"], c["ei"]], 1).contiguous(),
             b_out, out_lse=b_lse, sinks=c["sinks"], bmm1_scale=c["b1"],
             bmm2_scale=c["b2"], plan=plan)
    torch.cuda.synchronize()
    same_bits(out, b_out)
    assert torch.equal(lse, b_lse)
    toks = [0, 1, 255, 256, 511]
    compare(out, lse, oracle_of(c, toks), TOL_BF16, toks, "segments T=512 sampled")


def test_segments_validate_reports_virtual_columns_and_lengths():
    need_gpu()
    c = make(4, 50, 300, seed=5, neg=0.0)
    c["ei"][2, 17] = 900                   # one past the compressed pool
    plan = L.plan_splits(4, 128, 350)
    ws = L.alloc_workspace(plan, 4, 128, L.FLAG_VALIDATE_INDICES)
    c["el"][2] = 300                       # the bad column is active
    out, lse = run(c, plan, L.FLAG_VALIDATE_INDICES, ws)
    assert L.get_device_error(ws) == (1, 2, 50 + 17)
    # the bad slot was skipped: same as masking it
    c2 = dict(c, ei=c["ei"].clone())
    c2["ei"][2, 17] = -1
    compare(out, lse, oracle_of(c2, range(4)), TOL_BF16, what="bad extra slot skipped")
    c2["sl"] = c2["sl"].clone()
    c2["sl"][1] = 51                       # past the SWA width
    run(c2, plan, L.FLAG_VALIDATE_INDICES, ws)
    assert L.get_device_error(ws)[:2] == (2, 1)


@pytest.mark.parametrize("H", [64, 128])
def test_ragged_segments_batch_order_does_not_change_any_token(H):
    """Items start longest first within each XCD (ranked by the active
    columns of both tables); permuting the tokens of a ragged batch moves
    every item to another workgroup and must leave each token's bits
    unchanged, unsplit and split."""
    need_gpu()
    T, K1, K2 = 256, 128, 1920
    c = make(T, K1, K2, H=H, swa_rows=600, comp_rows=4000, seed=41)
    perm = torch.as_tensor(np.random.default_rng(5).permutation(T)).cuda()
    cp = dict(c)
    for k in ("q", "si", "ei", "sl", "el"):
        cp[k] = c[k][perm].contiguous()
    for S in (1, 2):
        log(f"[segments] ragged batch T={T} H={H} permuted, {S} split(s)")
        plan = L.plan_splits(T, H, K1 + K2, num_splits=S)
        a, la = run(c, plan=plan)
        b, lb = run(cp, plan=plan)
        same_bits(a[perm], b, str(S))
        assert torch.equal(la[perm], lb), S


@pytest.mark.parametrize("seed", range(24))
def test_random_segment_shapes_match_oracle(seed):
    """Seeded random two-segment calls: widths 0..300 / 0..1200 (not both
    0), both head counts and format pairs, -1 densities, lengths, sinks,
    planner, unsplit or random split counts."""
    need_gpu()
    rng = np.random.default_rng(7000 + seed)
    K1 = int(rng.choice([0, int(rng.integers(1, 300))]))
    K2 = int(rng.integers(0 if K1 else 1, 1200))
    H = int(rng.choice([64, 128]))
    q, kv = [(W.BF16, W.BF16), (W.BF16, W.FP8), (W.FP8, W.FP8)][int(rng.integers(3))]
    T = int(rng.integers(1, 7))
    c = make(T, K1, K2, H=H, kv=kv, q=q, seed=7000 + seed,
             neg=float(rng.choice([0.0, 0.1, 0.6])), lens=bool(rng.random() < 0.7),
             sinks=bool(rng.random() < 0.5), swa_rows=int(rng.integers(1, 700)),
             comp_rows=int(rng.integers(1, 3000)))
    K = K1 + K2
    S = int(rng.choice([0, 1, int(rng.integers(1, -(-K // 64) + 1))]))
    plan = L.plan_splits(T, H, K, L.dtype_code(c["q"]), L.dtype_code(c["swa"]), num_splits=S)
    check(c, f"random seed={seed} K1={K1} K2={K2} H={H} q={q} kv={kv} S={plan.num_splits}",
          plan=plan)
