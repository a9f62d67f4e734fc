"""GPU parity of the page-table form (sparse_mla_decode_paged) with the
oracle, element by element, and bitwise agreement with the two-segment call
given the expanded table (the same slots in the same column order)."""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W
from parity_utils import same_bits, TOL_BF16, TOL_FP8, compare, log, need_gpu

pytestmark = pytest.mark.gpu


def make(T, K1, pages, ps, H=128, kv=W.BF16, q=W.BF16, swa_rows=600, n_pages=200,
         seed=0, lens=True, sinks=True):
    rng = np.random.default_rng(seed)
    qq = W.normal_rows(T * H, seed + 1, "cuda", q, scale=0.05).view(T, H, 512)
    swa = W.normal_rows(swa_rows, seed + 2, "cuda", kv, scale=0.08)
    comp = W.normal_rows(n_pages * ps, seed + 3, "cuda", kv, scale=0.08)
    si = torch.as_tensor(rng.integers(0, swa_rows, (T, K1)).astype(np.int32)).cuda() \
        if K1 else None
    bt = torch.as_tensor(np.stack([rng.permutation(n_pages)[:pages] for _ in range(T)])
                         .astype(np.int32)).cuda() if pages else None
    sl = tot = None
    if lens:
        a = rng.integers(0, K1 + 1, T)
        n = rng.integers(0, pages * ps + 1, T)
        if T > 3:
            a[0], n[0] = K1, pages * ps         # everything
            a[1], n[1] = 0, 0                   # nothing
            a[2], n[2] = K1, 1                  # one compressed slot
            a[3], n[3] = 3 if K1 >= 3 else K1, -2   # total below the window
        sl = torch.as_tensor(a.astype(np.int32)).cuda()
        tot = torch.as_tensor((a + n).astype(np.int32)).cuda()
    g = torch.Generator().manual_seed(seed + 7)
    qs = 0.05 if q == W.FP8 else 1.0
    ks = 0.08 if kv == W.FP8 else 1.0
    return dict(q=qq, swa=swa, comp=comp, si=si, bt=bt, ps=ps, sl=sl, tot=tot, T=T, H=H,
                sinks=torch.randn(H, generator=g).cuda() if sinks else None,
                b1=qs * ks / math.sqrt(512), b2=ks, kv=kv, qd=q)


def run(c, plan=None, flags=0, workspace=None):
    out = torch.full((c["T"], c["H"], 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c["T"], c["H"]), float("nan"), device="cuda")
    L.decode_paged(c["q"], c["swa"] if c["si"] is not None else None,
                   c["comp"] if c["bt"] is not None else None, c["si"], c["bt"], c["ps"], out,
                   swa_topk_lens=c["sl"], topk_lens=c["tot"], out_lse=lse, sinks=c["sinks"],
                   bmm1_scale=c["b1"], bmm2_scale=c["b2"], plan=plan, flags=flags,
                   workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def oracle_of(c, tokens):
    tok = list(tokens)
    cpu = lambda x: None if x is None else x.cpu().numpy()
    pick = lambda x: None if x is None else cpu(x)[tok]
    return oracle.sparse_mla_decode_paged(
        W.raw_bits(c["q"][tok]), c["qd"], W.raw_bits(c["swa"]), W.raw_bits(c["comp"]),
        c["kv"], pick(c["si"]), pick(c["bt"]), c["ps"], pick(c["sl"]), pick(c["tot"]),
        cpu(c["sinks"]), c["b1"], c["b2"], 1.0)


def check(c, what, plan=None, tokens=None):
    tokens = list(range(c["T"])) if tokens is None else list(tokens)
    tol = TOL_FP8 if W.FP8 in (c["kv"], c["qd"]) else TOL_BF16
    log(f"[paged] {what}: T={c['T']} H={c['H']} plan={None if plan is None else plan.as_dict()}")
    out, lse = run(c, plan)
    e, le = compare(out, lse, oracle_of(c, tokens), tol, tokens, what)
    log(f"[paged] {what}: max|out err| {e:.3g}  max|lse err| {le:.3g}")
    return out, lse


@pytest.mark.parametrize("H,kv,q", [(128, W.BF16, W.BF16), (64, W.BF16, W.BF16),
                                    (128, W.FP8, W.BF16), (64, W.FP8, W.FP8)])
@pytest.mark.parametrize("K1,pages,ps", [(128, 10, 64), (9, 7, 16), (0, 5, 64),
                                         (128, 0, 64), (40, 13, 37)])
def test_paged_match_oracle(H, kv, q, K1, pages, ps):
    need_gpu()
    c = make(10, K1, pages, ps, H=H, kv=kv, q=q, seed=K1 + 3 * pages + ps)
    check(c, f"H={H} kv={kv} K1={K1} pages={pages}x{ps}")
    qc = L.DTYPE_FP8_E4M3FN if q == W.FP8 else L.DTYPE_BF16
    kc = L.DTYPE_FP8_E4M3FN if kv == W.FP8 else L.DTYPE_BF16
    K = K1 + pages * ps
    S = min(4, -(-K // 64))
    check(c, f"H={H} kv={kv} K1={K1} pages={pages}x{ps} S={S}",
          plan=L.plan_splits(10, H, K, qc, kc, num_splits=S))


def expanded(c):
    bt = c["bt"].long()
    ext = (bt[:, :, None] * c["ps"] + torch.arange(c["ps"], device="cuda")[None, None, :])
    return ext.reshape(bt.shape[0], -1).int().contiguous()


def test_paged_equals_the_expanded_two_segment_call_bitwise():
    need_gpu()
    for T, pages, ps, H, kv, S in ((12, 10, 64, 128, W.BF16, 1), (12, 7, 16, 64, W.BF16, 3),
                                   (8, 30, 64, 128, W.FP8, 1), (4, 30, 64, 128, W.BF16, 16)):
        c = make(T, 128, pages, ps, H=H, kv=kv, seed=T + pages)
        el = torch.clamp(c["tot"] - c["sl"], min=0).int()
        kc = L.DTYPE_FP8_E4M3FN if kv == W.FP8 else L.DTYPE_BF16
        plan = L.plan_splits(T, H, 128 + pages * ps, L.DTYPE_BF16, kc, num_splits=S)
        a_out, a_lse = run(c, plan)
        b_out = torch.full_like(a_out, float("nan"))
        b_lse = torch.full_like(a_lse, float("nan"))
        L.decode_segments(c["q"], c["swa"], c["comp"], c["si"], expanded(c), b_out,
                          swa_topk_lens=c["sl"], extra_topk_lens=el, out_lse=b_lse,
                          sinks=c["sinks"], bmm1_scale=c["b1"], bmm2_scale=c["b2"], plan=plan)
        torch.cuda.synchronize()
        log(f"[paged] expanded-table equality T={T} pages={pages}x{ps} H={H} kv={kv} S={S}")
        same_bits(a_out, b_out)
        assert torch.equal(a_lse, b_lse)


def test_paged_full_size_matches_expanded_and_sampled_oracle():
    """T=512, H=128: 128 window rows + 30 pages of 64 compressed rows, all
    visible.  Bitwise equal to the expanded two-segment call; sampled
    tokens against the oracle."""
    need_gpu()
    c = make(512, 128, 30, 64, seed=12, lens=False, swa_rows=40000, n_pages=4096)
    plan = L.plan_splits(512, 128, 2048)
    out, lse = run(c, plan)
    b_out, b_lse = torch.empty_like(out), torch.empty_like(lse)
    L.decode_segments(c["q"], c["swa"], c["comp"], c["si"], expanded(c), b_out, out_lse=b_lse,
                      sinks=c["sinks"], bmm1_scale=c["b1"], bmm2_scale=c["b2"], plan=plan)
    torch.cuda.synchronize()
    same_bits(out, b_out)
    assert torch.equal(lse, b_lse)
    toks = [0, 3, 300, 511]
    compare(out, lse, oracle_of(c, toks), TOL_BF16, toks, "paged T=512 sampled")


def test_paged_validate_reports_pages_and_lengths():
    need_gpu()
    c = make(4, 16, 4, 8, seed=6, n_pages=20, lens=False)
    c["bt"][1, 2] = 20                      # one page past the compressed pool
    plan = L.plan_splits(4, 128, 16 + 32)
    ws = L.alloc_workspace(plan, 4, 128, L.FLAG_VALIDATE_INDICES)
    out, lse = run(c, plan, L.FLAG_VALIDATE_INDICES, ws)
    assert L.get_device_error(ws) == (1, 1, 16 + 2 * 8)   # first slot of that page
    # its slots are skipped: the oracle over the same token without them
    ref = oracle_of(c, [0, 2, 3])
    compare(out, lse, ref, TOL_BF16, [0, 2, 3], "pages of other tokens unaffected")
    c["bt"][1, 2] = 3
    c["sl"] = torch.tensor([16, 5, 17, 0], dtype=torch.int32, device="cuda")   # 17 > width
    c["tot"] = torch.tensor([48, 5, 20, 10], dtype=torch.int32, device="cuda")
    run(c, plan, L.FLAG_VALIDATE_INDICES, ws)
    assert L.get_device_error(ws)[:2] == (2, 2)
    c["sl"][2] = 16
    c["tot"][3] = 49                        # beyond window + every slot
    run(c, plan, L.FLAG_VALIDATE_INDICES, ws)
    assert L.get_device_error(ws)[:2] == (2, 3)


@pytest.mark.parametrize("seed", range(24))
def test_random_paged_shapes_match_oracle(seed):
    """Seeded random page-table calls: window widths 0..128, 0..20 pages of
    1..96 rows, both head counts and format pairs, lengths, sinks, planner,
    unsplit or random split counts."""
    need_gpu()
    rng = np.random.default_rng(9000 + seed)
    K1 = int(rng.integers(0, 129))
    ps = int(rng.choice([1, 16, 37, 64, 96]))
    pages = int(rng.integers(0 if K1 else 1, 21))
    H = int(rng.choice([64, 128]))
    q, kv = [(W.BF16, W.BF16), (W.BF16, W.FP8), (W.FP8, W.FP8)][int(rng.integers(3))]
    T = int(rng.integers(1, 7))
    c = make(T, K1, pages, ps, H=H, kv=kv, q=q, seed=9000 + seed,
             swa_rows=int(rng.integers(1, 700)), n_pages=max(pages, int(rng.integers(1, 120))),
             lens=bool(rng.random() < 0.7), sinks=bool(rng.random() < 0.5))
    K = K1 + pages * ps
    S = int(rng.choice([0, 1, int(rng.integers(1, -(-K // 64) + 1))]))
    plan = L.plan_splits(T, H, K, L.dtype_code(c["q"]), L.dtype_code(c["swa"]), num_splits=S)
    check(c, f"random seed={seed} K1={K1} pages={pages}x{ps} H={H} q={q} kv={kv} "
             f"S={plan.num_splits}", plan=plan)
