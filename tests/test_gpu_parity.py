"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element on the same seeded inputs.

Bar: |out - ref| <= 1e-2 + 1e-2*|ref| (BF16 pools) or 3e-2 + 3e-2*|ref|
(FP8 pools), |lse - ref| <= 1e-3, -inf LSEs in the same places; selection
and masking are checked bit-exactly with one-hot probe rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import (same_bits, TOL_BF16, TOL_FP8, compare, log, need_gpu,
                          oracle_for, run_decode)

pytestmark = pytest.mark.gpu


def custom(idx, lens=None, H=128, swa_rows=600, comp_rows=900, sinks=True,
           kv=W.BF16, q=W.BF16, seed=0, b1=None, b2=1.0, lse_scale=1.0,
           row_stride=512):
    """A workload with an explicit table (CPU tensors -> GPU)."""
    idx = torch.as_tensor(np.asarray(idx, np.int32))
    T, K = idx.shape
    qq = W.normal_rows(T * H, seed + 1, "cuda", q, scale=0.05).view(T, H, 512)
    def pool(rows, sd):
        p = W.normal_rows(rows, sd, "cuda", kv, scale=0.08)
        if row_stride == 512:
            return p
        big = torch.zeros((rows, row_stride), dtype=p.dtype, device="cuda")
        big[:, :512] = p
        return big[:, :512]
    g = torch.Generator().manual_seed(seed + 7)
    qs = 0.05 if q == W.FP8 else 1.0
    ks = 0.08 if kv == W.FP8 else 1.0
    return W.Workload(
        name="custom", T=T, H=H, K=K, q=qq, q_dtype=q,
        swa_pool=pool(swa_rows, seed + 2),
        comp_pool=pool(comp_rows, seed + 3) if K > 128 else None,
        kv_dtype=kv, indices=idx.cuda(),
        topk_lens=None if lens is None else torch.as_tensor(
            np.asarray(lens, np.int32)).cuda(),
        seq_lens=torch.full((T,), 4096, dtype=torch.int32, device="cuda"),
        cum_seq_lens_q=None,
        sinks=torch.randn(H, generator=g).cuda() if sinks else None,
        bmm1_scale=(b1 if b1 is not None else qs * ks / math.sqrt(512)),
        bmm2_scale=b2 * ks, lse_scale=lse_scale)


def check(w, tokens=None, tol=None, plan=None, what=None):
    tol = tol or (TOL_FP8 if W.FP8 in (w.kv_dtype, w.q_dtype) else TOL_BF16)
    tokens = list(range(w.T)) if tokens is None else list(tokens)
    what = what or w.name
    log(f"[parity] {what}: T={w.T} H={w.H} K={w.K} q={w.q_dtype} "
        f"kv={w.kv_dtype} plan={None if plan is None else plan.as_dict()}")
    out, lse = run_decode(w, plan=plan)
    ref = oracle_for(w, tokens)
    e, le = compare(out, lse, ref, tol, tokens, what)
    log(f"[parity] {what}: max|out err| {e:.3g}  max|lse err| {le:.3g}")
    return out, lse


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_tiny_matches_oracle():
    """The tiny configuration at its stated single split, then at the
    planner's own choice and at 2 and 4 splits."""
    need_gpu()
    w = W.make_tiny("cuda")
    check(w, plan=L.plan_splits(w.T, w.H, w.K, num_splits=1), what="tiny split=1")
    check(w, what="tiny planner default")
    for s in (2, 4):
        check(w, plan=L.plan_splits(w.T, w.H, w.K, num_splits=s),
              what=f"tiny split={s}")


def test_batched_sinks_matches_oracle():
    need_gpu()
    w = W.make_batched_sinks("cuda")
    check(w)


def test_fp8_matches_oracle():
    need_gpu()
    w = W.make_fp8("cuda")
    check(w)


@pytest.mark.parametrize("T", [1, 4, 8])
def test_long_context_split_k_matches_oracle(T):
    need_gpu()
    w = W.make_long_context(T, "cuda")
    plan = L.plan_splits(T, 128, 2048)
    assert 1 < plan.num_splits <= 16
    check(w, plan=plan)
    check(w, plan=L.plan_splits(T, 128, 2048, num_splits=1), what=f"T={T} unsplit")


def test_spec_decode_matches_oracle_every_token():
    """All 512 tokens: both tokens of every request (the second shares ~90%
    of its compressed rows with the first, so the two run on rows the L2
    already holds)."""
    need_gpu()
    w = W.make_spec_decode("cuda")
    out, lse = check(w)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_full_size_long_context_batch_every_token():
    """The benchmark's shape and launch configuration (planner default):
    T=512 tokens, H=128, topk 2048, BF16, 128k context; every token."""
    need_gpu()
    w = W.make_long_context(512, "cuda", seed=4512)
    out, lse = check(w)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


# ---------------------------------------------------------------------------
# selection and masking, bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,dt", [(64, W.BF16), (128, W.BF16), (64, W.FP8),
                                   (128, W.FP8)])
def test_selection_probe_exact(H, dt):
    """q = 0 and no sink, pool row r = one-hot e_{r mod 512}: every logit is
    0, so 2^lse is the active-slot count and count*out[d] is the number of
    active slots whose row is d mod 512 -- exact integers on both sides.
    E4M3 holds 0 and 1 exactly, so the FP8 form (FP8 q and rows, widened
    exactly to BF16 before the BF16 MFMAs) is exact too."""
    need_gpu()
    code = L.DTYPE_FP8_E4M3FN if dt == W.FP8 else L.DTYPE_BF16
    tdt = torch.float8_e4m3fn if dt == W.FP8 else torch.bfloat16
    rng = np.random.default_rng(5)
    T, K = 9, 600
    idx = np.empty((T, K), np.int32)
    idx[:, :128] = rng.integers(0, 512, (T, 128))
    idx[:, 128:] = rng.integers(0, 1500, (T, K - 128))
    for t in range(T):
        idx[t, rng.choice(K, 40, replace=False)] = -1
    idx[8, :] = -1
    lens = np.array([0, 1, 127, 128, 129, 161, 600, 300, 600], np.int32)
    swa = torch.zeros((512, 512), dtype=torch.bfloat16)
    swa[torch.arange(512), torch.arange(512)] = 1
    comp = torch.zeros((1500, 512), dtype=torch.bfloat16)
    comp[torch.arange(1500), torch.arange(1500) % 512] = 1
    w = W.Workload(name="probe", T=T, H=H, K=K,
                   q=torch.zeros((T, H, 512), dtype=torch.bfloat16,
                                 device="cuda").to(tdt),
                   q_dtype=dt, swa_pool=swa.to(tdt).cuda(), comp_pool=comp.to(tdt).cuda(),
                   kv_dtype=dt, indices=torch.from_numpy(idx).cuda(),
                   topk_lens=torch.from_numpy(lens).cuda(),
                   seq_lens=torch.full((T,), 9000, dtype=torch.int32,
                                       device="cuda"),
                   cum_seq_lens_q=None, sinks=None, bmm1_scale=0.3,
                   bmm2_scale=1.0)
    for S in (1, 3):
        out, lse = run_decode(w, plan=L.plan_splits(T, H, K, code, code, num_splits=S))
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        for t in range(T):
            slots = oracle.active_slots(idx[t], lens[t])
            n = len(slots)
            want = np.zeros(512)
            for c, pool, r in slots:
                want[r % 512] += 1
            if n == 0:
                assert np.all(np.isneginf(l[t])) and not o[t].any()
                continue
            assert np.all(np.rint(np.exp2(l[t])) == n), (t, S)
            assert np.array_equal(np.rint(n * o[t]), np.tile(want, (H, 1))), (t, S)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def test_swa_only_table_without_compressed_pool():
    need_gpu()
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 600, (5, 128)).astype(np.int32)
    idx[2, 60:] = -1
    check(custom(idx, lens=[128, 100, 128, 1, 0]), what="swa-only K=128")
    check(custom(idx[:, :77], H=64, sinks=False), what="swa-only K=77")


def test_topk_edges_ragged_tiles_and_masks():
    need_gpu()
    rng = np.random.default_rng(2)
    T, K = 12, 700
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 900, (T, K - 128))], 1).astype(np.int32)
    idx[3, :] = -1
    idx[4, 1:] = -1
    idx[5, ::3] = -1
    lens = [0, 1, 31, 32, 33, 127, 128, 129, 700, 650, 64, 65]
    for H in (64, 128):
        w = custom(idx, lens=lens, H=H)
        check(w, what=f"edges H={H}")
        check(w, plan=L.plan_splits(T, H, K, num_splits=5), what=f"edges H={H} S=5")
        check(custom(idx, lens=lens, H=H, sinks=False), what=f"edges H={H} nosink")


@pytest.mark.parametrize("H", [64, 128])
def test_large_logit_range_restarts_are_exact(H):
    """Logits spread far wider than the 64 (base-2) slack the kernel allows
    above its first-tile reference max, so later tiles force the split to
    restart with a higher reference (at H=64 the two waves of a head block
    then agree on the larger raised max); the result must still match."""
    need_gpu()
    rng = np.random.default_rng(11)
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 1400))], 1).astype(np.int32)
    # scores ~ N(0, (2*sqrt(512))^2): std ~45 natural, ~65 in base 2
    w = custom(idx, lens=[1528, 900, 200, 1528], H=H, b1=2.0)
    check(w, what=f"wide logits H={H} unsplit", plan=L.plan_splits(4, H, 1528, num_splits=1))
    check(w, what=f"wide logits H={H} S=4", plan=L.plan_splits(4, H, 1528, num_splits=4))


@pytest.mark.parametrize("dt", [W.BF16, W.FP8])
def test_increasing_logits_force_repeated_restarts(dt):
    """Row i of the table is (i/40)*u for a fixed direction u and q = u, so
    the logits rise by ~37 (base-2) every 32 rows and the 64 units of slack
    are outgrown every 64 rows (every tile of the H=64 kernel).  FP8 rows
    round i/40 to E4M3 (the oracle reads the same bits)."""
    need_gpu()
    T, K, H = 2, 700, 64
    tdt = torch.float8_e4m3fn if dt == W.FP8 else torch.bfloat16
    u = torch.zeros(512)
    u[:8] = 1.0
    rows = torch.stack([u * (i / 40.0) for i in range(K)]).to(tdt)
    idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    idx[:, :128] = np.arange(128)
    w = W.Workload(name="rising", T=T, H=H, K=K,
                   q=u.to(tdt).expand(T, H, 512).contiguous().cuda(),
                   q_dtype=dt, swa_pool=rows.cuda(), comp_pool=rows.cuda(),
                   kv_dtype=dt, indices=torch.from_numpy(idx).cuda(),
                   topk_lens=None,
                   seq_lens=torch.full((T,), 4096, dtype=torch.int32, device="cuda"),
                   cum_seq_lens_q=None, sinks=None, bmm1_scale=4.0, bmm2_scale=1.0)
    check(w, what=f"rising logits {dt}")


def test_duplicate_indices_count_per_slot():
    need_gpu()
    idx = np.zeros((3, 300), np.int32)
    idx[:, :128] = 7
    idx[:, 128:] = np.arange(172) % 5
    idx[1, 200:] = -1
    check(custom(idx), what="duplicates")


def test_wide_table_multiple_segments():
    need_gpu()
    rng = np.random.default_rng(3)
    T, K = 3, 5000
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 20000, (T, K - 128))], 1).astype(np.int32)
    idx[1, 4000:] = -1
    w = custom(idx, lens=[5000, 4500, 2100], comp_rows=20000)
    check(w, what="K=5000 unsplit", plan=L.plan_splits(T, 128, K, num_splits=1))
    check(w, what="K=5000 S=3", plan=L.plan_splits(T, 128, K, num_splits=3))


@pytest.mark.parametrize("H,q", [(128, W.BF16), (128, W.FP8), (64, W.BF16),
                                  (64, W.FP8)])
def test_fp8_rows_edges_segments_and_restarts(H, q):
    """FP8 rows at H=128 take the register-staged path of the H=128 kernel
    (one register set: each row of tile i+1 is stored and the same row of
    tile i+2 loaded inside the S^T MFMAs of tile i; the first tile, the last
    and the drain are separate compile-time iterations); at H=64 they are
    loaded through registers one 64-row tile ahead (during the S^T MFMAs of
    a tile, stored during its O^T MFMAs); in both kernels FP8 rows (and
    FP8 q) are widened exactly to BF16 and multiplied on the BF16 MFMA.
    Ragged and tiny lengths give odd, single and empty tile counts; K=5000
    crosses segments; wide logits force restarts."""
    need_gpu()
    qc = L.DTYPE_FP8_E4M3FN if q == W.FP8 else L.DTYPE_BF16
    kc = L.DTYPE_FP8_E4M3FN
    rng = np.random.default_rng(21)
    T, K = 12, 700
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 900, (T, K - 128))], 1).astype(np.int32)
    idx[3, :] = -1
    idx[5, ::3] = -1
    idx[6, 200:230] = idx[6, 300]          # duplicates count per slot
    lens = [0, 1, 31, 32, 33, 127, 128, 129, 700, 650, 64, 97]
    w = custom(idx, lens=lens, H=H, kv=W.FP8, q=q)
    check(w, what=f"fp8 rows H={H} q={q} edges")
    check(w, plan=L.plan_splits(T, H, K, qc, kc, num_splits=5),
          what=f"fp8 rows H={H} q={q} edges S=5")

    T, K = 3, 5000
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 20000, (T, K - 128))], 1).astype(np.int32)
    idx[1, 4000:] = -1
    w = custom(idx, lens=[5000, 4500, 2100], comp_rows=20000, H=H, kv=W.FP8, q=q)
    check(w, what=f"fp8 rows H={H} q={q} K=5000",
          plan=L.plan_splits(T, H, K, qc, kc, num_splits=1))

    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 1400))], 1).astype(np.int32)
    # FP8 q holds x/0.05, so its bmm1 carries the 0.05 (as the workloads
    # fold it) and the logit spread - hence the restarts - matches the BF16
    # case; unscaled, the LSE would sit near 5e4, where one fp32 ulp already
    # exceeds the 1e-3 LSE bar.
    w = custom(idx, lens=[1528, 900, 200, 1528], H=H, kv=W.FP8, q=q,
               b1=2.0 * (0.05 if q == W.FP8 else 1.0))
    check(w, what=f"fp8 rows H={H} q={q} wide logits",
          plan=L.plan_splits(4, H, 1528, qc, kc, num_splits=1))


@pytest.mark.parametrize("H", [64, 128])
def test_first_and_last_pool_rows(H):
    """Tables that name row 0 and the last row of both pools (and -1 slots
    around them): every row load, including the FP8 rows' one-row buffer
    resource, reaches exactly the pool's ends."""
    need_gpu()
    swa_rows, comp_rows = 600, 900
    idx = np.full((3, 300), -1, np.int32)
    idx[:, 0], idx[:, 1], idx[:, 127] = 0, swa_rows - 1, swa_rows - 1
    idx[:, 128], idx[:, 129], idx[:, 299] = comp_rows - 1, 0, comp_rows - 1
    idx[1, 130:160] = np.arange(comp_rows - 30, comp_rows)
    idx[2, 2:40] = np.arange(swa_rows - 38, swa_rows)
    for kv in (W.BF16, W.FP8):
        w = custom(idx, kv=kv, q=kv, H=H, swa_rows=swa_rows, comp_rows=comp_rows)
        check(w, what=f"pool ends H={H} kv={kv}")
        qc = L.DTYPE_FP8_E4M3FN if kv == W.FP8 else L.DTYPE_BF16
        check(w, plan=L.plan_splits(3, H, 300, qc, qc, num_splits=3),
              what=f"pool ends H={H} kv={kv} S=3")


@pytest.mark.parametrize("H", [64, 128])
def test_padded_pool_rows(H):
    """Pool rows with a larger stride than their 512 elements: every row
    load (LDS-DMA, and for FP8 rows the per-row buffer resource) starts at
    the row's own address."""
    need_gpu()
    rng = np.random.default_rng(4)
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 200))], 1).astype(np.int32)
    for kv in (W.BF16, W.FP8):
        for q in ((W.BF16, W.FP8) if kv == W.FP8 else (W.BF16,)):
            w = custom(idx, kv=kv, q=q, H=H, row_stride=576)
            assert w.swa_pool.stride(0) == 576
            check(w, what=f"row stride 576 H={H} kv={kv} q={q}")


@pytest.mark.parametrize("q,kv,H", [(W.FP8, W.FP8, 128), (W.BF16, W.FP8, 64)])
def test_other_dtype_and_head_pairs(q, kv, H):
    need_gpu()
    rng = np.random.default_rng(6)
    idx = np.concatenate([rng.integers(0, 600, (6, 128)),
                          rng.integers(0, 900, (6, 400))], 1).astype(np.int32)
    check(custom(idx, q=q, kv=kv, H=H, lens=[528, 300, 129, 5, 400, 528]),
          what=f"q={q} kv={kv} H={H}")


def test_lse_scale_and_missing_lse():
    need_gpu()
    rng = np.random.default_rng(7)
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 100))], 1).astype(np.int32)
    for H in (64, 128):
        w = custom(idx, H=H, lse_scale=math.log(2.0), b2=0.5)
        check(w, what=f"lse_scale=ln2 bmm2=0.5 H={H}")
        # out_lse = NULL, unsplit and split (the split epilogue and the
        # combine then write no LSE; the outputs must not change)
        for S in (1, 3):
            plan = L.plan_splits(4, H, 228, num_splits=S)
            assert plan.num_splits == S
            out, lse = run_decode(w, plan=plan, out_lse=False)
            assert lse is None
            out2, lse2 = run_decode(w, plan=plan)
            same_bits(out, out2, f"no LSE H={H} S={S}")
            assert not torch.isnan(lse2).any()


def test_split_and_unsplit_agree():
    need_gpu()
    w = W.make_long_context(4, "cuda")
    a, la = run_decode(w, plan=L.plan_splits(4, 128, 2048, num_splits=1))
    b, lb = run_decode(w, plan=L.plan_splits(4, 128, 2048, num_splits=16))
    d = (a.float() - b.float()).abs()
    assert d.max().item() <= 1e-2 + 1e-2 * a.float().abs().max().item()
    assert (la - lb).abs().max().item() <= 1e-3


def test_runs_are_bitwise_deterministic():
    need_gpu()
    w = W.make_batched_sinks("cuda")
    a, la = run_decode(w)
    b, lb = run_decode(w)
    same_bits(a, b)
    assert torch.equal(la, lb)


def test_streaming_row_loads_match_plain_loads():
    """A call that can gather >= 256 MB of BF16 rows loads them with the
    non-temporal hint; the same tokens in a small call use plain loads.  The
    hint changes only cache placement, so both give identical bits."""
    need_gpu()
    T, K = 128, 2048                    # 128 x 2048 x 1 KB = 256 MB
    g = np.random.default_rng(11)
    idx = np.concatenate([
        np.stack([g.choice(600, 128, replace=False) for _ in range(T)]),
        np.stack([g.choice(4000, K - 128, replace=False) for _ in range(T)])],
        axis=1)
    lens = g.integers(1, K + 1, size=T)
    w = custom(idx, lens, swa_rows=600, comp_rows=4000, seed=21)
    n = 8
    small = W.Workload(
        name="custom8", T=n, H=w.H, K=K, q=w.q[:n].contiguous(), q_dtype=w.q_dtype,
        swa_pool=w.swa_pool, comp_pool=w.comp_pool, kv_dtype=w.kv_dtype,
        indices=w.indices[:n].contiguous(), topk_lens=w.topk_lens[:n].contiguous(),
        seq_lens=w.seq_lens[:n].contiguous(), cum_seq_lens_q=None, sinks=w.sinks,
        bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, lse_scale=w.lse_scale)
    for S in (1, 4):
        log(f"[parity] streaming vs plain loads: T={T} K={K} and T=8, {S} split(s)")
        big, lbig = run_decode(w, plan=L.plan_splits(T, 128, K, num_splits=S))
        out, lse = run_decode(small, plan=L.plan_splits(n, 128, K, num_splits=S))
        same_bits(out, big[:n], str(S))
        assert torch.equal(lse, lbig[:n]), S
    check(w, tokens=range(0, T, 16), plan=L.plan_splits(T, 128, K, num_splits=1),
          what="streaming loads vs oracle")


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("T", [256, 250])     # 250: XCD ranges of unequal size
def test_ragged_batch_order_does_not_change_any_token(T, H):
    """Workgroups start the items of their XCD longest first, so permuting
    the tokens of a ragged batch reassigns every item to another workgroup;
    each token's output and LSE must stay bit-identical (unsplit and split),
    and match the oracle on samples."""
    need_gpu()
    K = 2048
    g = np.random.default_rng(31)
    idx = np.concatenate([
        np.stack([g.choice(600, 128, replace=False) for _ in range(T)]),
        np.stack([g.choice(4000, K - 128, replace=False) for _ in range(T)])], axis=1)
    lens = g.integers(1, K + 1, size=T)
    w = custom(idx, lens, H=H, swa_rows=600, comp_rows=4000, seed=23)
    perm = torch.as_tensor(g.permutation(T)).cuda()
    wp = W.Workload(
        name="permuted", T=T, H=w.H, K=K, q=w.q[perm].contiguous(), q_dtype=w.q_dtype,
        swa_pool=w.swa_pool, comp_pool=w.comp_pool, kv_dtype=w.kv_dtype,
        indices=w.indices[perm].contiguous(), topk_lens=w.topk_lens[perm].contiguous(),
        seq_lens=w.seq_lens[perm].contiguous(), cum_seq_lens_q=None, sinks=w.sinks,
        bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale, lse_scale=w.lse_scale)
    for S in (1, 3):
        log(f"[parity] ragged batch T={T} H={H} permuted, {S} split(s)")
        plan = L.plan_splits(T, H, K, num_splits=S)
        a, la = run_decode(w, plan=plan)
        b, lb = run_decode(wp, plan=plan)
        same_bits(a[perm], b, str(S))
        assert torch.equal(la[perm], lb), S
    check(w, tokens=range(0, T, 32), what="ragged batch vs oracle")


def test_indices_past_topk_len_are_never_read():
    """Columns at or beyond topk_len hold indices far outside both pools;
    they must not be dereferenced (the result equals the table with those
    columns set to -1)."""
    need_gpu()
    rng = np.random.default_rng(8)
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 372))], 1).astype(np.int32)
    lens = [500, 300, 129, 200]
    garbage = idx.copy()
    for t, n in enumerate(lens):
        garbage[t, n:] = 2_000_000_000 - t
    w = custom(garbage, lens=lens)
    out, lse = run_decode(w)
    ref = oracle_for(custom(idx, lens=lens), range(4))
    compare(out, lse, ref, TOL_BF16, what="garbage past topk_len")


# ---------------------------------------------------------------------------
# validation mode and the combine kernel alone
# ---------------------------------------------------------------------------

def test_validate_flags_out_of_range_index_and_skips_it():
    need_gpu()
    rng = np.random.default_rng(9)
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 200))], 1).astype(np.int32)
    bad = idx.copy()
    bad[2, 150] = 900            # one past the compressed pool
    w = custom(bad)
    plan = L.plan_splits(4, 128, 328)
    ws = L.alloc_workspace(plan, 4, 128, L.FLAG_VALIDATE_INDICES)
    out, lse = run_decode(w, plan=plan, flags=L.FLAG_VALIDATE_INDICES,
                          workspace=ws)
    assert L.get_device_error(ws) == (1, 2, 150)
    masked = idx.copy()
    masked[2, 150] = -1
    ref = oracle_for(custom(masked), range(4))
    compare(out, lse, ref, TOL_BF16, what="validate: bad slot skipped")
    # a clean table clears the error block
    run_decode(custom(idx), plan=plan, flags=L.FLAG_VALIDATE_INDICES, workspace=ws)
    assert L.get_device_error(ws)[0] == 0
    # topk_len beyond the table width
    run_decode(custom(idx, lens=[328, 329, 10, 10]), plan=plan,
               flags=L.FLAG_VALIDATE_INDICES, workspace=ws)
    assert L.get_device_error(ws)[:2] == (2, 1)


@pytest.mark.parametrize("S,stride,H", [(1, 1, 64), (5, 8, 128), (16, 16, 128),
                                        (64, 64, 64)])
def test_combine_kernel_alone(S, stride, H):
    need_gpu()
    T = 6
    g = torch.Generator().manual_seed(S * 100 + H)
    mid_out = torch.randn((T, H, stride, 512), generator=g).to(torch.bfloat16)
    mid_lse = torch.randn((T, H, stride), generator=g) * 4
    mid_lse[0, :, : S // 2] = -math.inf       # some empty splits
    mid_lse[1] = -math.inf                    # a token with no rows at all
    sinks = torch.randn(H, generator=g)
    for sk in (sinks, None):
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, H), device="cuda")
        L.combine(mid_out.cuda(), mid_lse.cuda(), S, out, out_lse=lse,
                  sinks=None if sk is None else sk.cuda(), lse_scale=0.75)
        torch.cuda.synchronize()
        mo = W.raw_bits(mid_out[:, :, :S])
        ro, rl = oracle.combine(oracle.bf16_bits_to_f64(mo),
                                mid_lse[:, :, :S].double().numpy(),
                                None if sk is None else sk.numpy(), 0.75)
        compare(out, lse, {"out": ro, "lse": rl}, TOL_BF16,
                what=f"combine S={S} sink={sk is not None}")
