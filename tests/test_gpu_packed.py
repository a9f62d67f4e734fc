"""Packed block-scaled FP8 rows (584 bytes) on the GPU, through the C ABI,
against the oracle's decode of the same bytes.

* Single active slot, no sink: the output is the decoded row itself, which
  is exactly a BF16 row, so the GPU result must equal it bit for bit --
  this pins the byte layout, the per-block scale selection and the RoPE
  lanes' stores of the kernels, for both head counts, split and unsplit, at
  the first and last rows of both pools, for scale bytes far from 127 and
  for scale bytes at both ends of the UE8M0 range (0..2, 252..254).
* Element-wise parity (the FP8 bar, 3e-2 + 3e-2*|ref|, LSE 1e-3) with
  ragged lengths, -1 slots, several table segments, padded rows, the
  two-segment and page-table forms, and every token of the full-size
  long-context shape (T=512, H=128, topk 2048).
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import TOL_FP8, compare, log, need_gpu, oracle_for, run_decode

pytestmark = pytest.mark.gpu

PK = L.DTYPE_PACKED_FP8_584


def wl(idx, lens=None, H=128, swa=None, comp=None, sinks=True, seed=0, b1=0.04, b2=1.0,
       name="packed", q_zero=False):
    idx = torch.as_tensor(np.asarray(idx, np.int32))
    T, K = idx.shape
    g = torch.Generator().manual_seed(seed + 7)
    return W.Workload(
        name=name, T=T, H=H, K=K,
        q=(torch.zeros((T, H, 512), dtype=torch.bfloat16, device="cuda") if q_zero else
           W.normal_rows(T * H, seed + 1, "cuda", scale=1.0).view(T, H, 512) * 0.25),
        q_dtype=W.BF16, swa_pool=swa, comp_pool=comp, kv_dtype=W.PACKED,
        indices=idx.cuda(),
        topk_lens=None if lens is None else torch.as_tensor(np.asarray(lens, np.int32)).cuda(),
        seq_lens=torch.full((T,), 4096, dtype=torch.int32, device="cuda"),
        cum_seq_lens_q=None,
        sinks=torch.randn(H, generator=g).cuda() if sinks else None,
        bmm1_scale=b1, bmm2_scale=b2)


def extreme_rows(n, seed):
    """Packed rows whose scale bytes span 60..190 (every scaled value still a
    normal BF16 number)."""
    rows = W.packed_rows(n, seed, "cpu")
    g = torch.Generator().manual_seed(seed)
    rows[:, 576:] = torch.randint(60, 191, (n, 8), generator=g).to(torch.uint8)
    return rows


@pytest.mark.parametrize("H", [64, 128])
def test_single_slot_is_the_decoded_row_bit_for_bit(H):
    need_gpu()
    swa = extreme_rows(300, 3).cuda()
    comp = extreme_rows(500, 4).cuda()
    T, K = 10, 300
    idx = np.full((T, K), -1, np.int32)
    picks = [(0, 0), (1, 299), (5, 17), (127, 150), (64, 42)]          # SWA (col, row)
    picks += [(128, 0), (129, 499), (200, 250), (299, 1), (250, 498)]  # compressed
    for t, (c, r) in enumerate(picks):
        idx[t, c] = r
    # q = 0: the single logit is 0 whatever the row's magnitude (the rows
    # reach ~4e21), so out_lse is exactly 0
    w = wl(idx, H=H, swa=swa, comp=comp, sinks=False, q_zero=True)
    want = oracle.packed584_to_f64(np.concatenate(
        [W.raw_bits(swa[[r]]) if c < 128 else W.raw_bits(comp[[r]]) for c, r in picks]))
    assert np.array_equal(oracle.round_to_bf16(want), want)
    for S in (1, 3):
        log(f"[packed] single slot H={H} S={S}")
        out, lse = run_decode(w, plan=L.plan_splits(T, H, K, L.DTYPE_BF16, PK, num_splits=S))
        o = out.float().cpu().numpy()
        for t in range(T):
            assert np.array_equal(o[t], np.tile(want[t], (H, 1))), (H, S, t)
        assert np.all(lse.cpu().numpy() == 0.0), (H, S)
        ref = oracle_for(w, range(T))
        compare(out, lse, ref, TOL_FP8, what=f"packed single slot H={H} S={S}")


def edge_scale_rows(seed):
    """Rows whose scale bytes sit at the ends of the UE8M0 range, with codes
    that keep every decoded value a normal BF16 number: scale bytes 0..2
    (2^-127..2^-125) with codes of magnitude >= 2 (E4M3FN exponent field >=
    8) and scale bytes 252..254 with codes below 2 (field <= 7), one row of
    each kind and one alternating them block by block."""
    rng = np.random.default_rng(seed)
    rows = W.packed_rows(3, seed, "cpu").numpy().copy()

    def codes(n, big):
        ex = rng.integers(8, 16, n) if big else rng.integers(0, 8, n)
        man = rng.integers(0, 8, n)
        man = np.where((ex == 15) & (man == 7), 6, man)      # 0x7F / 0xFF are NaN
        return ((rng.integers(0, 2, n) << 7) | (ex << 3) | man).astype(np.uint8)
    lows, highs = rng.integers(0, 3, 8), rng.integers(252, 255, 8)
    for r, kinds in enumerate(([True] * 8, [False] * 8, [j % 2 == 0 for j in range(8)])):
        for j, big in enumerate(kinds):
            rows[r, 56 * j:56 * j + 56] = codes(56, big)
            rows[r, 576 + j] = lows[j] if big else highs[j]
    return torch.from_numpy(rows)


@pytest.mark.parametrize("H", [64, 128])
def test_scale_bytes_at_the_range_ends_decode_exactly(H):
    """UE8M0 bytes 0..2 and 252..254 (reading S20: 2^(e-127)): the single
    active slot returns the decoded row bit for bit, so byte 0 scales by
    2^-127 (not 0) and byte 254 by 2^127."""
    need_gpu()
    rows = edge_scale_rows(31)
    want = oracle.packed584_to_f64(W.raw_bits(rows))
    assert np.all(np.isfinite(want)) and np.array_equal(oracle.round_to_bf16(want), want)
    assert np.all(np.abs(want[:, :448][want[:, :448] != 0]) >= 2.0 ** -126)
    swa = rows.cuda()
    comp = rows.flip(0).contiguous().cuda()
    T, K = 6, 160
    idx = np.full((T, K), -1, np.int32)
    picks = [(0, 0), (5, 1), (127, 2), (128, 2), (140, 1), (159, 0)]   # (col, pool row)
    for t, (c, r) in enumerate(picks):
        idx[t, c] = r
    w = wl(idx, H=H, swa=swa, comp=comp, sinks=False, q_zero=True)
    expect = [want[r] if c < 128 else want[2 - r] for c, r in picks]
    for S in (1, 2):
        log(f"[packed] scale-byte ends H={H} S={S}")
        out, lse = run_decode(w, plan=L.plan_splits(T, H, K, L.DTYPE_BF16, PK, num_splits=S))
        o = out.float().cpu().numpy()
        for t in range(T):
            assert np.array_equal(o[t], np.tile(expect[t], (H, 1))), (H, S, t)
        assert np.all(lse.cpu().numpy() == 0.0), (H, S)


@pytest.mark.parametrize("H", [64, 128])
def test_packed_edges_match_oracle(H):
    need_gpu()
    rng = np.random.default_rng(21)
    swa = W.packed_rows(600, 11, "cuda")
    comp = W.packed_rows(900, 12, "cuda")
    T, K = 12, 700
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 900, (T, K - 128))], 1).astype(np.int32)
    idx[3, :] = -1
    idx[5, ::3] = -1
    idx[6, 200:230] = idx[6, 300]
    lens = [0, 1, 31, 32, 33, 127, 128, 129, 700, 650, 64, 97]
    w = wl(idx, lens=lens, H=H, swa=swa, comp=comp)
    for S in (1, 5):
        log(f"[packed] edges H={H} S={S}")
        out, lse = run_decode(w, plan=L.plan_splits(T, H, K, L.DTYPE_BF16, PK, num_splits=S))
        e, le = compare(out, lse, oracle_for(w, range(T)), TOL_FP8,
                        what=f"packed edges H={H} S={S}")
        log(f"[packed] edges H={H} S={S}: max|out err| {e:.3g} max|lse err| {le:.3g}")
    # several table segments
    T, K = 3, 5000
    comp2 = W.packed_rows(20000, 13, "cuda")
    idx = np.concatenate([rng.integers(0, 600, (T, 128)),
                          rng.integers(0, 20000, (T, K - 128))], 1).astype(np.int32)
    idx[1, 4000:] = -1
    w = wl(idx, lens=[5000, 4500, 2100], H=H, swa=swa, comp=comp2)
    out, lse = run_decode(w, plan=L.plan_splits(T, H, K, L.DTYPE_BF16, PK, num_splits=1))
    compare(out, lse, oracle_for(w, range(T)), TOL_FP8, what=f"packed K=5000 H={H}")


@pytest.mark.parametrize("H", [64, 128])
def test_packed_padded_rows(H):
    """Rows 592 bytes apart (8 bytes of padding): every load starts at its
    row's own address."""
    need_gpu()
    rng = np.random.default_rng(4)

    def padded(n, seed):
        big = torch.zeros((n, 592), dtype=torch.uint8, device="cuda")
        big[:, :584] = W.packed_rows(n, seed, "cuda")
        return big[:, :584]
    swa, comp = padded(600, 31), padded(900, 32)
    assert swa.stride(0) == 592
    idx = np.concatenate([rng.integers(0, 600, (4, 128)),
                          rng.integers(0, 900, (4, 200))], 1).astype(np.int32)
    w = wl(idx, H=H, swa=swa, comp=comp)
    out, lse = run_decode(w)
    compare(out, lse, oracle_for(w, range(4)), TOL_FP8, what=f"packed stride 592 H={H}")


@pytest.mark.parametrize("H", [64, 128])
def test_packed_two_segment_and_paged_forms(H):
    """The general table views with packed rows: bit-identical to the
    combined call on the same slots, and within the bar of the oracle."""
    need_gpu()
    rng = np.random.default_rng(8)
    swa = W.packed_rows(600, 41, "cuda")
    comp = W.packed_rows(64 * 20, 42, "cuda")
    T = 4
    swa_tab = rng.integers(0, 600, (T, 128)).astype(np.int32)
    pages = np.stack([rng.permutation(20)[:6] for _ in range(T)]).astype(np.int32)
    comp_tab = (pages[:, :, None] * 64 + np.arange(64)[None, None, :]).reshape(T, -1)
    comb = np.concatenate([swa_tab, comp_tab], 1).astype(np.int32)
    w = wl(comb, H=H, swa=swa, comp=comp)
    out, lse = run_decode(w)
    compare(out, lse, oracle_for(w, range(T)), TOL_FP8, what=f"packed combined H={H}")
    o2 = torch.full_like(out, float("nan"))
    l2 = torch.full_like(lse, float("nan"))
    L.decode_segments(w.q, swa, comp, torch.from_numpy(swa_tab).cuda(),
                      torch.from_numpy(comp_tab.astype(np.int32)).cuda(), o2, out_lse=l2,
                      sinks=w.sinks, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
    o3 = torch.full_like(out, float("nan"))
    l3 = torch.full_like(lse, float("nan"))
    L.decode_paged(w.q, swa, comp, torch.from_numpy(swa_tab).cuda(),
                   torch.from_numpy(pages).cuda(), 64, o3, out_lse=l3,
                   sinks=w.sinks, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale)
    torch.cuda.synchronize()
    from parity_utils import same_bits
    same_bits(o2, out, f"packed two-segment vs combined H={H}")
    same_bits(o3, out, f"packed page table vs combined H={H}")
    assert torch.equal(l2, lse) and torch.equal(l3, lse)


def test_packed_full_size_every_token():
    """T=512, H=128, topk 2048 (128 SWA + 1920 compressed), 128k context,
    packed rows, planner default: every token against the oracle."""
    need_gpu()
    w = W.make_packed(512, "cuda")
    log(f"[packed] full size T={w.T} H={w.H} K={w.K}")
    out, lse = run_decode(w)
    e, le = compare(out, lse, oracle_for(w, range(w.T)), TOL_FP8, what="packed T=512")
    log(f"[packed] full size: max|out err| {e:.3g} max|lse err| {le:.3g}")
    w64 = W.make_packed(64, "cuda", H=64)
    out, lse = run_decode(w64)
    compare(out, lse, oracle_for(w64, range(w64.T)), TOL_FP8, what="packed T=64 H=64")
