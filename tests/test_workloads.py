"""Seeded input generators: determinism and the table structure each
workload promises (CPU only, index tables without the large pools)."""

import numpy as np
import torch

from sparse_mla_decode_gather_amd import workloads as W


def test_tiny_is_deterministic_and_structured():
    a, b = W.make_tiny(), W.make_tiny()
    for x, y in [(a.q, b.q), (a.swa_pool, b.swa_pool), (a.comp_pool, b.comp_pool),
                 (a.indices, b.indices), (a.topk_lens, b.topk_lens)]:
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)
    idx = a.indices.numpy()
    assert idx.shape == (4, 256) and a.q.shape == (4, 64, 512)
    assert a.swa_pool.shape == (1024, 512) and a.comp_pool.shape == (4096, 512)
    for t in range(4):
        assert (idx[t] == -1).sum() == 13
        sw = idx[t, :128][idx[t, :128] >= 0]
        cp = idx[t, 128:][idx[t, 128:] >= 0]
        assert len(set(sw)) == len(sw) and sw.max() < 1024
        assert len(set(cp)) == len(cp) and cp.max() < 4096
    assert ((a.topk_lens >= 129) & (a.topk_lens <= 256)).all()
    assert a.sinks is None


def _swa_positions_ok(w, q_len):
    idx = w.indices.numpy()
    seq = w.meta["seq_lens"]
    for r, s in enumerate(seq):
        rows = [idx[r * q_len + i, :128] for i in range(q_len)]
        for i, rw in enumerate(rows):
            live = rw[rw >= 0]
            assert len(set(live.tolist())) == len(live) >= 100
            # consecutive positions in a page sit in consecutive rows
            pos = np.arange(s - q_len + i - 127, s - q_len + i + 1)
            same_page = (pos[1:] // 64) == (pos[:-1] // 64)
            both = (rw[1:] >= 0) & (rw[:-1] >= 0) & same_page
            assert np.all(np.diff(rw)[both] == 1)
        if q_len == 2:      # the two windows overlap by 127 positions
            a, b = rows[0][1:], rows[1][:-1]
            both = (a >= 0) & (b >= 0)
            assert np.array_equal(a[both], b[both])
    assert idx[:, :128].max() < w.meta["swa_rows"]


def _compressed_in_region(w, q_len):
    idx = w.indices.numpy()
    base = 0
    for r, s in enumerate(w.meta["seq_lens"]):
        reg = s // 4
        for i in range(q_len):
            c = idx[r * q_len + i, 128:]
            c = c[c >= 0]
            assert len(set(c.tolist())) == len(c)
            assert c.min() >= base and c.max() < base + reg
        base += reg
    assert base == w.meta["comp_rows"]


def test_batched_sinks_tables():
    w = W.make_batched_sinks(pools=False)
    assert w.indices.shape == (64, 512) and w.q.shape == (64, 128, 512)
    assert ((w.topk_lens >= 256) & (w.topk_lens <= 512)).all()
    assert (w.indices >= 0).all()
    assert all(4096 <= s <= 32768 for s in w.meta["seq_lens"])
    assert w.sinks.shape == (128,)
    _swa_positions_ok(w, 1)
    _compressed_in_region(w, 1)


def test_fp8_tables_and_scales():
    w = W.make_fp8(pools=False)
    assert w.q.dtype == torch.float8_e4m3fn and w.indices.shape == (128, 1024)
    assert (w.topk_lens == 1024).all() and (w.indices >= 0).all()
    assert abs(w.bmm1_scale - w.sm_scale * 0.05 * 0.08) < 1e-15
    assert w.bmm2_scale == 0.08
    _compressed_in_region(w, 1)


def test_long_context_tables():
    for T in (1, 4, 8):
        w = W.make_long_context(T, pools=False)
        assert w.indices.shape == (T, 2048) and (w.topk_lens == 2048).all()
        assert w.meta["comp_rows"] == T * 32768
        _swa_positions_ok(w, 1)
        _compressed_in_region(w, 1)


def test_spec_decode_tables():
    w = W.make_spec_decode(pools=False, B=32)
    idx = w.indices.numpy()
    assert idx.shape == (64, 2048) and w.cum_seq_lens_q.tolist()[-1] == 64
    assert all((idx[t] == -1).sum() == 41 for t in range(64))
    assert ((w.topk_lens >= 1024) & (w.topk_lens <= 2048)).all()
    assert w.q.dtype == torch.bfloat16 and w.kv_dtype == W.FP8
    assert w.bmm2_scale == 0.08
    shares = []
    for r in range(32):
        a = set(idx[2 * r, 128:].tolist()) - {-1}
        b = set(idx[2 * r + 1, 128:].tolist()) - {-1}
        shares.append(len(a & b) / 1920)
    assert 0.85 < np.mean(shares) < 0.95
    _swa_positions_ok(w, 2)


def test_fp8_quantisation_is_clamped_rne():
    x = W.normal_rows(64, seed=9, dtype=W.FP8, scale=0.08)
    ref = (W.normal_rows(64, seed=9, dtype=W.BF16).float() * 0 +
           torch.randn((64, 512), generator=torch.Generator().manual_seed(9)))
    want = (ref / 0.08).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert torch.equal(x.view(torch.uint8), want.view(torch.uint8))
