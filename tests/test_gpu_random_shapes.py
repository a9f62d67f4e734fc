"""Seeded random shapes against the oracle, element by element, through the
C ABI: both head counts, every (q, rows) format pair, table widths below
and above the 128 SWA columns and off the 64-column chunk grid, pools of a
few rows (so indices repeat), -1 densities from none to all, lengths from
0 to K or none, with and without sinks, and planner-chosen, unsplit or
random split counts.  Each case prints its parameters before it runs."""

import math

import numpy as np
import pytest
import torch

from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import TOL_BF16, TOL_FP8, compare, log, need_gpu, oracle_for, run_decode

pytestmark = pytest.mark.gpu

PAIRS = [(W.BF16, W.BF16), (W.BF16, W.FP8), (W.FP8, W.FP8), (W.BF16, W.PACKED)]


def random_case(seed):
    rng = np.random.default_rng(seed)
    H = int(rng.choice([64, 128]))
    q_dt, kv_dt = PAIRS[int(rng.integers(len(PAIRS)))]
    T = int(rng.integers(1, 9))
    K = int(rng.integers(1, 128)) if rng.random() < 0.3 else int(rng.integers(128, 700))
    swa_rows = int(rng.integers(1, 300))
    comp_rows = int(rng.integers(1, 2000))
    k1 = min(K, 128)
    idx = np.empty((T, K), np.int32)
    idx[:, :k1] = rng.integers(0, swa_rows, (T, k1))
    if K > k1:
        idx[:, k1:] = rng.integers(0, comp_rows, (T, K - k1))
    neg = float(rng.choice([0.0, 0.05, 0.5, 1.0]))
    idx[rng.random((T, K)) < neg] = -1
    lens = None if rng.random() < 0.3 else rng.integers(0, K + 1, T).astype(np.int32)
    sinks = bool(rng.random() < 0.5)
    nch = -(-K // 64)
    S = int(rng.choice([0, 1, int(rng.integers(1, nch + 1))]))

    def pool(rows, sd):
        if kv_dt == W.PACKED:
            return W.packed_rows(rows, sd, "cuda")
        return W.normal_rows(rows, sd, "cuda", kv_dt, scale=0.08 if kv_dt == W.FP8 else 1.0)
    qs = 0.05 if q_dt == W.FP8 else 1.0
    ks = 0.08 if kv_dt == W.FP8 else 1.0
    g = torch.Generator().manual_seed(seed)
    w = W.Workload(
        name=f"random{seed}", T=T, H=H, K=K,
        q=W.normal_rows(T * H, seed + 1, "cuda", q_dt,
                        scale=qs if q_dt == W.FP8 else 1.0).view(T, H, 512),
        q_dtype=q_dt, swa_pool=pool(swa_rows, seed + 2),
        comp_pool=pool(comp_rows, seed + 3) if K > 128 else None,
        kv_dtype=kv_dt, indices=torch.as_tensor(idx).cuda(),
        topk_lens=None if lens is None else torch.as_tensor(lens).cuda(),
        seq_lens=torch.full((T,), 4096, dtype=torch.int32, device="cuda"),
        cum_seq_lens_q=None,
        sinks=torch.randn(H, generator=g).cuda() if sinks else None,
        bmm1_scale=qs * ks / math.sqrt(512), bmm2_scale=ks, lse_scale=1.0)
    desc = (f"seed={seed} T={T} H={H} K={K} q={q_dt} kv={kv_dt} swa_rows={swa_rows} "
            f"comp_rows={comp_rows} neg={neg} lens={'none' if lens is None else 'given'} "
            f"sinks={sinks} S={S or 'planner'}")
    return w, S, desc


@pytest.mark.parametrize("seed", range(64))
def test_random_shape_matches_oracle(seed):
    need_gpu()
    w, S, desc = random_case(5000 + seed)
    log(f"[random] {desc}")
    plan = L.plan_splits(w.T, w.H, w.K, L.dtype_code(w.q), L.dtype_code(w.swa_pool),
                         num_splits=S)
    out, lse = run_decode(w, plan=plan)
    tol = TOL_BF16 if w.kv_dtype == W.BF16 else TOL_FP8
    compare(out, lse, oracle_for(w, range(w.T)), tol, what=desc)
