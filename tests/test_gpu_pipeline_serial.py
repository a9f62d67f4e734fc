"""LDS-race check of the kernels' tile pipelines, through the C ABI.

With SMLA_FLAG_SERIAL_PIPELINE the decode kernels finish every step of
their tile pipeline (row loads included) and meet at a barrier before the
next step starts; the arithmetic is the same instruction for instruction.
So the pipelined call, where the row loads of later tiles, the S^T products
of one tile and the O^T products and softmax of another overlap, must give
exactly the same bits: a difference would be one step disturbing another
(a stage overwritten while still read, a tile read before it landed, P^T
read before every wave wrote it).  Every kernel family is covered: H=128
with BF16 rows (LDS-DMA), FP8 rows with BF16 or FP8 q and packed rows
(register staging); H=64 with BF16 rows (LDS-DMA) and FP8 or packed rows
(register staging); unsplit and split; tile counts 1..5 and ragged tails;
and the full 64-tile loop.
"""

import numpy as np
import pytest
import torch

from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import log, need_gpu, run_decode, same_bits
from test_gpu_parity import custom

pytestmark = pytest.mark.gpu


def serial_equals_pipelined(w, splits, what):
    for S in splits:
        plan = L.plan_splits(w.T, w.H, w.K, L.dtype_code(w.q), L.dtype_code(w.swa_pool),
                             num_splits=S)
        log(f"[serial] {what}: T={w.T} H={w.H} K={w.K} S={plan.num_splits}")
        a, la = run_decode(w, plan=plan)
        b, lb = run_decode(w, plan=plan, flags=L.FLAG_SERIAL_PIPELINE)
        same_bits(a, b, f"{what} S={plan.num_splits}")
        assert torch.equal(la, lb), f"{what} S={plan.num_splits}: LSE bits differ"


def ragged_table(T, K, lens, swa_rows, comp_rows, seed):
    """Distinct rows per token, a few -1 slots, per-token lengths that give
    1..5 tiles with ragged tails."""
    g = np.random.default_rng(seed)
    idx = np.concatenate([
        np.stack([g.choice(swa_rows, 128, replace=False) for _ in range(T)]),
        np.stack([g.choice(comp_rows, K - 128, replace=False) for _ in range(T)])],
        axis=1).astype(np.int32)
    idx[:, 5::37] = -1
    return idx, np.asarray(lens[:T], np.int32)


LENS = [1, 31, 32, 33, 64, 65, 97, 150, 160, 300]


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("kv,q", [(W.BF16, W.BF16), (W.FP8, W.BF16), (W.FP8, W.FP8)])
def test_serial_pipeline_short_and_ragged(H, kv, q):
    need_gpu()
    idx, lens = ragged_table(10, 400, LENS, 600, 900, seed=H + 3)
    w = custom(idx, lens, H=H, kv=kv, q=q, seed=5)
    serial_equals_pipelined(w, (1, 3), f"ragged H={H} q={q} kv={kv}")


@pytest.mark.parametrize("H", [64, 128])
def test_serial_pipeline_packed_rows(H):
    need_gpu()
    w = W.make_packed(8, "cuda", H=H)
    serial_equals_pipelined(w, (1, 4), f"packed H={H}")


def test_serial_pipeline_full_tile_loop():
    """The steady 64-tile loop of the long-context shape (128 + 1920 rows,
    BF16, H=128), unsplit and split, and FP8 rows at the same length."""
    need_gpu()
    w = W.make_long_context(8, "cuda")
    serial_equals_pipelined(w, (1, 16), "long context BF16")
    w = W._decode_batch("fp8_rows_long", 9, "cuda", B=8, q_len=1, H=128, K=2048,
                        seq_lo=0, seq_hi=0, q_dtype=W.BF16, kv_dtype=W.FP8,
                        topk_lo=2048, topk_hi=2048, fixed_seq=131072, kv_scale=0.08)
    serial_equals_pipelined(w, (1,), "long context FP8 rows")


def test_serial_pipeline_configs():
    """The small configurations as they are benchmarked (default plans)."""
    need_gpu()
    for w in (W.make_tiny("cuda"), W.make_fp8("cuda"), W.make_spec_decode("cuda", B=16)):
        serial_equals_pipelined(w, (0,), w.name)
