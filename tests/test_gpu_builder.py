"""GPU: sparse_mla_build_indices through the C ABI against the CPU oracle's
builder, bit for bit (it is integer work), and the built table fed to the
decode.  The builder (vLLM DeepseekV4FlashInferMLAAttention,
_build_sparse_index_metadata, feeding FlashInfer
trtllm_batch_decode_sparse_mla_dsv4's sparse_indices / sparse_topk_lens)
translates request-local compressed positions through a block table with
the canonical page expansion page_id * page_size + offset.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_decode_gather_amd import lib as L
from sparse_mla_decode_gather_amd import workloads as W

from parity_utils import same_bits, log, need_gpu, run_decode

pytestmark = pytest.mark.gpu


def case(seed, T=6, Wd=128, K2=300, B=3, max_blocks=10, ps=16, local=True,
         bad=True, lens=True, valid=True, q_len=2):
    rng = np.random.default_rng(seed)
    swa = rng.integers(-1, 5000, (T, Wd)).astype(np.int32)
    n = max_blocks * ps
    comp = rng.integers(0, n, (T, K2)).astype(np.int32) if local else \
        rng.integers(0, 1 << 20, (T, K2)).astype(np.int32)
    if K2:
        comp[rng.random((T, K2)) < 0.05] = -1
    bt = np.stack([rng.permutation(200)[:max_blocks] for _ in range(B)]).astype(np.int32)
    tok2req = (np.arange(T) // q_len).astype(np.int32) % B
    if bad and local and K2:
        comp[0, 0] = n + 3               # page index past the table
        bt[0, 1] = -4                    # a negative page id
        tok2req[-1] = B + 1              # a request outside the table
    cl = rng.integers(-2, K2 + 5, T).astype(np.int32) if lens else None
    vt = (rng.random(T) > 0.2).astype(np.int32) if valid else None
    return dict(swa=swa, comp=comp, bt=bt, ps=ps, local=local, tok2req=tok2req,
                cl=cl, vt=vt)


def reference(c):
    return oracle.build_combined_indices(
        c["swa"], c["comp"], local=c["local"], page_size=c["ps"], block_tables=c["bt"],
        token_to_req=c["tok2req"], comp_topk_lens=c["cl"], valid_tokens=c["vt"])


def gpu(c, with_err=True, out_stride_pad=0):
    d = lambda a: None if a is None else torch.from_numpy(a).cuda()
    T = c["swa"].shape[0]
    K = c["swa"].shape[1] + c["comp"].shape[1]
    out = torch.full((T, K + out_stride_pad), 12345, dtype=torch.int32, device="cuda")
    err = torch.full((4,), 77, dtype=torch.int32, device="cuda") if with_err else None
    idx, lens = L.build_indices(
        d(c["swa"]) if c["swa"].shape[1] else None,
        d(c["comp"]) if c["comp"].shape[1] else None, comp_local=c["local"],
        comp_topk_lens=d(c["cl"]), block_tables=d(c["bt"]), page_size=c["ps"],
        token_to_req=d(c["tok2req"]), valid_tokens=d(c["vt"]),
        out=out[:, :K], err=err)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), lens.cpu().numpy(), out, err


@pytest.mark.parametrize("kw", [
    dict(), dict(local=False), dict(Wd=0), dict(K2=0), dict(Wd=7, K2=1),
    dict(lens=False, valid=False, bad=False), dict(T=33, K2=1920, max_blocks=40, ps=64),
    dict(ps=1, max_blocks=300), dict(K2=257, ps=5),
])
def test_build_matches_oracle_bit_for_bit(kw):
    need_gpu()
    c = case(3, **kw)
    log(f"[builder] case {kw}")
    ref_idx, ref_lens, bad = reference(c)
    idx, lens, out, err = gpu(c, out_stride_pad=5)
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(lens, ref_lens)
    assert (out[:, idx.shape[1]:] == 12345).all()      # padding columns untouched
    e = err.cpu().numpy()
    if bad:
        assert e[0] == 1 and (int(e[1]), int(e[2])) in bad
    else:
        assert e[0] == 0 and e[1] == -1 and e[2] == -1


def test_build_at_the_headline_size():
    need_gpu()
    T, K2, ps, blocks = 512, 1920, 64, 512    # 32768 compressed rows per request
    rng = np.random.default_rng(8)
    swa = rng.integers(0, 1 << 16, (T, 128)).astype(np.int32)
    comp = np.stack([rng.choice(blocks * ps, K2, replace=False) for _ in range(T)]).astype(np.int32)
    bt = np.stack([rng.permutation(T * blocks)[:blocks] for _ in range(T)]).astype(np.int32)
    c = dict(swa=swa, comp=comp, bt=bt, ps=ps, local=True, tok2req=None, cl=None, vt=None)
    log("[builder] headline size T=512 W=128 K2=1920")
    ref_idx, ref_lens, bad = reference(c)
    idx, lens, _, err = gpu(c)
    assert bad == [] and np.array_equal(idx, ref_idx) and np.array_equal(lens, ref_lens)
    assert int(err[0].item()) == 0


def test_built_table_feeds_the_decode_like_the_page_table_form():
    """Positions 0..n-1 in order: the built combined table decodes to the same
    bits as the page-table call on the same block table, and within tolerance
    of the oracle's decode of the oracle-built table."""
    need_gpu()
    T, pages, ps = 6, 30, 64
    w = W.make_long_context(T, "cuda")       # pools sized for 128 + 1920 rows
    rng = np.random.default_rng(4)
    region = w.comp_pool.shape[0] // ps
    bt = np.stack([rng.permutation(region)[:pages] for _ in range(T)]).astype(np.int32)
    comp = np.tile(np.arange(pages * ps, dtype=np.int32), (T, 1))
    cl = rng.integers(0, pages * ps + 1, T).astype(np.int32)
    swa = w.indices[:, :128].contiguous()
    idx, lens = L.build_indices(swa, torch.from_numpy(comp).cuda(), comp_local=True,
                                comp_topk_lens=torch.from_numpy(cl).cuda(),
                                block_tables=torch.from_numpy(bt).cuda(), page_size=ps)
    log(f"[builder] built table -> decode, T={T}")
    wb = W.Workload(name="built", T=T, H=w.H, K=idx.shape[1], q=w.q, q_dtype=w.q_dtype,
                    swa_pool=w.swa_pool, comp_pool=w.comp_pool, kv_dtype=w.kv_dtype,
                    indices=idx, topk_lens=lens, seq_lens=w.seq_lens, cum_seq_lens_q=None,
                    sinks=w.sinks, bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                    lse_scale=w.lse_scale)
    plan = L.plan_splits(T, w.H, idx.shape[1], num_splits=4)
    out, lse = run_decode(wb, plan=plan)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    L.decode_paged(w.q, w.swa_pool, w.comp_pool, swa, torch.from_numpy(bt).cuda(), ps,
                   out2, topk_lens=lens, out_lse=lse2, sinks=w.sinks,
                   bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                   lse_scale=w.lse_scale, plan=plan)
    torch.cuda.synchronize()
    same_bits(out, out2)
    assert torch.equal(lse, lse2)
    ref_idx, ref_lens, _ = oracle.build_combined_indices(
        swa.cpu().numpy(), comp, local=True, page_size=ps, block_tables=bt,
        comp_topk_lens=cl)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.array_equal(lens.cpu().numpy(), ref_lens)


def test_graph_replays_of_the_builder_match_eager():
    """The builder with an error block (cleared by a kernel, not a memset)
    captured into a HIP graph and replayed four times, with eager work and
    synchronisation in between, gives the eager result every time."""
    need_gpu()
    c = case(12, T=9, K2=700)
    d = lambda a: torch.from_numpy(a).cuda()
    T, K = c["swa"].shape[0], c["swa"].shape[1] + c["comp"].shape[1]
    args = [d(c["swa"]), d(c["comp"]), d(c["cl"]), d(c["bt"]), d(c["tok2req"]), d(c["vt"])]
    out = torch.empty((T, K), dtype=torch.int32, device="cuda")
    lens = torch.empty((T,), dtype=torch.int32, device="cuda")
    err = torch.empty((4,), dtype=torch.int32, device="cuda")

    def call():
        L.build_indices(args[0], args[1], comp_local=True, comp_topk_lens=args[2],
                        block_tables=args[3], page_size=c["ps"], token_to_req=args[4],
                        valid_tokens=args[5], out=out, out_topk_lens=lens, err=err)
    log("[builder] graph replays T=9")
    call()
    torch.cuda.synchronize()
    ref = (out.clone(), lens.clone(), err.clone())
    assert int(ref[2][0].item()) == 1          # the case has untranslatable entries
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up off the capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(7)                           # eager work between replays
        lens.fill_(7)
        err.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lens, ref[1]), rep
        assert int(err[0].item()) == 1, rep
