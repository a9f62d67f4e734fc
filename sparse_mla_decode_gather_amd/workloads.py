"""Seeded synthetic inputs for sparse MLA decode (DeepSeek-V4 style).

This module only draws random inputs: query rows, the two KV pools, the
combined index table and its per-token lengths, sinks and scales.  It holds
none of the attention arithmetic, so both the GPU path and the CPU oracle can
consume what it produces without sharing any of the method's code.

The shapes follow the workloads the pages describe:

* FlashInfer ``trtllm_batch_decode_sparse_mla_dsv4`` (introduction and the
  ``query`` / ``sparse_indices`` / ``sparse_topk_lens`` parameters): head dim
  512, the first 128 table columns index the SWA pool, the rest the compressed
  pool, and each token's top-k length counts the 128 SWA columns.
* FlashInfer ``cake_sparse_mla_sm120_dsv4_nvfp4_decode`` (``q`` parameter):
  448 NoPE dims followed by 64 RoPE dims; ``indices``: -1 masks a slot.
* vLLM ``deepseek_v4/nvidia/flashinfer_sparse``
  (``DeepseekV4FlashInferMLAAttention._build_sparse_index_metadata``): the
  compressed block is the KV block divided by the compress ratio (4 here).

There are no real DeepSeek-V4 latents, weights or indexer outputs here, so
N(0,1) values and uniformly drawn distinct rows stand in for them.  The SWA
pool is paged (64-row pages whose physical IDs are a seeded permutation), and
an SWA row index is ``page_id * 64 + position % 64``, the canonical page
expansion the FlashInfer page describes for ``hca_sparse_indices_format``.

FP8 inputs are produced by torch's own float8_e4m3fn cast (round to nearest
even) after clamping x/scale to the format's +-448 range; the consumers only
ever see the resulting bytes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

HEAD_DIM = 512          # 448 NoPE + 64 RoPE, shared by q and both pools
SWA_COLUMNS = 128       # fixed SWA segment width of the combined table
SWA_PAGE = 64           # page size of the paged SWA pool
COMPRESS_RATIO = 4      # compressed pool: seq_len // 4 rows per request
E4M3_MAX = 448.0

BF16 = "bf16"
FP8 = "fp8_e4m3fn"
PACKED = "packed_fp8_584"   # 584-byte rows: 448 E4M3FN + 64 BF16 + 8 UE8M0 bytes

PACKED_ROW_BYTES = 584
PACKED_BLOCKS = 8           # UE8M0 scale bytes per row, one per 56 NoPE dims
PACKED_BLOCK_DIMS = 56


@dataclass
class Workload:
    """One batch of decode inputs.  Tensors live on ``device``."""

    name: str
    T: int
    H: int
    K: int
    q: torch.Tensor                 # [T, H, 512] bf16 or float8_e4m3fn
    q_dtype: str
    swa_pool: torch.Tensor          # [swa_rows, 512]
    comp_pool: torch.Tensor         # [comp_rows, 512]
    kv_dtype: str
    indices: torch.Tensor           # [T, K] int32
    topk_lens: Optional[torch.Tensor]   # [T] int32 or None (every column)
    seq_lens: torch.Tensor          # [B] int32
    cum_seq_lens_q: Optional[torch.Tensor]  # [B+1] int32 or None
    sinks: Optional[torch.Tensor]   # [H] fp32 or None
    bmm1_scale: float
    bmm2_scale: float
    lse_scale: float = 1.0
    q_scale: float = 1.0
    kv_scale: float = 1.0
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    meta: dict = field(default_factory=dict)

    @property
    def num_requests(self) -> int:
        return int(self.seq_lens.numel())

    def to(self, device) -> "Workload":
        def mv(x):
            return None if x is None else x.to(device)
        return Workload(
            name=self.name, T=self.T, H=self.H, K=self.K, q=mv(self.q),
            q_dtype=self.q_dtype, swa_pool=mv(self.swa_pool),
            comp_pool=mv(self.comp_pool), kv_dtype=self.kv_dtype,
            indices=mv(self.indices), topk_lens=mv(self.topk_lens),
            seq_lens=mv(self.seq_lens), cum_seq_lens_q=mv(self.cum_seq_lens_q),
            sinks=mv(self.sinks), bmm1_scale=self.bmm1_scale,
            bmm2_scale=self.bmm2_scale, lse_scale=self.lse_scale,
            q_scale=self.q_scale, kv_scale=self.kv_scale,
            sm_scale=self.sm_scale, meta=dict(self.meta))


# ---------------------------------------------------------------------------
# random building blocks
# ---------------------------------------------------------------------------

def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal_rows(rows: int, seed: int, device="cpu", dtype: str = BF16,
                scale: float = 1.0, chunk_rows: int = 1 << 18) -> torch.Tensor:
    """[rows, 512] N(0,1) values stored as bf16, or quantised to E4M3FN bytes
    as clamp(x / scale, +-448) rounded to nearest even.  Generated in chunks
    on ``device`` with a seeded generator of that device."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out_dtype = torch.bfloat16 if dtype == BF16 else torch.float8_e4m3fn
    out = torch.empty((rows, HEAD_DIM), dtype=out_dtype, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, HEAD_DIM), generator=g, device=device,
                        dtype=torch.float32)
        if dtype == BF16:
            out[r0:r1] = x.to(torch.bfloat16)
        else:
            out[r0:r1] = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(
                torch.float8_e4m3fn)
        del x
    return out


def packed_rows(rows: int, seed: int, device="cpu", chunk_rows: int = 1 << 17,
                spread: int = 1) -> torch.Tensor:
    """[rows, 584] uint8 packed block-scaled FP8 rows, written the way a KV
    cache writer would fill them (the layout the library and the oracle read:
    bytes 0..447 E4M3FN NoPE codes, 448..575 the 64 RoPE dims as BF16,
    576..583 one UE8M0 scale byte per 56 NoPE dims).  Values are N(0,1),
    each 56-dim NoPE block multiplied by a seeded 2^k, k uniform in
    [-spread, spread] (default 1: magnitudes stay those of N(0,1) latents
    within a factor 2, the scale bytes vary from block to block); a block's
    scale is the
    smallest power of two 2^(e-127) with max|x| / 2^(e-127) <= 448, and its
    codes are torch's float8_e4m3fn cast of x / 2^(e-127)."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((rows, PACKED_ROW_BYTES), dtype=torch.uint8, device=device)
    nope = PACKED_BLOCKS * PACKED_BLOCK_DIMS
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        n = r1 - r0
        x = torch.randn((n, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
        k = torch.randint(-spread, spread + 1, (n, PACKED_BLOCKS, 1), generator=g,
                          device=device).float()
        blocks = x[:, :nope].view(n, PACKED_BLOCKS, PACKED_BLOCK_DIMS) * torch.exp2(k)
        amax = blocks.abs().amax(-1, keepdim=True).clamp_min(2.0 ** -100)
        e = (torch.ceil(torch.log2(amax / E4M3_MAX)) + 127).clamp_(1, 254)
        codes = (blocks / torch.exp2(e - 127)).clamp_(-E4M3_MAX, E4M3_MAX).to(
            torch.float8_e4m3fn).view(torch.uint8)
        out[r0:r1, :nope] = codes.reshape(n, nope)
        out[r0:r1, nope:nope + 128] = x[:, nope:].to(torch.bfloat16).contiguous().view(
            torch.uint8).view(n, 128)
        out[r0:r1, nope + 128:] = e.view(n, PACKED_BLOCKS).to(torch.uint8)
        del x, blocks, codes
    return out


def pool_rows(rows: int, seed: int, device="cpu", dtype: str = BF16,
              scale: float = 1.0) -> torch.Tensor:
    """A KV pool of ``rows`` rows in ``dtype`` (see normal_rows and
    packed_rows)."""
    if dtype == PACKED:
        return packed_rows(rows, seed, device)
    return normal_rows(rows, seed, device, dtype, scale)


def _distinct(g: torch.Generator, n: int, k: int) -> torch.Tensor:
    """k distinct integers drawn uniformly from [0, n)."""
    assert k <= n
    return torch.randperm(n, generator=g)[:k]


def _uniform_int(g: torch.Generator, lo: int, hi: int, size) -> torch.Tensor:
    """Integers uniform on the closed range [lo, hi]."""
    return torch.randint(lo, hi + 1, size, generator=g)


def _paged_swa(g: torch.Generator, spans):
    """Lay out each request's SWA positions in a paged pool.

    ``spans[r] = (lo, hi)`` is the half-open range of positions that the
    SWA windows of request r's tokens cover.  Every 64-position logical page
    touched by a span gets its own physical page, numbered by a seeded
    permutation.  Returns a function mapping (request, position) to a
    physical row, and the pool row count.
    """
    pages = []           # (request, logical page)
    for r, (lo, hi) in enumerate(spans):
        for lp in range(lo // SWA_PAGE, (hi - 1) // SWA_PAGE + 1):
            pages.append((r, lp))
    perm = torch.randperm(len(pages), generator=g).tolist()
    table = {pg: perm[i] for i, pg in enumerate(pages)}

    def row_of(r: int, pos: int) -> int:
        return table[(r, pos // SWA_PAGE)] * SWA_PAGE + pos % SWA_PAGE

    return row_of, len(pages) * SWA_PAGE


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def make_tiny(device="cpu", seed: int = 1) -> Workload:
    """Tiny decode: T=4, H=64, SWA pool 1024 rows, compressed pool 4096 rows,
    table [4,256] of distinct random rows (128 + 128), exactly 13 slots per
    token (5% of 256) set to -1, topk_len ~ U{129..256}, no sink."""
    T, H, K = 4, 64, 256
    g = _cpu_gen(seed)
    swa_rows, comp_rows = 1024, 4096
    idx = torch.empty((T, K), dtype=torch.int32)
    for t in range(T):
        idx[t, :SWA_COLUMNS] = _distinct(g, swa_rows, SWA_COLUMNS).int()
        idx[t, SWA_COLUMNS:] = _distinct(g, comp_rows, K - SWA_COLUMNS).int()
        idx[t, _distinct(g, K, 13)] = -1
    topk = _uniform_int(g, 129, 256, (T,)).int()
    q = normal_rows(T * H, seed * 1000 + 1, device).view(T, H, HEAD_DIM)
    sm = 1.0 / math.sqrt(HEAD_DIM)
    return Workload(
        name="tiny", T=T, H=H, K=K, q=q, q_dtype=BF16,
        swa_pool=normal_rows(swa_rows, seed * 1000 + 2, device),
        comp_pool=normal_rows(comp_rows, seed * 1000 + 3, device),
        kv_dtype=BF16, indices=idx.to(device), topk_lens=topk.to(device),
        seq_lens=torch.full((T,), 4 * comp_rows // T, dtype=torch.int32,
                            device=device),
        cum_seq_lens_q=None, sinks=None, bmm1_scale=sm, bmm2_scale=1.0,
        sm_scale=sm)


def _requests_tables(g, seq_lens, q_len, K, n_neg, topk_lo, topk_hi,
                     share=None):
    """Combined tables for B requests x q_len tokens.

    Token i of request r sits at position seq_len - q_len + i; its SWA
    segment is the 128 positions ending there (paged pool).  Its compressed
    segment holds K-128 distinct rows of the request's region of
    seq_len // 4 rows.  With ``share`` the next token of a request keeps a
    random ``share`` fraction of the previous token's compressed rows and
    draws the rest from rows the previous token did not use.
    """
    B = len(seq_lens)
    T = B * q_len
    ncomp = K - SWA_COLUMNS
    spans = [(s - q_len - SWA_COLUMNS + 1, s) for s in seq_lens]
    row_of, swa_rows = _paged_swa(g, spans)
    comp_base, base = [], 0
    for s in seq_lens:
        comp_base.append(base)
        base += s // COMPRESS_RATIO
    idx = torch.empty((T, K), dtype=torch.int32)
    for r, s in enumerate(seq_lens):
        region = s // COMPRESS_RATIO
        prev = None
        for i in range(q_len):
            t = r * q_len + i
            pos = s - q_len + i
            idx[t, :SWA_COLUMNS] = torch.tensor(
                [row_of(r, p) for p in range(pos - SWA_COLUMNS + 1, pos + 1)],
                dtype=torch.int32)
            if prev is None or share is None:
                local = _distinct(g, region, ncomp)
            else:
                unused = torch.ones(region, dtype=torch.bool)
                unused[prev] = False
                fresh_pool = unused.nonzero().flatten()
                n_new = min(ncomp - int(round(share * ncomp)),
                            int(fresh_pool.numel()))
                keep = prev[torch.randperm(ncomp, generator=g)[:ncomp - n_new]]
                new = fresh_pool[torch.randperm(fresh_pool.numel(),
                                                generator=g)[:n_new]]
                local = torch.cat([keep, new])
                local = local[torch.randperm(ncomp, generator=g)]
            prev = local
            idx[t, SWA_COLUMNS:] = (local + comp_base[r]).int()
            if n_neg:
                idx[t, _distinct(g, K, n_neg)] = -1
    if topk_lo == topk_hi == K:
        topk = torch.full((T,), K, dtype=torch.int32)
    else:
        topk = _uniform_int(g, topk_lo, topk_hi, (T,)).int()
    return idx, topk, swa_rows, base


def _decode_batch(name, seed, device, B, q_len, H, K, seq_lo, seq_hi,
                  q_dtype, kv_dtype, topk_lo, topk_hi, n_neg=0, share=None,
                  sinks=True, q_scale=1.0, kv_scale=1.0, fixed_seq=None,
                  pools=True):
    g = _cpu_gen(seed)
    if fixed_seq is not None:
        seq = [fixed_seq] * B
    else:
        seq = _uniform_int(g, seq_lo, seq_hi, (B,)).tolist()
    idx, topk, swa_rows, comp_rows = _requests_tables(
        g, seq, q_len, K, n_neg, topk_lo, topk_hi, share)
    T = B * q_len
    sink = torch.randn((H,), generator=g, dtype=torch.float32) if sinks else None
    sm = 1.0 / math.sqrt(HEAD_DIM)
    q = normal_rows(T * H, seed * 1000 + 1, device, q_dtype,
                    scale=q_scale).view(T, H, HEAD_DIM)
    if pools:
        swa = pool_rows(swa_rows, seed * 1000 + 2, device, kv_dtype, kv_scale)
        comp = pool_rows(comp_rows, seed * 1000 + 3, device, kv_dtype, kv_scale)
    else:
        swa = comp = None
    qs = q_scale if q_dtype == FP8 else 1.0
    ks = kv_scale if kv_dtype == FP8 else 1.0
    cu = None
    if q_len > 1:
        cu = torch.arange(0, T + 1, q_len, dtype=torch.int32).to(device)
    return Workload(
        name=name, T=T, H=H, K=K, q=q, q_dtype=q_dtype, swa_pool=swa,
        comp_pool=comp, kv_dtype=kv_dtype, indices=idx.to(device),
        topk_lens=topk.to(device),
        seq_lens=torch.tensor(seq, dtype=torch.int32).to(device),
        cum_seq_lens_q=cu,
        sinks=None if sink is None else sink.to(device),
        bmm1_scale=sm * qs * ks, bmm2_scale=ks, q_scale=qs, kv_scale=ks,
        sm_scale=sm, meta={"seq_lens": seq, "swa_rows": swa_rows,
                           "comp_rows": comp_rows})


def make_batched_sinks(device="cpu", seed: int = 2, pools=True) -> Workload:
    """Batched BF16 decode with sinks: T=B=64, H=128, seq_len ~ U{4096..32768},
    table [64,512] = 128 paged SWA rows + 384 distinct compressed rows of the
    request's region, topk_len ~ U{256..512}, sinks N(0,1)."""
    return _decode_batch("batched_sinks", seed, device, B=64, q_len=1, H=128,
                         K=512, seq_lo=4096, seq_hi=32768, q_dtype=BF16,
                         kv_dtype=BF16, topk_lo=256, topk_hi=512, pools=pools)


def make_fp8(device="cpu", seed: int = 3, pools=True) -> Workload:
    """FP8 E4M3 decode: T=B=128, H=64, q quantised with scale 0.05 and both
    pools with 0.08, seq_len ~ U{65536..131072}, table [128,1024] all valid,
    bmm1 = sm_scale*q_scale*kv_scale, bmm2 = kv_scale, sinks N(0,1)."""
    return _decode_batch("fp8", seed, device, B=128, q_len=1, H=64, K=1024,
                         seq_lo=65536, seq_hi=131072, q_dtype=FP8,
                         kv_dtype=FP8, topk_lo=1024, topk_hi=1024,
                         q_scale=0.05, kv_scale=0.08, pools=pools)


def make_long_context(T: int, device="cpu", seed: Optional[int] = None,
                      pools=True) -> Workload:
    """Small-batch long-context decode: T=B tokens, H=128, BF16,
    seq_len=131072 (32768 compressed rows each), table [T,2048] of 128 SWA +
    1920 distinct compressed rows, topk_len=2048, sinks N(0,1).  Large T
    gives the same per-token shape as a full decode batch."""
    return _decode_batch(f"long_context_T{T}",
                         40 + T if seed is None else seed, device, B=T,
                         q_len=1, H=128, K=2048, seq_lo=0, seq_hi=0,
                         q_dtype=BF16, kv_dtype=BF16, topk_lo=2048,
                         topk_hi=2048, fixed_seq=131072, pools=pools)


def make_spec_decode(device="cpu", seed: int = 5, B: int = 256,
                     pools=True) -> Workload:
    """Speculative-token decode: B=256 requests x q_len 2 (varlen,
    cum_seq_lens_q), T=512, H=128, BF16 q, FP8 E4M3 pools (kv_scale 0.08),
    seq_len ~ U{8192..131072}, table [512,2048] of 128 SWA + 1920 compressed
    rows, topk_len ~ U{1024..2048}, exactly 41 slots (2%) per token set to
    -1, and a request's second token keeping ~90% of the first's compressed
    rows.  bmm1 = sm_scale*kv_scale and bmm2 = kv_scale (q stays BF16)."""
    return _decode_batch("spec_decode", seed, device, B=B, q_len=2, H=128,
                         K=2048, seq_lo=8192, seq_hi=131072, q_dtype=BF16,
                         kv_dtype=FP8, topk_lo=1024, topk_hi=2048, n_neg=41,
                         share=0.9, kv_scale=0.08, pools=pools)


def make_packed(T: int = 512, device="cpu", seed: int = 6, H: int = 128,
                pools=True) -> Workload:
    """The long-context decode shape (H heads, topk 2048 = 128 SWA + 1920
    compressed rows, seq_len 131072, sinks) with both pools in the 584-byte
    packed block-scaled FP8 row and BF16 q; bmm1 = sm_scale, bmm2 = 1 (the
    scales are inside the rows)."""
    return _decode_batch(f"packed_T{T}_H{H}", seed, device, B=T, q_len=1, H=H,
                         K=2048, seq_lo=0, seq_hi=0, q_dtype=BF16,
                         kv_dtype=PACKED, topk_lo=2048, topk_hi=2048,
                         fixed_seq=131072, pools=pools)


CONFIGS = {
    "tiny": make_tiny,
    "batched_sinks": make_batched_sinks,
    "fp8": make_fp8,
    "long_context_T1": lambda device="cpu", **kw: make_long_context(1, device, **kw),
    "long_context_T4": lambda device="cpu", **kw: make_long_context(4, device, **kw),
    "long_context_T8": lambda device="cpu", **kw: make_long_context(8, device, **kw),
    "spec_decode": make_spec_decode,
}


def raw_bits(x: torch.Tensor):
    """The stored bit patterns of a bf16 / fp8 tensor as a CPU numpy array
    (uint16 or uint8), for consumers that decode the formats themselves."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float8_e4m3fn:
        return x.view(torch.uint8).numpy()
    if x.dtype == torch.uint8:          # packed rows: already bytes
        return x.numpy()
    raise TypeError(f"unsupported dtype {x.dtype}")
