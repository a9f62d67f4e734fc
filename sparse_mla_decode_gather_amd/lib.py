"""ctypes binding of libsparsemla (``include/sparsemla.h``).

Argument marshalling only: tensors become device pointers, dtypes become the
library's enums, torch's current HIP stream is passed through.  Every step
of the decode runs in the library's HIP kernels; nothing here computes.  If
the shared library is missing this module raises instead of falling back.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

from .build import LIB_PATH, INCLUDE

SMLA_OK = 0
STATUS = {
    0: "SMLA_OK", 1: "SMLA_ERR_INVALID_ARG", 2: "SMLA_ERR_UNSUPPORTED_DTYPE",
    3: "SMLA_ERR_UNSUPPORTED_SHAPE", 4: "SMLA_ERR_WORKSPACE_TOO_SMALL",
    5: "SMLA_ERR_MISALIGNED", 6: "SMLA_ERR_BAD_PLAN", 7: "SMLA_ERR_HIP",
    8: "SMLA_ERR_TOO_LARGE",
}
NOALLOC_SCRATCH_BYTES = 64 << 20
DTYPE_BF16 = 0
DTYPE_FP8_E4M3FN = 1
DTYPE_PACKED_FP8_584 = 2        # uint8 pools of 584-byte packed rows
PACKED_ROW_BYTES = 584
FLAG_VALIDATE_INDICES = 1
FLAG_SERIAL_PIPELINE = 2        # LDS-race check: the serialized tile pipeline
DEVERR = {0: "none", 1: "index out of range", 2: "topk_len out of range"}


class SparseMLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({_status_string(status)})")


class Plan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("head_tiles", ctypes.c_int32),
                ("chunk_cols", ctypes.c_int32),
                ("chunks_per_split", ctypes.c_int32),
                ("num_chunks", ctypes.c_int32), ("K", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]

    def as_dict(self):
        return {"num_splits": self.num_splits, "head_tiles": self.head_tiles,
                "chunk_cols": self.chunk_cols,
                "chunks_per_split": self.chunks_per_split,
                "num_chunks": self.num_chunks, "K": self.K}


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("K", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("q", ctypes.c_void_p),
        ("swa_pool", ctypes.c_void_p), ("swa_rows", ctypes.c_int64),
        ("compressed_pool", ctypes.c_void_p),
        ("compressed_rows", ctypes.c_int64), ("kv_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("pool_row_stride", ctypes.c_int64),
        ("indices", ctypes.c_void_p), ("index_row_stride", ctypes.c_int64),
        ("topk_lens", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("cum_seq_lens_q", ctypes.c_void_p), ("num_requests", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("sinks", ctypes.c_void_p),
        ("bmm1_scale", ctypes.c_float), ("bmm2_scale", ctypes.c_float),
        ("lse_scale", ctypes.c_float), ("reserved1", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("out_lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class Segments(ctypes.Structure):
    """smla_segments: the two-segment form of the token tables."""
    _fields_ = [
        ("swa_indices", ctypes.c_void_p), ("swa_row_stride", ctypes.c_int64),
        ("swa_topk_lens", ctypes.c_void_p),
        ("extra_indices", ctypes.c_void_p), ("extra_row_stride", ctypes.c_int64),
        ("extra_topk_lens", ctypes.c_void_p),
        ("swa_width", ctypes.c_int32), ("extra_width", ctypes.c_int32),
    ]


class Paged(ctypes.Structure):
    """smla_paged: window rows plus a compressed-pool page table."""
    _fields_ = [
        ("swa_indices", ctypes.c_void_p), ("swa_row_stride", ctypes.c_int64),
        ("swa_topk_lens", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
        ("hca_seq_lens", ctypes.c_void_p),
        ("swa_width", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class BuildArgs(ctypes.Structure):
    """smla_build_args: decode metadata -> combined table."""
    _fields_ = [
        ("T", ctypes.c_int32), ("swa_width", ctypes.c_int32),
        ("comp_width", ctypes.c_int32), ("comp_local", ctypes.c_int32),
        ("swa_indices", ctypes.c_void_p), ("swa_row_stride", ctypes.c_int64),
        ("comp_indices", ctypes.c_void_p), ("comp_row_stride", ctypes.c_int64),
        ("comp_topk_lens", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
        ("max_blocks", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_requests", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("token_to_req", ctypes.c_void_p), ("valid_tokens", ctypes.c_void_p),
        ("out_indices", ctypes.c_void_p), ("out_row_stride", ctypes.c_int64),
        ("out_topk_lens", ctypes.c_void_p), ("err", ctypes.c_void_p),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libsparsemla.so from the package directory (no fallback).  The
    environment variable SPARSEMLA_LIB names another build of the same ABI
    instead (the sanitizer build of the host layer that the host tests run
    against)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SPARSEMLA_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing; build it first "
            "(python -m sparse_mla_decode_gather_amd.build)")
    lib = ctypes.CDLL(path)
    lib.sparse_mla_plan_splits.argtypes = [ctypes.c_int] * 8 + [
        ctypes.POINTER(Plan)]
    lib.sparse_mla_plan_splits.restype = ctypes.c_int
    lib.sparse_mla_workspace_size.argtypes = [ctypes.POINTER(Plan), ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int]
    lib.sparse_mla_workspace_size.restype = ctypes.c_size_t
    lib.sparse_mla_workspace_layout.argtypes = [
        ctypes.POINTER(Plan), ctypes.c_int, ctypes.c_int,
        ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_mla_workspace_layout.restype = ctypes.c_int
    lib.sparse_mla_decode.argtypes = [ctypes.POINTER(DecodeArgs),
                                      ctypes.POINTER(Plan), ctypes.c_void_p]
    lib.sparse_mla_decode.restype = ctypes.c_int
    lib.sparse_mla_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs),
                                              ctypes.POINTER(Plan), ctypes.c_void_p]
    lib.sparse_mla_decode_noalloc.restype = ctypes.c_int
    lib.sparse_mla_decode_segments.argtypes = [
        ctypes.POINTER(DecodeArgs), ctypes.POINTER(Segments), ctypes.POINTER(Plan),
        ctypes.c_void_p]
    lib.sparse_mla_decode_segments.restype = ctypes.c_int
    lib.sparse_mla_decode_paged.argtypes = [
        ctypes.POINTER(DecodeArgs), ctypes.POINTER(Paged), ctypes.POINTER(Plan),
        ctypes.c_void_p]
    lib.sparse_mla_decode_paged.restype = ctypes.c_int
    lib.sparse_mla_build_indices.argtypes = [ctypes.POINTER(BuildArgs), ctypes.c_void_p]
    lib.sparse_mla_build_indices.restype = ctypes.c_int
    lib.sparse_mla_gather_only.argtypes = [ctypes.POINTER(DecodeArgs),
                                           ctypes.POINTER(Plan), ctypes.c_void_p]
    lib.sparse_mla_gather_only.restype = ctypes.c_int
    lib.sparse_mla_combine.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.sparse_mla_combine.restype = ctypes.c_int
    lib.sparse_mla_get_device_error.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.sparse_mla_get_device_error.restype = ctypes.c_int
    lib.sparse_mla_status_string.argtypes = [ctypes.c_int]
    lib.sparse_mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions include/sparsemla.h declares."""
    with open(os.path.join(INCLUDE, "sparsemla.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_mla_[a-z_]+)\s*\(", text)))


def _status_string(status: int) -> str:
    try:
        return load().sparse_mla_status_string(status).decode()
    except Exception:          # the library itself may be what is missing
        return "?"


def _check(status: int, where: str):
    if status != SMLA_OK:
        raise SparseMLAError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DTYPE_FP8_E4M3FN
    if t.dtype == torch.uint8 and t.dim() == 2 and t.shape[1] == PACKED_ROW_BYTES:
        return DTYPE_PACKED_FP8_584
    raise TypeError(f"unsupported element type {t.dtype}")


def _require(ok: bool, what: str):
    if not ok:
        raise ValueError(what)


def _check_tensors(q, out, out_lse, pools, tables, vectors, sinks):
    """Layout checks of the arguments the C ABI takes as bare pointers, so
    that a tensor whose memory does not have the layout the library reads
    is refused here instead of being misread (the library cannot see
    strides or dtypes).  q / out / out_lse contiguous [T,H,512] / [T,H];
    pools [rows, 512] views with unit column stride, one dtype and one row
    stride for both; tables int32 with unit column stride; per-token
    vectors int32 and contiguous; sinks float32 and contiguous."""
    _require(q.dim() == 3 and q.shape[2] == 512, "q must be [T, H, 512]")
    _require(q.is_contiguous(), "q must be contiguous")
    T, H = int(q.shape[0]), int(q.shape[1])
    if out is not None:
        _require(out.dtype == torch.bfloat16 and tuple(out.shape) == (T, H, 512)
                 and out.is_contiguous(), "out must be a contiguous BF16 [T, H, 512]")
    if out_lse is not None:
        _require(out_lse.dtype == torch.float32 and tuple(out_lse.shape) == (T, H)
                 and out_lse.is_contiguous(), "out_lse must be a contiguous fp32 [T, H]")
    live = [p for p in pools if p is not None]
    for p in live:
        width = PACKED_ROW_BYTES if p.dtype == torch.uint8 else 512
        _require(p.dim() == 2 and p.shape[1] == width and p.stride(1) == 1,
                 "pools must be [rows, 512] (uint8 packed rows: [rows, 584]) "
                 "with unit column stride")
    if len(live) == 2:
        _require(live[0].dtype == live[1].dtype, "both pools must have one dtype")
        _require(live[0].stride(0) == live[1].stride(0),
                 "both pools must have one row stride")
    for t in tables:
        if t is not None:
            _require(t.dtype == torch.int32 and t.dim() == 2 and t.stride(1) == 1,
                     "index tables must be int32 [rows, width] with unit column stride")
    for v in vectors:
        if v is not None:
            _require(v.dtype == torch.int32 and v.is_contiguous(),
                     "per-token lengths / request vectors must be contiguous int32")
    if sinks is not None:
        _require(sinks.dtype == torch.float32 and sinks.is_contiguous()
                 and sinks.numel() >= H, "sinks must be a contiguous fp32 [H]")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def plan_splits(T: int, H: int, K: int, q_dtype: int = DTYPE_BF16,
                kv_dtype: int = DTYPE_BF16, max_splits: int = 0,
                num_splits: int = 0, num_cus: int = 0) -> Plan:
    plan = Plan()
    _check(load().sparse_mla_plan_splits(T, H, K, q_dtype, kv_dtype, max_splits,
                                         num_splits, num_cus,
                                         ctypes.byref(plan)),
           "sparse_mla_plan_splits")
    return plan


def workspace_size(plan: Plan, T: int, H: int, flags: int = 0) -> int:
    n = load().sparse_mla_workspace_size(ctypes.byref(plan), T, H, flags)
    if n == ctypes.c_size_t(-1).value:
        raise SparseMLAError(1, "sparse_mla_workspace_size")
    return int(n)


def workspace_layout(plan: Plan, T: int, H: int):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().sparse_mla_workspace_layout(ctypes.byref(plan), T, H,
                                              ctypes.byref(a), ctypes.byref(b)),
           "sparse_mla_workspace_layout")
    return int(a.value), int(b.value)


def alloc_workspace(plan: Plan, T: int, H: int, flags: int = 0,
                    device="cuda") -> Optional[torch.Tensor]:
    """A device byte buffer of the size the plan needs (None if zero).
    torch's caching allocator returns 256-B aligned storage."""
    n = workspace_size(plan, T, H, flags)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def make_args(q, swa_pool, compressed_pool, indices, out, *, out_lse=None,
              topk_lens=None, seq_lens=None, cum_seq_lens_q=None, sinks=None,
              bmm1_scale=1.0, bmm2_scale=1.0, lse_scale=1.0, workspace=None,
              flags=0, pool_row_stride=0) -> DecodeArgs:
    _check_tensors(q, out, out_lse, (swa_pool, compressed_pool), (indices,),
                   (topk_lens, seq_lens, cum_seq_lens_q), sinks)
    a = DecodeArgs()
    T, H = int(q.shape[0]), int(q.shape[1])
    a.T, a.H, a.K = T, H, int(indices.shape[1])
    a.q_dtype = dtype_code(q)
    a.q = _ptr(q)
    a.swa_pool = _ptr(swa_pool)
    a.swa_rows = int(swa_pool.shape[0])
    a.compressed_pool = _ptr(compressed_pool)
    a.compressed_rows = 0 if compressed_pool is None else int(
        compressed_pool.shape[0])
    a.kv_dtype = dtype_code(swa_pool)
    a.flags = flags
    a.pool_row_stride = pool_row_stride or int(swa_pool.stride(0))
    a.indices = _ptr(indices)
    a.index_row_stride = int(indices.stride(0))
    a.topk_lens = _ptr(topk_lens)
    a.seq_lens = _ptr(seq_lens)
    a.cum_seq_lens_q = _ptr(cum_seq_lens_q)
    a.num_requests = 0 if seq_lens is None else int(seq_lens.numel())
    a.sinks = _ptr(sinks)
    a.bmm1_scale, a.bmm2_scale, a.lse_scale = bmm1_scale, bmm2_scale, lse_scale
    a.out = _ptr(out)
    a.out_lse = _ptr(out_lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * \
        workspace.element_size()
    return a


def decode(q, swa_pool, compressed_pool, indices, out, *, out_lse=None,
           topk_lens=None, seq_lens=None, cum_seq_lens_q=None, sinks=None,
           bmm1_scale=1.0, bmm2_scale=1.0, lse_scale=1.0, workspace=None,
           plan: Optional[Plan] = None, flags=0, stream=None) -> Plan:
    """sparse_mla_decode: writes ``out`` (and ``out_lse``) in place on the
    current (or given) stream and returns the plan used.  With no workspace
    given, one of the size the plan needs is allocated (device memory only).
    """
    T, H, K = int(q.shape[0]), int(q.shape[1]), int(indices.shape[1])
    if plan is None:
        plan = plan_splits(T, H, K, dtype_code(q), dtype_code(swa_pool))
    if workspace is None:
        workspace = alloc_workspace(plan, T, H, flags, q.device)
    args = make_args(q, swa_pool, compressed_pool, indices, out,
                     out_lse=out_lse, topk_lens=topk_lens, seq_lens=seq_lens,
                     cum_seq_lens_q=cum_seq_lens_q, sinks=sinks,
                     bmm1_scale=bmm1_scale, bmm2_scale=bmm2_scale,
                     lse_scale=lse_scale, workspace=workspace, flags=flags)
    _check(load().sparse_mla_decode(ctypes.byref(args), ctypes.byref(plan),
                                    _stream(stream)), "sparse_mla_decode")
    return plan


def decode_noalloc(q, swa_pool, compressed_pool, indices, out, *, out_lse=None,
                   topk_lens=None, seq_lens=None, cum_seq_lens_q=None, sinks=None,
                   bmm1_scale=1.0, bmm2_scale=1.0, lse_scale=1.0,
                   plan: Optional[Plan] = None, stream=None) -> Plan:
    """sparse_mla_decode_noalloc: sparse_mla_decode with no workspace (the
    split partials live in the library's own static device scratch; nothing
    is allocated here or in the library).  Writes ``out`` (and ``out_lse``)
    in place and returns the plan used."""
    T, H, K = int(q.shape[0]), int(q.shape[1]), int(indices.shape[1])
    if plan is None:
        plan = plan_splits(T, H, K, dtype_code(q), dtype_code(swa_pool))
    args = make_args(q, swa_pool, compressed_pool, indices, out,
                     out_lse=out_lse, topk_lens=topk_lens, seq_lens=seq_lens,
                     cum_seq_lens_q=cum_seq_lens_q, sinks=sinks,
                     bmm1_scale=bmm1_scale, bmm2_scale=bmm2_scale,
                     lse_scale=lse_scale)
    _check(load().sparse_mla_decode_noalloc(ctypes.byref(args), ctypes.byref(plan),
                                            _stream(stream)), "sparse_mla_decode_noalloc")
    return plan


def make_segments(swa_indices, extra_indices, swa_topk_lens=None,
                  extra_topk_lens=None) -> Segments:
    g = Segments()
    g.swa_indices = _ptr(swa_indices)
    g.swa_row_stride = 0 if swa_indices is None else int(swa_indices.stride(0))
    g.swa_topk_lens = _ptr(swa_topk_lens)
    g.extra_indices = _ptr(extra_indices)
    g.extra_row_stride = 0 if extra_indices is None else int(extra_indices.stride(0))
    g.extra_topk_lens = _ptr(extra_topk_lens)
    g.swa_width = 0 if swa_indices is None else int(swa_indices.shape[1])
    g.extra_width = 0 if extra_indices is None else int(extra_indices.shape[1])
    return g


def _args_without_table(q, swa_pool, compressed_pool, K, out, out_lse, topk_lens,
                        seq_lens, cum_seq_lens_q, sinks, bmm1_scale, bmm2_scale,
                        lse_scale, workspace, flags, tables=()) -> DecodeArgs:
    _check_tensors(q, out, out_lse, (swa_pool, compressed_pool), tables,
                   (topk_lens, seq_lens, cum_seq_lens_q), sinks)
    a = DecodeArgs()
    a.T, a.H, a.K = int(q.shape[0]), int(q.shape[1]), K
    a.q_dtype = dtype_code(q)
    a.q = _ptr(q)
    a.swa_pool = _ptr(swa_pool)
    a.swa_rows = 0 if swa_pool is None else int(swa_pool.shape[0])
    a.compressed_pool = _ptr(compressed_pool)
    a.compressed_rows = 0 if compressed_pool is None else int(compressed_pool.shape[0])
    pool = swa_pool if swa_pool is not None else compressed_pool
    a.kv_dtype = dtype_code(pool)
    a.flags = flags
    a.pool_row_stride = int(pool.stride(0))
    a.topk_lens = _ptr(topk_lens)
    a.seq_lens = _ptr(seq_lens)
    a.cum_seq_lens_q = _ptr(cum_seq_lens_q)
    a.num_requests = 0 if seq_lens is None else int(seq_lens.numel())
    a.sinks = _ptr(sinks)
    a.bmm1_scale, a.bmm2_scale, a.lse_scale = bmm1_scale, bmm2_scale, lse_scale
    a.out = _ptr(out)
    a.out_lse = _ptr(out_lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * \
        workspace.element_size()
    return a


def decode_paged(q, swa_pool, compressed_pool, swa_indices, block_tables,
                 page_size: int, out, *, swa_topk_lens=None, topk_lens=None,
                 hca_seq_lens=None, out_lse=None, seq_lens=None,
                 cum_seq_lens_q=None, sinks=None, bmm1_scale=1.0, bmm2_scale=1.0,
                 lse_scale=1.0, workspace=None, plan: Optional[Plan] = None,
                 flags=0, stream=None) -> Plan:
    """sparse_mla_decode_paged: window rows (``swa_indices``, visible
    ``swa_topk_lens``) plus the page expansion of ``block_tables`` (page IDs
    of ``page_size`` compressed rows); ``topk_lens`` counts window +
    compressed slots.  Writes ``out`` (and ``out_lse``) in place and returns
    the plan used, made for K = window width + pages * page_size."""
    g = Paged()
    g.swa_indices = _ptr(swa_indices)
    g.swa_row_stride = 0 if swa_indices is None else int(swa_indices.stride(0))
    g.swa_topk_lens = _ptr(swa_topk_lens)
    g.block_tables = _ptr(block_tables)
    g.block_table_stride = 0 if block_tables is None else int(block_tables.stride(0))
    g.hca_seq_lens = _ptr(hca_seq_lens)
    g.swa_width = 0 if swa_indices is None else int(swa_indices.shape[1])
    g.max_pages = 0 if block_tables is None else int(block_tables.shape[1])
    g.page_size = int(page_size)
    T, H = int(q.shape[0]), int(q.shape[1])
    K = int(g.swa_width) + int(g.max_pages) * int(page_size)
    if plan is None:
        plan = plan_splits(T, H, K, dtype_code(q), dtype_code(
            swa_pool if swa_pool is not None else compressed_pool))
    if workspace is None:
        workspace = alloc_workspace(plan, T, H, flags, q.device)
    _check_tensors(q, None, None, (), (), (swa_topk_lens, hca_seq_lens), None)
    a = _args_without_table(q, swa_pool, compressed_pool, K, out, out_lse, topk_lens,
                            seq_lens, cum_seq_lens_q, sinks, bmm1_scale, bmm2_scale,
                            lse_scale, workspace, flags,
                            tables=(swa_indices, block_tables))
    _check(load().sparse_mla_decode_paged(ctypes.byref(a), ctypes.byref(g),
                                          ctypes.byref(plan), _stream(stream)),
           "sparse_mla_decode_paged")
    return plan


def decode_segments(q, swa_pool, compressed_pool, swa_indices, extra_indices, out,
                    *, swa_topk_lens=None, extra_topk_lens=None, out_lse=None,
                    seq_lens=None, cum_seq_lens_q=None, sinks=None,
                    bmm1_scale=1.0, bmm2_scale=1.0, lse_scale=1.0,
                    workspace=None, plan: Optional[Plan] = None, flags=0,
                    stream=None) -> Plan:
    """sparse_mla_decode_segments: the two-segment form (an SWA table and an
    extra compressed table, each with its own active length; either table
    may be None).  Writes ``out`` (and ``out_lse``) in place and returns the
    plan used, which is made for K = swa width + extra width."""
    g = make_segments(swa_indices, extra_indices, swa_topk_lens, extra_topk_lens)
    T, H = int(q.shape[0]), int(q.shape[1])
    K = int(g.swa_width) + int(g.extra_width)
    if plan is None:
        plan = plan_splits(T, H, K, dtype_code(q), dtype_code(
            swa_pool if swa_pool is not None else compressed_pool))
    if workspace is None:
        workspace = alloc_workspace(plan, T, H, flags, q.device)
    _check_tensors(q, None, None, (), (), (swa_topk_lens, extra_topk_lens), None)
    a = _args_without_table(q, swa_pool, compressed_pool, K, out, out_lse, None,
                            seq_lens, cum_seq_lens_q, sinks, bmm1_scale, bmm2_scale,
                            lse_scale, workspace, flags,
                            tables=(swa_indices, extra_indices))
    _check(load().sparse_mla_decode_segments(ctypes.byref(a), ctypes.byref(g),
                                             ctypes.byref(plan), _stream(stream)),
           "sparse_mla_decode_segments")
    return plan


def build_args(T: int, swa_indices, comp_indices, *, comp_local: bool,
               comp_topk_lens=None, block_tables=None, page_size: int = 0,
               token_to_req=None, valid_tokens=None, out=None, out_topk_lens=None,
               err=None) -> BuildArgs:
    """Fill smla_build_args from int32 tensors (argument marshalling only)."""
    b = BuildArgs()
    b.T = int(T)
    b.swa_width = 0 if swa_indices is None else int(swa_indices.shape[1])
    b.comp_width = 0 if comp_indices is None else int(comp_indices.shape[1])
    b.comp_local = 1 if comp_local else 0
    b.swa_indices = _ptr(swa_indices)
    b.swa_row_stride = 0 if swa_indices is None else int(swa_indices.stride(0))
    b.comp_indices = _ptr(comp_indices)
    b.comp_row_stride = 0 if comp_indices is None else int(comp_indices.stride(0))
    b.comp_topk_lens = _ptr(comp_topk_lens)
    b.block_tables = _ptr(block_tables)
    b.block_table_stride = 0 if block_tables is None else int(block_tables.stride(0))
    b.max_blocks = 0 if block_tables is None else int(block_tables.shape[1])
    b.page_size = int(page_size)
    b.num_requests = 0 if block_tables is None else int(block_tables.shape[0])
    b.token_to_req = _ptr(token_to_req)
    b.valid_tokens = _ptr(valid_tokens)
    b.out_indices = _ptr(out)
    b.out_row_stride = 0 if out is None else int(out.stride(0))
    b.out_topk_lens = _ptr(out_topk_lens)
    b.err = _ptr(err)
    return b


def build_indices(swa_indices, comp_indices, *, comp_local: bool,
                  comp_topk_lens=None, block_tables=None, page_size: int = 0,
                  token_to_req=None, valid_tokens=None, out=None,
                  out_topk_lens=None, err=None, stream=None):
    """sparse_mla_build_indices: the combined table [T, W + K2] and its
    lengths [T] (int32, allocated here unless given) from the token's SWA
    rows and compressed entries (request-local positions through
    ``block_tables`` with ``page_size`` rows per block when ``comp_local``,
    else global rows).  ``err`` (int32[4] on the device, optional) receives
    the first untranslatable entry."""
    ref = swa_indices if swa_indices is not None else comp_indices
    T = int(ref.shape[0])
    K = (0 if swa_indices is None else int(swa_indices.shape[1])) + \
        (0 if comp_indices is None else int(comp_indices.shape[1]))
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=ref.device)
    if out_topk_lens is None:
        out_topk_lens = torch.empty((T,), dtype=torch.int32, device=ref.device)
    b = build_args(T, swa_indices, comp_indices, comp_local=comp_local,
                   comp_topk_lens=comp_topk_lens, block_tables=block_tables,
                   page_size=page_size, token_to_req=token_to_req,
                   valid_tokens=valid_tokens, out=out, out_topk_lens=out_topk_lens,
                   err=err)
    _check(load().sparse_mla_build_indices(ctypes.byref(b), _stream(stream)),
           "sparse_mla_build_indices")
    return out, out_topk_lens


def gather_only(q, swa_pool, compressed_pool, indices, *, topk_lens=None,
                plan: Optional[Plan] = None, stream=None) -> Plan:
    """sparse_mla_gather_only: the compaction and row gather of
    sparse_mla_decode with no arithmetic and no output (measurement aid,
    H = 128 BF16 only).  Returns the plan used."""
    T, H, K = int(q.shape[0]), int(q.shape[1]), int(indices.shape[1])
    if plan is None:
        plan = plan_splits(T, H, K, dtype_code(q), dtype_code(swa_pool))
    args = make_args(q, swa_pool, compressed_pool, indices, None,
                     topk_lens=topk_lens)
    _check(load().sparse_mla_gather_only(ctypes.byref(args), ctypes.byref(plan),
                                         _stream(stream)), "sparse_mla_gather_only")
    return plan


def combine(mid_out, mid_lse, S: int, out, *, out_lse=None, sinks=None,
            lse_scale=1.0, stream=None):
    """sparse_mla_combine over mid_out [T,H,stride,512] / mid_lse
    [T,H,stride] (first S splits)."""
    T, H, stride = (int(x) for x in mid_lse.shape)
    _check(load().sparse_mla_combine(_ptr(mid_out), _ptr(mid_lse), T, H, S,
                                     stride, _ptr(sinks), lse_scale, _ptr(out),
                                     _ptr(out_lse), _stream(stream)),
           "sparse_mla_combine")


def get_device_error(workspace, stream=None):
    """sparse_mla_get_device_error (synchronises): (code, token, column)."""
    c, t, col = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().sparse_mla_get_device_error(_ptr(workspace), _stream(stream),
                                              ctypes.byref(c), ctypes.byref(t),
                                              ctypes.byref(col)),
           "sparse_mla_get_device_error")
    return int(c.value), int(t.value), int(col.value)


def status_string(status: int) -> str:
    return load().sparse_mla_status_string(status).decode()


def decode_workload(w, out=None, out_lse=None, plan=None, flags=0,
                    workspace=None, stream=None):
    """Run sparse_mla_decode on a ``workloads.Workload`` resident on the GPU."""
    if out is None:
        out = torch.empty((w.T, w.H, 512), dtype=torch.bfloat16,
                          device=w.q.device)
    if out_lse is None:
        out_lse = torch.empty((w.T, w.H), dtype=torch.float32,
                              device=w.q.device)
    plan = decode(w.q, w.swa_pool, w.comp_pool, w.indices, out,
                  out_lse=out_lse, topk_lens=w.topk_lens, seq_lens=w.seq_lens,
                  cum_seq_lens_q=w.cum_seq_lens_q, sinks=w.sinks,
                  bmm1_scale=w.bmm1_scale, bmm2_scale=w.bmm2_scale,
                  lse_scale=w.lse_scale, workspace=workspace, plan=plan,
                  flags=flags, stream=stream)
    return out, out_lse, plan
