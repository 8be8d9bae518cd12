"""ctypes binding of libidx.so (include/idx.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the indexer path runs inside the library's
kernels.  The library must have been built (``python -m
sparse_attention_indexer_decode_amd._build`` or ``__graft_entry__.build()``);
nothing here falls back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_size_t, c_uint32, c_void_p

import torch

from ._build import LIB_PATH

IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_ENOSPC, IDX_EHIP = 0, 1, 2, 3, 4
IDX_FMT_FP8_E4M3, IDX_FMT_MXFP4 = 0, 1
IDX_ROWS_DECODE, IDX_ROWS_PREFILL = 0, 1
IDX_OP_LOGITS, IDX_OP_TOPK, IDX_OP_DECODE_TOPK, IDX_OP_CACHE_WRITE = 0, 1, 2, 3
IDX_OP_POOL_TOPK, IDX_OP_DECODE_POOL_TOPK = 4, 5
IDX_DEV_BAD_PAGE, IDX_DEV_BAD_SLOT = 1, 2

FMT_CODES = {"fp8": IDX_FMT_FP8_E4M3, "mxfp4": IDX_FMT_MXFP4}

EXPORTED = (
    "idx_num_rows",
    "idx_workspace_bytes",
    "idx_logits_paged",
    "idx_topk",
    "idx_decode_topk",
    "idx_decode_topk_noalloc",
    "idx_pool_topk",
    "idx_decode_pool_topk",
    "idx_cache_write",
    "idx_prefill_chunks",
    "idx_read_device_status",
    "idx_status_string",
    "idx_last_error",
    "idx_version",
)


class IdxCache(ctypes.Structure):
    _fields_ = [("base", c_void_p), ("num_pages", c_int64), ("page_bytes", c_int64),
                ("page_size", c_int32), ("head_dim", c_int32), ("fmt", c_int32),
                ("reserved", c_int32)]


class IdxRows(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("num_req", c_int32), ("block_table", c_void_p),
                ("bt_stride", c_int64), ("bt_width", c_int32), ("max_seq_len", c_int32),
                ("seq_lens", c_void_p), ("decode_lens", c_void_p), ("next_n", c_int32),
                ("q_packed", c_int32), ("query_start_loc", c_void_p), ("q_begin", c_int32),
                ("q_end", c_int32), ("compress_ratio", c_int32)]


class IdxChunk(ctypes.Structure):
    _fields_ = [("req_begin", c_int32), ("req_end", c_int32), ("q_begin", c_int32),
                ("q_end", c_int32), ("total_seq_lens", c_int64), ("token_begin", c_int64),
                ("token_end", c_int64), ("skip_kv_gather", c_int32), ("over_budget", c_int32)]


class IdxPools(ctypes.Structure):
    _fields_ = [("pool_size", c_int32), ("topk_pools", c_int32), ("init_pools", c_int32),
                ("local_pools", c_int32)]


class IdxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    # IDX_LIB_PATH selects another build of the same library (the host
    # sanitizer build of the CPU tests)
    p = path or os.environ.get("IDX_LIB_PATH") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libidx.so not built at {p}; run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    lib.idx_num_rows.argtypes = [POINTER(IdxRows)]
    lib.idx_num_rows.restype = c_int64
    lib.idx_workspace_bytes.argtypes = [c_int32, POINTER(IdxCache), POINTER(IdxRows), c_int32, c_int32]
    lib.idx_workspace_bytes.restype = c_size_t
    lib.idx_logits_paged.argtypes = [POINTER(IdxCache), POINTER(IdxRows), c_void_p, c_void_p, c_int32,
                                     c_void_p, c_int64, c_void_p, c_size_t, c_void_p]
    lib.idx_logits_paged.restype = c_int32
    lib.idx_topk.argtypes = [c_void_p, c_int64, POINTER(IdxRows), c_int32, c_void_p, c_void_p,
                             c_size_t, c_void_p]
    lib.idx_topk.restype = c_int32
    lib.idx_decode_topk.argtypes = [POINTER(IdxCache), POINTER(IdxRows), c_void_p, c_void_p, c_int32,
                                    c_int32, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.idx_decode_topk.restype = c_int32
    lib.idx_decode_topk_noalloc.argtypes = [POINTER(IdxCache), POINTER(IdxRows), c_void_p, c_void_p, c_int32,
                                            c_int32, c_void_p, c_void_p, c_void_p]
    lib.idx_decode_topk_noalloc.restype = c_int32
    lib.idx_pool_topk.argtypes = [c_void_p, c_int64, POINTER(IdxRows), POINTER(IdxPools), c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]
    lib.idx_pool_topk.restype = c_int32
    lib.idx_decode_pool_topk.argtypes = [POINTER(IdxCache), POINTER(IdxRows), c_void_p, c_void_p, c_int32,
                                         POINTER(IdxPools), c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.idx_decode_pool_topk.restype = c_int32
    lib.idx_cache_write.argtypes = [POINTER(IdxCache), c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_size_t,
                                    c_void_p]
    lib.idx_cache_write.restype = c_int32
    lib.idx_prefill_chunks.argtypes = [POINTER(c_int32), POINTER(c_int32), c_int32, c_int64, c_int64,
                                       c_int32, POINTER(IdxChunk), c_int32, POINTER(c_int32)]
    lib.idx_prefill_chunks.restype = c_int32
    lib.idx_read_device_status.argtypes = [c_void_p, POINTER(c_uint32), c_void_p]
    lib.idx_read_device_status.restype = c_int32
    lib.idx_status_string.argtypes = [c_int32]
    lib.idx_status_string.restype = c_char_p
    lib.idx_last_error.argtypes = []
    lib.idx_last_error.restype = c_char_p
    lib.idx_version.argtypes = []
    lib.idx_version.restype = c_char_p
    if path is None:
        _LIB = lib
    return lib


def _check(fn: str, st: int):
    if st != IDX_OK:
        lib = load()
        raise IdxError(fn, st, f"{lib.idx_status_string(st).decode()}: {lib.idx_last_error().decode()}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _row_stride(t: torch.Tensor) -> int:
    """Element stride between rows of a 2-D table (a single row's stride is
    irrelevant, so its width is reported)."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ---------------------------------------------------------------------------
# Descriptors (hold the tensors alive while their pointers are in use)
# ---------------------------------------------------------------------------

class Cache:
    """Paged index cache: a uint8 device tensor [num_pages, page_bytes]."""

    def __init__(self, pages: torch.Tensor, head_dim: int, fmt: str = "fp8", page_size: int = 64):
        assert pages.dtype == torch.uint8 and pages.dim() == 2 and pages.is_contiguous()
        self.pages = pages
        self.c = IdxCache(pages.data_ptr(), pages.shape[0], pages.shape[1], page_size, head_dim,
                          FMT_CODES[fmt], 0)


class Rows:
    """Query rows (DECODE grid or PREFILL chunk slice); see idx_rows in idx.h."""

    def __init__(self, c: IdxRows, keep: tuple):
        self.c = c
        self._keep = keep

    @property
    def num_rows(self) -> int:
        return int(load().idx_num_rows(ctypes.byref(self.c)))

    @staticmethod
    def decode(block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, next_n: int = 1,
               decode_lens: torch.Tensor | None = None, q_packed: bool = False,
               compress_ratio: int = 1) -> "Rows":
        for t in (block_table, seq_lens, decode_lens):
            assert t is None or t.dtype == torch.int32
        c = IdxRows(IDX_ROWS_DECODE, seq_lens.shape[0], _ptr(block_table), _row_stride(block_table),
                    block_table.shape[1], int(max_seq_len), _ptr(seq_lens), _ptr(decode_lens), next_n,
                    int(q_packed), None, 0, 0, int(compress_ratio))
        return Rows(c, (block_table, seq_lens, decode_lens))

    @staticmethod
    def prefill(block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                q_begin: int, q_end: int, max_seq_len: int, compress_ratio: int = 1) -> "Rows":
        for t in (block_table, seq_lens, query_start_loc):
            assert t.dtype == torch.int32
        c = IdxRows(IDX_ROWS_PREFILL, seq_lens.shape[0], _ptr(block_table), _row_stride(block_table),
                    block_table.shape[1], int(max_seq_len), _ptr(seq_lens), None, 1, 0,
                    _ptr(query_start_loc), int(q_begin), int(q_end), int(compress_ratio))
        return Rows(c, (block_table, seq_lens, query_start_loc))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def idx_workspace_bytes(op: int, cache: Cache | None, rows: Rows | None, heads: int, k: int) -> int:
    return int(load().idx_workspace_bytes(op, ctypes.byref(cache.c) if cache else None,
                                          ctypes.byref(rows.c) if rows else None, heads, k))


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled, 256-byte aligned device workspace of at least nbytes."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def idx_logits_paged(cache: Cache, rows: Rows, q: torch.Tensor, w: torch.Tensor, logits: torch.Tensor,
                     workspace: torch.Tensor, stream=None) -> None:
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
    assert logits.dtype == torch.float32 and logits.stride(-1) == 1
    heads = q.shape[1]
    _check("idx_logits_paged", load().idx_logits_paged(
        ctypes.byref(cache.c), ctypes.byref(rows.c), q.data_ptr(), w.data_ptr(), heads,
        logits.data_ptr(), _row_stride(logits), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def idx_topk(logits: torch.Tensor, rows: Rows, k: int, out: torch.Tensor, workspace: torch.Tensor,
             stream=None) -> None:
    assert logits.dtype == torch.float32 and logits.stride(-1) == 1
    assert out.dtype == torch.int32 and out.is_contiguous()
    _check("idx_topk", load().idx_topk(logits.data_ptr(), _row_stride(logits), ctypes.byref(rows.c), k,
                                       out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                       _stream(stream)))


def idx_decode_topk(cache: Cache, rows: Rows, q: torch.Tensor, w: torch.Tensor, k: int, out: torch.Tensor,
                    workspace: torch.Tensor, stream=None) -> None:
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
    assert out.dtype == torch.int32 and out.is_contiguous()
    _check("idx_decode_topk", load().idx_decode_topk(
        ctypes.byref(cache.c), ctypes.byref(rows.c), q.data_ptr(), w.data_ptr(), q.shape[1], k,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def idx_decode_topk_noalloc(cache: Cache, rows: Rows, q: torch.Tensor, w: torch.Tensor, k: int,
                            out: torch.Tensor, status: torch.Tensor | None = None, stream=None) -> None:
    """idx_decode_topk without a workspace (the library's static scratch);
    status: optional int32/uint32 device tensor of one element."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
    assert out.dtype == torch.int32 and out.is_contiguous()
    assert status is None or (status.numel() >= 1 and status.element_size() == 4)
    _check("idx_decode_topk_noalloc", load().idx_decode_topk_noalloc(
        ctypes.byref(cache.c), ctypes.byref(rows.c), q.data_ptr(), w.data_ptr(), q.shape[1], k,
        out.data_ptr(), _ptr(status), _stream(stream)))


def pools(pool_size: int, topk_pools: int, init_pools: int = 0, local_pools: int = 0) -> IdxPools:
    """Pool-selection parameters (idx_pools)."""
    return IdxPools(pool_size, topk_pools, init_pools, local_pools)


def idx_pool_topk(logits: torch.Tensor, rows: Rows, pl: IdxPools, out_tokens: torch.Tensor,
                  out_pools: torch.Tensor | None, workspace: torch.Tensor, stream=None) -> None:
    """out_tokens: int32 [rows, (topk_pools + 1) * pool_size]; out_pools:
    int32 [rows, topk_pools] or None."""
    assert logits.dtype == torch.float32 and logits.stride(-1) == 1
    assert out_tokens.dtype == torch.int32 and out_tokens.is_contiguous()
    assert out_pools is None or (out_pools.dtype == torch.int32 and out_pools.is_contiguous())
    _check("idx_pool_topk", load().idx_pool_topk(
        logits.data_ptr(), _row_stride(logits), ctypes.byref(rows.c), ctypes.byref(pl), out_tokens.data_ptr(),
        _ptr(out_pools), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def idx_decode_pool_topk(cache: Cache, rows: Rows, q: torch.Tensor, w: torch.Tensor, pl: IdxPools,
                         out_tokens: torch.Tensor, out_pools: torch.Tensor | None, workspace: torch.Tensor,
                         stream=None) -> None:
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
    assert out_tokens.dtype == torch.int32 and out_tokens.is_contiguous()
    assert out_pools is None or (out_pools.dtype == torch.int32 and out_pools.is_contiguous())
    _check("idx_decode_pool_topk", load().idx_decode_pool_topk(
        ctypes.byref(cache.c), ctypes.byref(rows.c), q.data_ptr(), w.data_ptr(), q.shape[1], ctypes.byref(pl),
        out_tokens.data_ptr(), _ptr(out_pools), workspace.data_ptr(), workspace.numel(), _stream(stream)))


def idx_cache_write(cache: Cache, k: torch.Tensor, slot_mapping: torch.Tensor, workspace: torch.Tensor,
                    stream=None) -> None:
    """k: bf16 [num_tokens, >= head_dim] (unit element stride); slot_mapping:
    int64 [num_tokens]."""
    assert k.dtype == torch.bfloat16 and k.dim() == 2 and k.stride(1) == 1
    assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
    assert slot_mapping.shape[0] == k.shape[0]
    _check("idx_cache_write", load().idx_cache_write(
        ctypes.byref(cache.c), k.data_ptr(), _row_stride(k), slot_mapping.data_ptr(), k.shape[0],
        workspace.data_ptr(), workspace.numel(), _stream(stream)))


def idx_prefill_chunks(seq_lens, query_lens, workspace_tokens: int, max_logits_bytes: int,
                       request_offset: int = 0) -> list[dict]:
    seq = [int(x) for x in seq_lens]
    ql = [int(x) for x in query_lens]
    n = len(seq)
    lib = load()
    SeqArr = c_int32 * max(n, 1)
    sa, qa = SeqArr(*seq), SeqArr(*ql)
    cap = 16
    while True:
        out = (IdxChunk * cap)()
        n_out = c_int32(0)
        st = lib.idx_prefill_chunks(sa, qa, n, workspace_tokens, max_logits_bytes, request_offset,
                                    out, cap, ctypes.byref(n_out))
        if st == IDX_ENOSPC:
            cap = n_out.value
            continue
        _check("idx_prefill_chunks", st)
        return [{f: getattr(out[i], f) for f, _ in IdxChunk._fields_} for i in range(n_out.value)]


def idx_read_device_status(workspace: torch.Tensor, stream=None) -> int:
    flags = c_uint32(0)
    _check("idx_read_device_status", load().idx_read_device_status(workspace.data_ptr(), ctypes.byref(flags),
                                                                   _stream(stream)))
    return int(flags.value)


def idx_version() -> str:
    return load().idx_version().decode()
