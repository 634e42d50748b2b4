"""ctypes binding of libpkv.so (include/pkv.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, their data pointers and the current HIP stream are passed to the
C ABI, and a non-zero status becomes a RuntimeError carrying
pkv_last_error().  Every step of the computation runs in the library's HIP
kernels; if the library is missing, importing any entry point fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_lib = None


def _header_constants():
    """Integer #defines of pkv.h (status codes, flags, limits)."""
    consts = {}
    with open(HEADER) as f:
        for line in f:
            m = re.match(r"#define (PKV_\w+)\s+([-0-9u() <]+?)\s*(/\*.*)?$", line)
            if m:
                expr = m.group(2).replace("u", "")
                if not re.fullmatch(r"[-0-9() <]+", expr):
                    continue
                consts[m.group(1)] = int(eval(expr, {"__builtins__": {}}))
    return consts


_C = _header_constants()
PKV_F_ASSUME_CONTIGUOUS = _C["PKV_F_ASSUME_CONTIGUOUS"]
PKV_F_NO_CONTIG_DETECT = _C["PKV_F_NO_CONTIG_DETECT"]
PKV_F_BALANCED = _C["PKV_F_BALANCED"]
PKV_MAX_SPLITS = _C["PKV_MAX_SPLITS"]


def load_library(path: str = LIB_PATH):
    """Load libpkv.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback path")
    L = ctypes.CDLL(path)
    L.paged_kv_append.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P, _P, _I32,
                                  _P, _P, _P]
    L.paged_kv_append.restype = ctypes.c_int
    L.paged_decode_workspace_size.argtypes = [_I32, _I32, _I32, _I32, _I32, ctypes.c_uint32]
    L.paged_decode_workspace_size.restype = ctypes.c_size_t
    L.paged_decode_num_splits.argtypes = [_I32, _I32, _I32]
    L.paged_decode_num_splits.restype = _I32
    L.paged_decode_balanced_parts.argtypes = [_I32, _I32, _I32]
    L.paged_decode_balanced_parts.restype = _I32
    L.paged_decode_attn.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P, _P,
                                    _I32, _I32, ctypes.c_float, _I32, _I32, ctypes.c_uint32, _P,
                                    ctypes.c_size_t, _P, _P, _P]
    L.paged_decode_attn.restype = ctypes.c_int
    L.paged_decode_attn_append.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32,
                                           _I32, _P, _P, _I32, _I32, ctypes.c_float, _I32, _I32,
                                           ctypes.c_uint32, _P, ctypes.c_size_t, _P, _P, _P]
    L.paged_decode_attn_append.restype = ctypes.c_int
    L.packed_prefill_attn.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      ctypes.c_float, _P, _P, _P]
    L.packed_prefill_attn.restype = ctypes.c_int
    L.packed_prefill_attn_append.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                             ctypes.c_float, _P, _P, _P, _P, _I32, _I32, _P,
                                             _I32, _I32, _P, _P]
    L.packed_prefill_attn_append.restype = ctypes.c_int
    L.paged_prefill_attn.argtypes = [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                     ctypes.c_float, _P, _P, _I32, _I32, _P, _I32, _I32, _P, _P,
                                     _P]
    L.paged_prefill_attn.restype = ctypes.c_int
    L.pkv_validate_decode.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _P]
    L.pkv_validate_decode.restype = ctypes.c_int
    L.pkv_validate_prefill.argtypes = [_P, _I32, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P]
    L.pkv_validate_prefill.restype = ctypes.c_int
    L.pkv_last_error.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def last_error() -> str:
    return load_library().pkv_last_error().decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc}): {last_error()}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype, ndim: int) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got {tuple(t.shape)}")
    return t.data_ptr()


def paged_kv_append(k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                    batch_idx: torch.Tensor, input_pos: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor, page_size: int, stream=None) -> None:
    """Scatter k_new/v_new [N, H_kv, D] into the pools [H_kv, num_pages*page_size, D]."""
    L = load_library()
    H_kv, rows, D = k_pool.shape
    if rows % page_size:
        raise ValueError("pool rows must be a multiple of page_size")
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    N = batch_idx.shape[0]
    if tuple(k_new.shape) != (N, H_kv, D) or tuple(v_new.shape) != (N, H_kv, D):
        raise ValueError("k_new/v_new must be [N, H_kv, D]")
    if input_pos.shape[0] != N:
        raise ValueError("input_pos and batch_idx differ in length")
    num_slots, max_blocks = page_table.shape
    rc = L.paged_kv_append(_dev(k_pool, "k_pool", torch.bfloat16, 3),
                           _dev(v_pool, "v_pool", torch.bfloat16, 3), rows // page_size, page_size,
                           H_kv, D, _dev(page_table, "page_table", torch.int32, 2), num_slots,
                           max_blocks, _dev(batch_idx, "batch_idx", torch.int32, 1),
                           _dev(input_pos, "input_pos", torch.int32, 1), N,
                           _dev(k_new, "k_new", torch.bfloat16, 3),
                           _dev(v_new, "v_new", torch.bfloat16, 3), _stream(stream))
    _check(rc, "paged_kv_append")


def paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                num_splits: int = 0, flags: int = 0) -> int:
    return int(load_library().paged_decode_workspace_size(batch, num_q_heads, num_kv_heads,
                                                          head_dim, num_splits, flags))


def paged_decode_num_splits(batch: int, num_kv_heads: int, max_kv_len: int) -> int:
    return int(load_library().paged_decode_num_splits(batch, num_kv_heads, max_kv_len))


def paged_decode_balanced_parts(batch: int, num_kv_heads: int, max_kv_len: int) -> int:
    return int(load_library().paged_decode_balanced_parts(batch, num_kv_heads, max_kv_len))


def paged_decode_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      page_table: torch.Tensor, batch_idx: torch.Tensor, kv_len: torch.Tensor,
                      page_size: int, scale: float, max_kv_len: int = 0, num_splits: int = 0,
                      flags: int = 0, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode attention; returns (out bf16 [B, H_q, D], lse fp32 [B, H_q]).

    num_splits = 0 chooses automatically (per-row splits up to a key bound of
    2048, the balanced schedule above it), 1 is a single pass, >1 per-row
    splits; flags |= PKV_F_BALANCED (with num_splits = 0) forces the balanced
    schedule.  The workspace (uint8 tensor) is allocated
    here when not given and the schedule needs one.
    """
    L = load_library()
    B, H_q, D = q.shape
    H_kv, rows, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape or rows % page_size:
        raise ValueError("pool shape does not match q / page_size")
    num_slots, max_blocks = page_table.shape
    if batch_idx.shape[0] != B or kv_len.shape[0] != B:
        raise ValueError("batch_idx and kv_len must have one entry per row")
    S = int(num_splits)
    need = paged_decode_workspace_size(B, H_q, H_kv, D, S, int(flags))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = L.paged_decode_attn(_dev(q, "q", torch.bfloat16, 3), _dev(k_pool, "k_pool", torch.bfloat16, 3),
                             _dev(v_pool, "v_pool", torch.bfloat16, 3), rows // page_size,
                             page_size, H_kv, D, _dev(page_table, "page_table", torch.int32, 2),
                             num_slots, max_blocks, _dev(batch_idx, "batch_idx", torch.int32, 1),
                             _dev(kv_len, "kv_len", torch.int32, 1), B, H_q, float(scale),
                             int(max_kv_len), S, int(flags), ws_ptr, ws_bytes,
                             _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2),
                             _stream(stream))
    _check(rc, "paged_decode_attn")
    return out, lse


def paged_decode_attn_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                             k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                             batch_idx: torch.Tensor, kv_len: torch.Tensor, page_size: int,
                             scale: float, max_kv_len: int = 0, num_splits: int = 0, flags: int = 0,
                             workspace: Optional[torch.Tensor] = None,
                             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Append each row's new token (k_new/v_new [B, H_kv, D], position kv_len-1) and decode,
    in one launch; returns (out, lse) as paged_decode_attn."""
    L = load_library()
    B, H_q, D = q.shape
    H_kv, rows, D2 = k_pool.shape
    if D2 != D or v_pool.shape != k_pool.shape or rows % page_size:
        raise ValueError("pool shape does not match q / page_size")
    if tuple(k_new.shape) != (B, H_kv, D) or tuple(v_new.shape) != (B, H_kv, D):
        raise ValueError("k_new/v_new must be [B, H_kv, D]")
    num_slots, max_blocks = page_table.shape
    if batch_idx.shape[0] != B or kv_len.shape[0] != B:
        raise ValueError("batch_idx and kv_len must have one entry per row")
    S = int(num_splits)
    need = paged_decode_workspace_size(B, H_q, H_kv, D, S, int(flags))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel())
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = L.paged_decode_attn_append(
        _dev(q, "q", torch.bfloat16, 3), _dev(k_new, "k_new", torch.bfloat16, 3),
        _dev(v_new, "v_new", torch.bfloat16, 3), _dev(k_pool, "k_pool", torch.bfloat16, 3),
        _dev(v_pool, "v_pool", torch.bfloat16, 3), rows // page_size, page_size, H_kv, D,
        _dev(page_table, "page_table", torch.int32, 2), num_slots, max_blocks,
        _dev(batch_idx, "batch_idx", torch.int32, 1), _dev(kv_len, "kv_len", torch.int32, 1), B,
        H_q, float(scale), int(max_kv_len), S, int(flags), ws_ptr, ws_bytes,
        _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2), _stream(stream))
    _check(rc, "paged_decode_attn_append")
    return out, lse


def packed_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, scale: float,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Document-causal prefill; returns (out bf16 [L, H_q, D], lse fp32 [L, H_q])."""
    L = load_library()
    Lt, H_q, D = q.shape
    _, H_kv, _ = k.shape
    if tuple(k.shape) != (Lt, H_kv, D) or tuple(v.shape) != (Lt, H_kv, D):
        raise ValueError("k/v must be [L, H_kv, D] matching q")
    n_docs = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((Lt, H_q, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Lt, H_q), dtype=torch.float32, device=q.device)
    rc = L.packed_prefill_attn(_dev(q, "q", torch.bfloat16, 3), _dev(k, "k", torch.bfloat16, 3),
                               _dev(v, "v", torch.bfloat16, 3),
                               _dev(cu_seqlens, "cu_seqlens", torch.int32, 1), n_docs, Lt, H_q,
                               H_kv, D, float(scale), _dev(out, "out", torch.bfloat16, 3),
                               _dev(lse, "lse", torch.float32, 2), _stream(stream))
    _check(rc, "packed_prefill_attn")
    return out, lse


def packed_prefill_attn_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               cu_seqlens: torch.Tensor, scale: float, k_pool: torch.Tensor,
                               v_pool: torch.Tensor, page_table: torch.Tensor,
                               doc_slots: torch.Tensor, page_size: int,
                               out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None,
                               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Document-causal prefill plus the scatter of each document's K/V (slot doc_slots[d],
    positions 0..n_d-1) into the pools, in one launch; returns (out, lse)."""
    L = load_library()
    Lt, H_q, D = q.shape
    _, H_kv, _ = k.shape
    if tuple(k.shape) != (Lt, H_kv, D) or tuple(v.shape) != (Lt, H_kv, D):
        raise ValueError("k/v must be [L, H_kv, D] matching q")
    Hp, rows, Dp = k_pool.shape
    if Hp != H_kv or Dp != D or v_pool.shape != k_pool.shape or rows % page_size:
        raise ValueError("pool shape does not match k / page_size")
    n_docs = cu_seqlens.shape[0] - 1
    if doc_slots.shape[0] != n_docs:
        raise ValueError("doc_slots must have one entry per document")
    num_slots, max_blocks = page_table.shape
    if out is None:
        out = torch.empty((Lt, H_q, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Lt, H_q), dtype=torch.float32, device=q.device)
    rc = L.packed_prefill_attn_append(
        _dev(q, "q", torch.bfloat16, 3), _dev(k, "k", torch.bfloat16, 3),
        _dev(v, "v", torch.bfloat16, 3), _dev(cu_seqlens, "cu_seqlens", torch.int32, 1), n_docs,
        Lt, H_q, H_kv, D, float(scale), _dev(out, "out", torch.bfloat16, 3),
        _dev(lse, "lse", torch.float32, 2), _dev(k_pool, "k_pool", torch.bfloat16, 3),
        _dev(v_pool, "v_pool", torch.bfloat16, 3), rows // page_size, page_size,
        _dev(page_table, "page_table", torch.int32, 2), num_slots, max_blocks,
        _dev(doc_slots, "doc_slots", torch.int32, 1), _stream(stream))
    _check(rc, "packed_prefill_attn_append")
    return out, lse


def paged_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                       prefix_lens: torch.Tensor, doc_slots: torch.Tensor, scale: float,
                       k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                       page_size: int, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked prefill: chunk rows attend to their sequence's cached prefix (pages) and to
    the chunk causally; the chunk's K/V are written into the pages.  Returns (out, lse)."""
    L = load_library()
    Lt, H_q, D = q.shape
    _, H_kv, _ = k.shape
    if tuple(k.shape) != (Lt, H_kv, D) or tuple(v.shape) != (Lt, H_kv, D):
        raise ValueError("k/v must be [L, H_kv, D] matching q")
    Hp, rows, Dp = k_pool.shape
    if Hp != H_kv or Dp != D or v_pool.shape != k_pool.shape or rows % page_size:
        raise ValueError("pool shape does not match k / page_size")
    n_docs = cu_seqlens.shape[0] - 1
    if doc_slots.shape[0] != n_docs or prefix_lens.shape[0] != n_docs:
        raise ValueError("doc_slots and prefix_lens must have one entry per document")
    num_slots, max_blocks = page_table.shape
    if out is None:
        out = torch.empty((Lt, H_q, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Lt, H_q), dtype=torch.float32, device=q.device)
    rc = L.paged_prefill_attn(
        _dev(q, "q", torch.bfloat16, 3), _dev(k, "k", torch.bfloat16, 3),
        _dev(v, "v", torch.bfloat16, 3), _dev(cu_seqlens, "cu_seqlens", torch.int32, 1),
        _dev(prefix_lens, "prefix_lens", torch.int32, 1),
        _dev(doc_slots, "doc_slots", torch.int32, 1), n_docs, Lt, H_q, H_kv, D, float(scale),
        _dev(k_pool, "k_pool", torch.bfloat16, 3), _dev(v_pool, "v_pool", torch.bfloat16, 3),
        rows // page_size, page_size, _dev(page_table, "page_table", torch.int32, 2), num_slots,
        max_blocks, _dev(out, "out", torch.bfloat16, 3), _dev(lse, "lse", torch.float32, 2),
        _stream(stream))
    _check(rc, "paged_prefill_attn")
    return out, lse


def validate_decode(page_table: torch.Tensor, batch_idx: torch.Tensor, kv_len: torch.Tensor,
                    page_size: int, num_pages: int, report: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Debug check of decode's device-side inputs.  Returns the int32 report [4] on the GPU:
    (violating rows, first violating row or -1, its PKV_V_* code, block or -1)."""
    L = load_library()
    B = batch_idx.shape[0]
    if kv_len.shape[0] != B:
        raise ValueError("kv_len and batch_idx differ in length")
    num_slots, max_blocks = page_table.shape
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=batch_idx.device)
    rc = L.pkv_validate_decode(_dev(page_table, "page_table", torch.int32, 2), num_pages, page_size,
                               num_slots, max_blocks, _dev(batch_idx, "batch_idx", torch.int32, 1),
                               _dev(kv_len, "kv_len", torch.int32, 1), B,
                               _dev(report, "report", torch.int32, 1), _stream(stream))
    _check(rc, "pkv_validate_decode")
    return report


def validate_prefill(cu_seqlens: torch.Tensor, total_len: int,
                     doc_slots: Optional[torch.Tensor] = None,
                     prefix_lens: Optional[torch.Tensor] = None,
                     page_table: Optional[torch.Tensor] = None, page_size: int = 16,
                     num_pages: int = 1, report: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Debug check of the prefill calls' device-side inputs.  Returns the int32 report [4]
    on the GPU: (violating documents, first violating document or -1, its PKV_V_* code,
    block or -1)."""
    L = load_library()
    n_docs = cu_seqlens.shape[0] - 1
    num_slots, max_blocks = page_table.shape if page_table is not None else (1, 1)
    for t, name in ((doc_slots, "doc_slots"), (prefix_lens, "prefix_lens")):
        if t is not None and t.shape[0] != n_docs:
            raise ValueError(f"{name} must have one entry per document")
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=cu_seqlens.device)
    opt = lambda t, name, nd: _dev(t, name, torch.int32, nd) if t is not None else None  # noqa: E731
    rc = L.pkv_validate_prefill(_dev(cu_seqlens, "cu_seqlens", torch.int32, 1), n_docs, total_len,
                                opt(doc_slots, "doc_slots", 1), opt(prefix_lens, "prefix_lens", 1),
                                opt(page_table, "page_table", 2), num_pages, page_size, num_slots,
                                max_blocks, _dev(report, "report", torch.int32, 1), _stream(stream))
    _check(rc, "pkv_validate_prefill")
    return report
