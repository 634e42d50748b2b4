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
    L.paged_decode_auto_balanced.argtypes = [_I32, _I32, _I32]
    L.paged_decode_auto_balanced.restype = _I32
    L.paged_decode_attn.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P, _P,
                                    _I32, _I32, ctypes.c_float, _I32, _I32, ctypes.c_uint32, _P,
                                    ctypes.c_size_t, _P, _P, _P]
    L.paged_decode_attn.restype = ctypes.c_int
    L.paged_decode_attn_noalloc.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32,
                                            _P, _P, _I32, _I32, ctypes.c_float, _I32, _I32,
                                            ctypes.c_uint32, _P, _P, _P]
    L.paged_decode_attn_noalloc.restype = ctypes.c_int
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


def _dev(t: torch.Tensor, name: str, dtype, ndim: int, shape=None, device=None) -> int:
    """Data pointer of a contiguous GPU tensor, after checking dtype, rank, and (when
    given) the exact shape and the device.  The C ABI sees pointers only, so every
    buffer a kernel writes is checked here against the size the kernel will use."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _workspace(workspace: Optional[torch.Tensor], device) -> Tuple[int, int]:
    """(pointer, bytes) of an optional uint8 workspace on the call's device."""
    if workspace is None:
        return 0, 0
    ptr = _dev(workspace, "workspace", torch.uint8, 1, device=device)
    return ptr, workspace.numel()


def paged_kv_append(k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                    batch_idx: torch.Tensor, input_pos: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor, page_size: int, stream=None) -> None:
    """Scatter k_new/v_new [N, H_kv, D] into the pools [H_kv, num_pages*page_size, D]."""
    L = load_library()
    H_kv, rows, D = k_pool.shape
    if rows % page_size:
        raise ValueError("pool rows must be a multiple of page_size")
    N = batch_idx.shape[0]
    dv = k_pool.device
    num_slots, max_blocks = page_table.shape
    rc = L.paged_kv_append(_dev(k_pool, "k_pool", torch.bfloat16, 3),
                           _dev(v_pool, "v_pool", torch.bfloat16, 3, k_pool.shape, dv),
                           rows // page_size, page_size, H_kv, D,
                           _dev(page_table, "page_table", torch.int32, 2, device=dv), num_slots,
                           max_blocks, _dev(batch_idx, "batch_idx", torch.int32, 1, device=dv),
                           _dev(input_pos, "input_pos", torch.int32, 1, (N,), dv), N,
                           _dev(k_new, "k_new", torch.bfloat16, 3, (N, H_kv, D), dv),
                           _dev(v_new, "v_new", torch.bfloat16, 3, (N, H_kv, D), dv),
                           _stream(stream))
    _check(rc, "paged_kv_append")


def paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                num_splits: int = 0, flags: int = 0) -> int:
    return int(load_library().paged_decode_workspace_size(batch, num_q_heads, num_kv_heads,
                                                          head_dim, num_splits, flags))


def paged_decode_num_splits(batch: int, num_kv_heads: int, max_kv_len: int) -> int:
    return int(load_library().paged_decode_num_splits(batch, num_kv_heads, max_kv_len))


def paged_decode_balanced_parts(batch: int, num_kv_heads: int, max_kv_len: int) -> int:
    return int(load_library().paged_decode_balanced_parts(batch, num_kv_heads, max_kv_len))


def paged_decode_auto_balanced(batch: int, num_kv_heads: int, max_kv_len: int) -> bool:
    return bool(load_library().paged_decode_auto_balanced(batch, num_kv_heads, max_kv_len))


def _decode_args(q, k_pool, v_pool, page_table, batch_idx, kv_len, page_size, num_splits, flags,
                 workspace, out, lse, alloc_workspace=True):
    """Shapes, pointers and output buffers shared by the decode wrappers."""
    B, H_q, D = q.shape
    H_kv, rows, D2 = k_pool.shape
    if D2 != D or rows % page_size:
        raise ValueError("pool shape does not match q / page_size")
    dv = q.device
    num_slots, max_blocks = page_table.shape
    need = paged_decode_workspace_size(B, H_q, H_kv, D, int(num_splits), int(flags))
    if need and workspace is None and alloc_workspace:
        workspace = torch.empty(need, dtype=torch.uint8, device=dv)
    ws_ptr, ws_bytes = _workspace(workspace, dv)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=dv)
    if lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=dv)
    ptrs = dict(
        q=_dev(q, "q", torch.bfloat16, 3),
        k_pool=_dev(k_pool, "k_pool", torch.bfloat16, 3, device=dv),
        v_pool=_dev(v_pool, "v_pool", torch.bfloat16, 3, k_pool.shape, dv),
        page_table=_dev(page_table, "page_table", torch.int32, 2, device=dv),
        batch_idx=_dev(batch_idx, "batch_idx", torch.int32, 1, (B,), dv),
        kv_len=_dev(kv_len, "kv_len", torch.int32, 1, (B,), dv),
        out=_dev(out, "out", torch.bfloat16, 3, (B, H_q, D), dv),
        lse=_dev(lse, "lse", torch.float32, 2, (B, H_q), dv))
    geo = dict(B=B, H_q=H_q, H_kv=H_kv, D=D, num_pages=rows // page_size, num_slots=num_slots,
               max_blocks=max_blocks)
    return ptrs, geo, ws_ptr, ws_bytes, out, lse


def paged_decode_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      page_table: torch.Tensor, batch_idx: torch.Tensor, kv_len: torch.Tensor,
                      page_size: int, scale: float, max_kv_len: int = 0, num_splits: int = 0,
                      flags: int = 0, workspace: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode attention; returns (out bf16 [B, H_q, D], lse fp32 [B, H_q]).

    num_splits = 0 chooses automatically (the balanced schedule for a key
    bound above 2048 or at least 4 (row, KV head) units per compute unit,
    per-row splits otherwise: paged_decode_auto_balanced), 1 is a single
    pass, >1 per-row splits; flags |= PKV_F_BALANCED (with num_splits = 0) forces the balanced
    schedule.  The workspace (uint8 tensor) is allocated
    here when not given and the schedule needs one.
    """
    L = load_library()
    p, g, ws_ptr, ws_bytes, out, lse = _decode_args(q, k_pool, v_pool, page_table, batch_idx,
                                                    kv_len, page_size, num_splits, flags,
                                                    workspace, out, lse)
    rc = L.paged_decode_attn(p["q"], p["k_pool"], p["v_pool"], g["num_pages"], page_size,
                             g["H_kv"], g["D"], p["page_table"], g["num_slots"], g["max_blocks"],
                             p["batch_idx"], p["kv_len"], g["B"], g["H_q"], float(scale),
                             int(max_kv_len), int(num_splits), int(flags), ws_ptr, ws_bytes,
                             p["out"], p["lse"], _stream(stream))
    _check(rc, "paged_decode_attn")
    return out, lse


def paged_decode_attn_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                              page_table: torch.Tensor, batch_idx: torch.Tensor,
                              kv_len: torch.Tensor, page_size: int, scale: float,
                              out: torch.Tensor, lse: torch.Tensor, max_kv_len: int = 0,
                              num_splits: int = 0, flags: int = 0,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """paged_decode_attn without a workspace: split partials go to the library's fixed
    per-GPU scratch, so neither this call nor the library allocates anything.  The
    caller passes out and lse.  Calls overlapping on one GPU share that scratch."""
    if out is None or lse is None:
        raise ValueError("paged_decode_attn_noalloc writes into caller buffers: pass out and lse")
    L = load_library()
    p, g, _, _, out, lse = _decode_args(q, k_pool, v_pool, page_table, batch_idx, kv_len,
                                        page_size, num_splits, flags, None, out, lse,
                                        alloc_workspace=False)
    rc = L.paged_decode_attn_noalloc(p["q"], p["k_pool"], p["v_pool"], g["num_pages"], page_size,
                                     g["H_kv"], g["D"], p["page_table"], g["num_slots"],
                                     g["max_blocks"], p["batch_idx"], p["kv_len"], g["B"],
                                     g["H_q"], float(scale), int(max_kv_len), int(num_splits),
                                     int(flags), p["out"], p["lse"], _stream(stream))
    _check(rc, "paged_decode_attn_noalloc")
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
    p, g, ws_ptr, ws_bytes, out, lse = _decode_args(q, k_pool, v_pool, page_table, batch_idx,
                                                    kv_len, page_size, num_splits, flags,
                                                    workspace, out, lse)
    new_shape = (g["B"], g["H_kv"], g["D"])
    rc = L.paged_decode_attn_append(
        p["q"], _dev(k_new, "k_new", torch.bfloat16, 3, new_shape, q.device),
        _dev(v_new, "v_new", torch.bfloat16, 3, new_shape, q.device), p["k_pool"], p["v_pool"],
        g["num_pages"], page_size, g["H_kv"], g["D"], p["page_table"], g["num_slots"],
        g["max_blocks"], p["batch_idx"], p["kv_len"], g["B"], g["H_q"], float(scale),
        int(max_kv_len), int(num_splits), int(flags), ws_ptr, ws_bytes, p["out"], p["lse"],
        _stream(stream))
    _check(rc, "paged_decode_attn_append")
    return out, lse


def _prefill_args(q, k, v, cu_seqlens, out, lse):
    """Shapes, pointers and output buffers shared by the prefill wrappers."""
    Lt, H_q, D = q.shape
    H_kv = k.shape[1] if k.dim() == 3 else 0
    dv = q.device
    n_docs = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((Lt, H_q, D), dtype=torch.bfloat16, device=dv)
    if lse is None:
        lse = torch.empty((Lt, H_q), dtype=torch.float32, device=dv)
    ptrs = dict(
        q=_dev(q, "q", torch.bfloat16, 3),
        k=_dev(k, "k", torch.bfloat16, 3, (Lt, H_kv, D), dv),
        v=_dev(v, "v", torch.bfloat16, 3, (Lt, H_kv, D), dv),
        cu_seqlens=_dev(cu_seqlens, "cu_seqlens", torch.int32, 1, device=dv),
        out=_dev(out, "out", torch.bfloat16, 3, (Lt, H_q, D), dv),
        lse=_dev(lse, "lse", torch.float32, 2, (Lt, H_q), dv))
    geo = dict(L=Lt, H_q=H_q, H_kv=H_kv, D=D, n_docs=n_docs)
    return ptrs, geo, out, lse


def _pool_args(k_pool, v_pool, page_table, page_size, H_kv, D, device):
    """Pointers and sizes of the paged pools the fused prefill calls write."""
    if k_pool.dim() != 3:
        raise ValueError("k_pool must be [H_kv, num_pages*page_size, D]")
    Hp, rows, Dp = k_pool.shape
    if Hp != H_kv or Dp != D or rows % page_size:
        raise ValueError("pool shape does not match k / page_size")
    num_slots, max_blocks = page_table.shape
    ptrs = dict(k_pool=_dev(k_pool, "k_pool", torch.bfloat16, 3, device=device),
                v_pool=_dev(v_pool, "v_pool", torch.bfloat16, 3, k_pool.shape, device),
                page_table=_dev(page_table, "page_table", torch.int32, 2, device=device))
    return ptrs, dict(num_pages=rows // page_size, num_slots=num_slots, max_blocks=max_blocks)


def packed_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, scale: float,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Document-causal prefill; returns (out bf16 [L, H_q, D], lse fp32 [L, H_q])."""
    L = load_library()
    p, g, out, lse = _prefill_args(q, k, v, cu_seqlens, out, lse)
    rc = L.packed_prefill_attn(p["q"], p["k"], p["v"], p["cu_seqlens"], g["n_docs"], g["L"],
                               g["H_q"], g["H_kv"], g["D"], float(scale), p["out"], p["lse"],
                               _stream(stream))
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
    p, g, out, lse = _prefill_args(q, k, v, cu_seqlens, out, lse)
    pp, pg = _pool_args(k_pool, v_pool, page_table, page_size, g["H_kv"], g["D"], q.device)
    rc = L.packed_prefill_attn_append(
        p["q"], p["k"], p["v"], p["cu_seqlens"], g["n_docs"], g["L"], g["H_q"], g["H_kv"],
        g["D"], float(scale), p["out"], p["lse"], pp["k_pool"], pp["v_pool"], pg["num_pages"],
        page_size, pp["page_table"], pg["num_slots"], pg["max_blocks"],
        _dev(doc_slots, "doc_slots", torch.int32, 1, (g["n_docs"],), q.device), _stream(stream))
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
    p, g, out, lse = _prefill_args(q, k, v, cu_seqlens, out, lse)
    pp, pg = _pool_args(k_pool, v_pool, page_table, page_size, g["H_kv"], g["D"], q.device)
    nd = (g["n_docs"],)
    rc = L.paged_prefill_attn(
        p["q"], p["k"], p["v"], p["cu_seqlens"],
        _dev(prefix_lens, "prefix_lens", torch.int32, 1, nd, q.device),
        _dev(doc_slots, "doc_slots", torch.int32, 1, nd, q.device), g["n_docs"], g["L"], g["H_q"],
        g["H_kv"], g["D"], float(scale), pp["k_pool"], pp["v_pool"], pg["num_pages"], page_size,
        pp["page_table"], pg["num_slots"], pg["max_blocks"], p["out"], p["lse"], _stream(stream))
    _check(rc, "paged_prefill_attn")
    return out, lse


def validate_decode(page_table: torch.Tensor, batch_idx: torch.Tensor, kv_len: torch.Tensor,
                    page_size: int, num_pages: int, report: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Debug check of decode's device-side inputs.  Returns the int32 report [4] on the GPU:
    (violating rows, first violating row or -1, its PKV_V_* code, block or -1)."""
    L = load_library()
    B = batch_idx.shape[0]
    dv = batch_idx.device
    num_slots, max_blocks = page_table.shape
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=dv)
    rc = L.pkv_validate_decode(_dev(page_table, "page_table", torch.int32, 2, device=dv),
                               num_pages, page_size, num_slots, max_blocks,
                               _dev(batch_idx, "batch_idx", torch.int32, 1),
                               _dev(kv_len, "kv_len", torch.int32, 1, (B,), dv), B,
                               _dev(report, "report", torch.int32, 1, (4,), dv), _stream(stream))
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
    dv = cu_seqlens.device
    num_slots, max_blocks = page_table.shape if page_table is not None else (1, 1)
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=dv)
    opt = lambda t, name, nd, shp: (  # noqa: E731
        _dev(t, name, torch.int32, nd, shp, dv) if t is not None else None)
    rc = L.pkv_validate_prefill(_dev(cu_seqlens, "cu_seqlens", torch.int32, 1), n_docs, total_len,
                                opt(doc_slots, "doc_slots", 1, (n_docs,)),
                                opt(prefix_lens, "prefix_lens", 1, (n_docs,)),
                                opt(page_table, "page_table", 2, None), num_pages, page_size,
                                num_slots, max_blocks,
                                _dev(report, "report", torch.int32, 1, (4,), dv), _stream(stream))
    _check(rc, "pkv_validate_prefill")
    return report
