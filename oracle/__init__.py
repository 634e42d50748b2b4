"""Python access to the float64 CPU reference (oracle.c) through ctypes.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use this package; the GPU library never imports it.

Each wrapper takes numpy arrays in the cache layout of the flex paged-attention
commit page ("Why this works", point 1) and returns float64 results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP, IEEE float64: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load(path):
    L = ctypes.CDLL(path)
    L.oracle_append.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _I, _P, _P]
    L.oracle_append.restype = _I
    L.oracle_decode.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _I, _I,
                                ctypes.c_double, _P, _P]
    L.oracle_decode.restype = _I
    L.oracle_merge.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.oracle_merge.restype = _I
    L.oracle_prefill.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_double, _P, _P]
    L.oracle_prefill.restype = _I
    L.oracle_num_threads.restype = _I
    L.oracle_set_threads.argtypes = [_I]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _load(_LIB_PATH)
    return _lib


def use_library(path: str) -> None:
    """Route every wrapper below through another build of oracle.c (used by the
    mutation tests, which check that the pins reject deliberately broken copies)."""
    global _lib
    _lib = _load(path)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def append_pages(k_pool, v_pool, num_pages, page_size, page_table, batch_idx, input_pos,
                 k_new, v_new):
    """KV append on copies of the pools ([H_kv][num_pages*page_size][D] uint16).

    Returns the new (k_pool, v_pool).  Bytes not written keep their values.
    """
    kp = np.array(k_pool, dtype=np.uint16, copy=True, order="C")
    vp = np.array(v_pool, dtype=np.uint16, copy=True, order="C")
    H_kv, rows, D = kp.shape
    assert rows == num_pages * page_size
    pt, ptp = _c(page_table, np.int32)
    num_slots, max_blocks = pt.shape
    bi, bip = _c(batch_idx, np.int32)
    ip, ipp = _c(input_pos, np.int32)
    kn, knp = _c(k_new, np.uint16)
    vn, vnp = _c(v_new, np.uint16)
    N = int(bi.shape[0])
    assert kn.shape == (N, H_kv, D) and vn.shape == (N, H_kv, D)
    rc = lib().oracle_append(kp.ctypes.data, vp.ctypes.data, num_pages, page_size, H_kv, D, ptp,
                             num_slots, max_blocks, bip, ipp, N, knp, vnp)
    if rc != 0:
        raise ValueError("oracle_append rejected its arguments")
    return kp, vp


def decode(q, k_pool, v_pool, num_pages, page_size, page_table, batch_idx, key_lo, key_hi,
           scale):
    """Decode attention of each row over its keys [key_lo, key_hi).

    q: uint16 [B, H_q, D]; pools uint16 [H_kv, num_pages*page_size, D].
    Returns (out float64 [B, H_q, D], lse float64 [B, H_q]).
    """
    qa, qp = _c(q, np.uint16)
    B, H_q, D = qa.shape
    kp, kpp = _c(k_pool, np.uint16)
    vp, vpp = _c(v_pool, np.uint16)
    H_kv = kp.shape[0]
    assert kp.shape == (H_kv, num_pages * page_size, D)
    pt, ptp = _c(page_table, np.int32)
    num_slots, max_blocks = pt.shape
    bi, bip = _c(batch_idx, np.int32)
    lo, lop = _c(key_lo, np.int32)
    hi, hip = _c(key_hi, np.int32)
    out = np.empty((B, H_q, D), dtype=np.float64)
    lse = np.empty((B, H_q), dtype=np.float64)
    rc = lib().oracle_decode(qp, kpp, vpp, num_pages, page_size, H_kv, D, ptp, num_slots,
                             max_blocks, bip, lop, hip, B, H_q, float(np.float32(scale)),
                             out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out, lse


def decode_case(case, k_pool=None, v_pool=None):
    """Full decode (keys [0, kv_len)) of a workloads.DecodeCase."""
    B = case.B
    return decode(case.q, case.k_pool if k_pool is None else k_pool,
                  case.v_pool if v_pool is None else v_pool, case.num_pages, case.page_size,
                  case.page_table, case.batch_idx, np.zeros(B, np.int32), case.kv_len, case.scale)


def merge(o_part, lse_part):
    """Merge split partials: o_part [S, B, H_q, D], lse_part [S, B, H_q] (float64)."""
    op, opp = _c(o_part, np.float64)
    lp, lpp = _c(lse_part, np.float64)
    S, B, H_q, D = op.shape
    out = np.empty((B, H_q, D), dtype=np.float64)
    lse = np.empty((B, H_q), dtype=np.float64)
    rc = lib().oracle_merge(S, B, H_q, D, opp, lpp, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_merge rejected its arguments")
    return out, lse


def prefill(q, k, v, cu_seqlens, scale):
    """Document-causal prefill over packed q [L, H_q, D], k/v [L, H_kv, D] (uint16 bf16 bits)."""
    qa, qp = _c(q, np.uint16)
    ka, kap = _c(k, np.uint16)
    va, vap = _c(v, np.uint16)
    L, H_q, D = qa.shape
    H_kv = ka.shape[1]
    cu, cup = _c(cu_seqlens, np.int32)
    out = np.empty((L, H_q, D), dtype=np.float64)
    lse = np.empty((L, H_q), dtype=np.float64)
    rc = lib().oracle_prefill(qp, kap, vap, cup, int(cu.shape[0] - 1), L, H_q, H_kv, D,
                              float(np.float32(scale)), out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return out, lse


def prefill_case(case):
    return prefill(case.q, case.k, case.v, case.cu_seqlens, case.scale)
