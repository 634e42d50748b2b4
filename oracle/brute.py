"""Independent pure-Python brute force for tiny shapes.

TEST INFRASTRUCTURE ONLY.  It is written separately from oracle.c (it shares
no code with it or with the GPU library) and exists to pin the C reference's
indexing on tiny inputs: explicit Python loops, math.fsum for every sum
(correctly rounded), and weights taken as exp(x_j - LSE) rather than via a
separate normaliser.  Inputs may be numpy arrays; all arithmetic is done on
Python floats and ints.

Definitions follow the flex paged-attention commit page ("Why this works"):
physical row = page_table[slot][pos // page_size] * page_size + pos % page_size,
slot 0 / page 0 are padding; the qwen3_flex_inference.py page for the
document-causal prefill mask; softmax attention with scale and GQA.
"""
from __future__ import annotations

import math
import struct


def _bf(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _attend(qv, keys, vals, scale):
    """Softmax attention of query vector qv over lists of key/value vectors."""
    D = len(qv)
    if not keys:
        return [0.0] * D, -math.inf
    xs = [scale * math.fsum(qv[d] * k[d] for d in range(D)) for k in keys]
    m = max(xs)
    lse = m + math.log(math.fsum(math.exp(x - m) for x in xs))
    ws = [math.exp(x - lse) for x in xs]
    out = [math.fsum(ws[j] * vals[j][d] for j in range(len(vals))) for d in range(D)]
    return out, lse


def decode(q, k_pool, v_pool, page_size, page_table, batch_idx, key_lo, key_hi, scale):
    """Decode rows over logical keys [key_lo[r], key_hi[r]); returns nested lists."""
    q = q.tolist()
    kp = k_pool.tolist()
    vp = v_pool.tolist()
    pt = page_table.tolist()
    B = len(q)
    H_q = len(q[0])
    H_kv = len(kp)
    G = H_q // H_kv
    scale = float(scale)
    outs, lses = [], []
    for r in range(B):
        s = int(batch_idx[r])
        lo, hi = int(key_lo[r]), int(key_hi[r])
        row_o, row_l = [], []
        for h in range(H_q):
            g = h // G
            keys, vals = [], []
            if s != 0:
                for j in range(lo, hi):
                    phys = pt[s][j // page_size] * page_size + j % page_size
                    keys.append([_bf(x) for x in kp[g][phys]])
                    vals.append([_bf(x) for x in vp[g][phys]])
            o, l = _attend([_bf(x) for x in q[r][h]], keys, vals, scale)
            row_o.append(o)
            row_l.append(l)
        outs.append(row_o)
        lses.append(row_l)
    return outs, lses


def prefill(q, k, v, cu_seqlens, scale):
    """Packed document-causal attention; returns nested lists [L][H_q][D], [L][H_q]."""
    q = q.tolist()
    k = k.tolist()
    v = v.tolist()
    cu = [int(c) for c in cu_seqlens]
    L = len(q)
    H_q = len(q[0]) if L else 0
    H_kv = len(k[0]) if L else 1
    G = max(H_q // H_kv, 1)
    scale = float(scale)
    outs = [None] * L
    lses = [None] * L
    for d in range(len(cu) - 1):
        for i in range(cu[d], cu[d + 1]):
            row_o, row_l = [], []
            for h in range(H_q):
                g = h // G
                keys = [[_bf(x) for x in k[j][g]] for j in range(cu[d], i + 1)]
                vals = [[_bf(x) for x in v[j][g]] for j in range(cu[d], i + 1)]
                o, l = _attend([_bf(x) for x in q[i][h]], keys, vals, scale)
                row_o.append(o)
                row_l.append(l)
            outs[i] = row_o
            lses[i] = row_l
    return outs, lses


def append(k_pool, v_pool, num_pages, page_size, page_table, batch_idx, input_pos, k_new, v_new):
    """Token-by-token scatter into copies of the pools (nested lists of ints)."""
    kp = k_pool.tolist()
    vp = v_pool.tolist()
    pt = page_table.tolist()
    num_slots = len(pt)
    max_blocks = len(pt[0])
    kn = k_new.tolist()
    vn = v_new.tolist()
    for t in range(len(kn)):
        s, p = int(batch_idx[t]), int(input_pos[t])
        if s <= 0 or s >= num_slots or p < 0 or p // page_size >= max_blocks:
            continue
        page = pt[s][p // page_size]
        if page <= 0 or page >= num_pages:
            continue
        phys = page * page_size + p % page_size
        for h in range(len(kp)):
            kp[h][phys] = list(kn[t][h])
            vp[h][phys] = list(vn[t][h])
    return kp, vp
