"""Checks that pin the CPU reference to facts other than itself.

Each pin_* function raises AssertionError when the reference disagrees with
what the mathematics or a library routine fixes.  They run through whatever
build of oracle.c is active (oracle.use_library), so the mutation tests can
run the same pins against deliberately broken copies.

Sources: flex paged-attention commit page ("Why this works": pool layout,
page table, slot 0 / page 0 padding); qwen3_flex_inference.py page (cache
update before attention, scale and GQA, decode causal offset, packed
document-causal prefill, last-token positions cumsum(lengths) - 1);
flex_vs_vllm.md page ("What broke correctness": padded rows must not NaN).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import brute
from workloads import BF16_NAN, bf16_bits_to_f32, f32_to_bf16_bits, make_decode_case, \
    make_prefill_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _phys_rows(case, r):
    """Physical pool row of each logical key of row r (test-side page walk)."""
    s, n, ps = int(case.batch_idx[r]), int(case.kv_len[r]), case.page_size
    j = np.arange(n)
    return case.page_table[s, j // ps].astype(np.int64) * ps + j % ps


def _full_decode(case, kp=None, vp=None):
    return oracle.decode_case(case, kp, vp)


# ---------------------------------------------------------------- worked example
def pin_golden_two_keys():
    """Closed-form example in tests/golden/two_keys.json (softmax of scores 0 and 1)."""
    with open(os.path.join(GOLDEN, "two_keys.json")) as f:
        g = json.load(f)
    q = np.array(g["q_bits"], dtype=np.uint16).reshape(1, 1, -1)
    D = q.shape[2]
    ps = g["page_size"]
    kp = np.full((1, 2 * ps, D), BF16_NAN, dtype=np.uint16)
    vp = np.full((1, 2 * ps, D), BF16_NAN, dtype=np.uint16)
    for j, (kb, vb) in enumerate(zip(g["k_bits"], g["v_bits"])):
        kp[0, ps + j] = kb
        vp[0, ps + j] = vb
    pt = np.array([[0], [1]], dtype=np.int32)
    out, lse = oracle.decode(q, kp, vp, 2, ps, pt, np.array([1], np.int32),
                             np.array([0], np.int32), np.array([len(g["k_bits"])], np.int32),
                             np.float32(g["scale"]))
    exp_o = np.array(g["expected_out"], dtype=np.float64)
    assert np.allclose(out[0, 0], exp_o, rtol=0, atol=1e-15), (out[0, 0], exp_o)
    assert abs(lse[0, 0] - g["expected_lse"]) <= 1e-15, (lse[0, 0], g["expected_lse"])


# ---------------------------------------------------------------- P1
def pin_dense_equivalence():
    """Identity (sequential) page table: equals torch float64 SDPA on the dense K/V."""
    case = make_decode_case(name="p1", seed=11, H_q=8, H_kv=2, D=32, page_size=16, num_pages=64,
                            num_slots=5, max_blocks=8, row_slots=[1, 2, 3, 4],
                            row_lens=[1, 17, 64, 100], layout="sequential", fill="nan")
    out, lse = _full_decode(case)
    G = case.H_q // case.H_kv
    for r in range(case.B):
        rows = _phys_rows(case, r)
        base = int(case.page_table[case.batch_idx[r], 0]) * case.page_size
        assert np.array_equal(rows, base + np.arange(case.kv_len[r]))  # really dense
        K = torch.from_numpy(_f64(case.k_pool[:, rows, :]))[None]  # [1, H_kv, n, D]
        V = torch.from_numpy(_f64(case.v_pool[:, rows, :]))[None]
        Q = torch.from_numpy(_f64(case.q[r]))[None, :, None, :]    # [1, H_q, 1, D]
        sc = float(case.scale)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=sc, enable_gqa=True)
        Ke = K.repeat_interleave(G, dim=1)
        ref_lse = torch.logsumexp((Q @ Ke.transpose(-1, -2))[0, :, 0, :] * sc, dim=-1)
        assert np.allclose(out[r], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)
        assert np.allclose(lse[r], ref_lse.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P2
def pin_page_permutation_invariance():
    """Relabelling physical pages (pool contents and table together) changes nothing, bitwise."""
    case = make_decode_case(name="p2", seed=12, H_q=4, H_kv=2, D=16, page_size=8, num_pages=40,
                            num_slots=4, max_blocks=10, row_slots=[1, 2, 3],
                            row_lens=[5, 33, 80], layout="shuffled", fill="nan")
    out, lse = _full_decode(case)
    rng = np.random.default_rng(7)
    perm = np.concatenate([[0], 1 + rng.permutation(case.num_pages - 1)])  # page p -> perm[p]
    ps = case.page_size
    kp = np.empty_like(case.k_pool)
    vp = np.empty_like(case.v_pool)
    for p in range(case.num_pages):
        kp[:, perm[p] * ps:(perm[p] + 1) * ps] = case.k_pool[:, p * ps:(p + 1) * ps]
        vp[:, perm[p] * ps:(perm[p] + 1) * ps] = case.v_pool[:, p * ps:(p + 1) * ps]
    pt2 = perm[case.page_table].astype(np.int32)
    out2, lse2 = oracle.decode(case.q, kp, vp, case.num_pages, ps, pt2, case.batch_idx,
                               np.zeros(case.B, np.int32), case.kv_len, case.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------- P3
def pin_single_key():
    """One valid key: O = v_0 exactly and LSE = scale * q.k_0."""
    case = make_decode_case(name="p3", seed=13, H_q=6, H_kv=3, D=24, page_size=4, num_pages=8,
                            num_slots=3, max_blocks=2, row_slots=[2, 1], row_lens=[1, 1],
                            layout="shuffled", fill="nan")
    out, lse = _full_decode(case)
    G = case.H_q // case.H_kv
    for r in range(case.B):
        row = _phys_rows(case, r)[0]
        for h in range(case.H_q):
            g = h // G
            v0 = _f64(case.v_pool[g, row])
            k0 = _f64(case.k_pool[g, row])
            qv = _f64(case.q[r, h])
            assert np.array_equal(out[r, h], v0)
            want = float(case.scale) * math.fsum(qv * k0)
            assert abs(lse[r, h] - want) <= 1e-12 * max(1.0, abs(want))


# ---------------------------------------------------------------- P4
def pin_uniform_scores():
    """q = 0: O is the mean of the valid v_j and LSE = ln n exactly."""
    case = make_decode_case(name="p4", seed=14, H_q=4, H_kv=1, D=16, page_size=8, num_pages=32,
                            num_slots=4, max_blocks=8, row_slots=[3, 1, 2],
                            row_lens=[3, 29, 64], layout="shuffled", fill="nan")
    case.q[:] = 0
    out, lse = _full_decode(case)
    for r in range(case.B):
        rows = _phys_rows(case, r)
        n = len(rows)
        mean = _f64(case.v_pool[0, rows]).mean(axis=0)
        for h in range(case.H_q):
            assert lse[r, h] == math.log(n), (lse[r, h], math.log(n))
            assert np.allclose(out[r, h], mean, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P5
def _needle_case(n_rows, lens, ps, seed):
    return make_decode_case(name="p5", seed=seed, H_q=8, H_kv=2, D=32, page_size=ps,
                            num_pages=1 + sum(-(-n // ps) for n in lens) + 4,
                            num_slots=n_rows + 1, max_blocks=max(-(-n // ps) for n in lens),
                            row_slots=list(range(1, n_rows + 1)), row_lens=lens,
                            layout="shuffled", fill="zero")


def pin_needles():
    """A key equal to 8x the (shared) query dominates: O ~ v at that key.

    Needles sit at the first and last position of every page and at n-1;
    a needle planted just past the valid range must not be picked up.
    """
    ps = 16
    n = 70  # last page is partial: positions 70..79 exist in the pool but are invalid
    positions = sorted({p for b in range(0, n, ps) for p in (b, min(b + ps - 1, n - 1))} | {n - 1})
    lens = [n] * (len(positions) + 1)
    case = _needle_case(len(lens), lens, ps, seed=15)
    G = case.H_q // case.H_kv
    # every row: all heads of a group share one query
    for r in range(case.B):
        for g in range(case.H_kv):
            case.q[r, g * G:(g + 1) * G] = case.q[r, g * G]
    targets = positions + [n]  # last row: needle at the invalid position n
    ps_ = case.page_size
    for r, jstar in enumerate(targets):
        s = int(case.batch_idx[r])
        phys = int(case.page_table[s, jstar // ps_]) * ps_ + jstar % ps_
        for g in range(case.H_kv):
            qv = bf16_bits_to_f32(case.q[r, g * G])
            case.k_pool[g, phys] = f32_to_bf16_bits(8.0 * qv)
            if jstar >= n:  # make a wrongly admitted key impossible to miss
                case.v_pool[g, phys] = f32_to_bf16_bits(np.full(case.D, 5.0, np.float32))
    out, _ = _full_decode(case)
    for r, jstar in enumerate(targets):
        s = int(case.batch_idx[r])
        phys = int(case.page_table[s, jstar // ps_]) * ps_ + jstar % ps_
        for h in range(case.H_q):
            v = _f64(case.v_pool[h // G, phys])
            err = np.abs(out[r, h] - v).max()
            if jstar < n:
                assert err <= 1e-9, (r, jstar, h, err)
            else:
                assert err > 1e-3, (r, jstar, h, err)


# ---------------------------------------------------------------- P6
def pin_brute_force():
    """Independent pure-Python brute force agrees on tiny shapes, all sub-ranges."""
    for ps, seed in ((2, 21), (4, 22)):
        case = make_decode_case(name="p6", seed=seed, H_q=4, H_kv=2, D=8, page_size=ps,
                                num_pages=48, num_slots=4, max_blocks=20,
                                row_slots=[0, 2, 3], row_lens=[5, 13, 40], layout="shuffled",
                                fill="nan")
        B = case.B
        rng = np.random.default_rng(seed)
        for trial in range(3):
            lo = np.array([0 if trial == 0 else rng.integers(0, n + 1) for n in case.kv_len], np.int32)
            hi = np.array([n if trial == 0 else rng.integers(l, n + 1) for l, n in zip(lo, case.kv_len)],
                          np.int32)
            out, lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.num_pages, ps,
                                     case.page_table, case.batch_idx, lo, hi, case.scale)
            bo, bl = brute.decode(case.q, case.k_pool, case.v_pool, ps, case.page_table,
                                  case.batch_idx, lo, hi, case.scale)
            bo, bl = np.array(bo), np.array(bl)
            assert np.allclose(out, bo, rtol=0, atol=1e-12)
            fin = np.isfinite(bl)
            assert np.array_equal(fin, np.isfinite(lse))
            assert np.allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)
        del B
    pc = make_prefill_case(name="p6p", seed=23, doc_lens=[3, 0, 1, 7, 5], H_q=4, H_kv=2, D=8,
                           page_size=4, num_pages=16, max_blocks=2)
    out, lse = oracle.prefill_case(pc)
    bo, bl = brute.prefill(pc.q, pc.k, pc.v, pc.cu_seqlens, pc.scale)
    assert np.allclose(out, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12)
    # append: tokens into pages, including padding slot, page-0 blocks and repeats of a slot
    kp0 = np.full((pc.H_kv, pc.num_pages * pc.page_size, pc.D), BF16_NAN, np.uint16)
    vp0 = kp0.copy()
    bi = pc.batch_idx.copy()
    bi[0] = 0
    ka, va = oracle.append_pages(kp0, vp0, pc.num_pages, pc.page_size, pc.page_table, bi,
                                 pc.input_pos, pc.k, pc.v)
    kb, vb = brute.append(kp0, vp0, pc.num_pages, pc.page_size, pc.page_table, bi, pc.input_pos,
                          pc.k, pc.v)
    assert np.array_equal(ka, np.array(kb, np.uint16)) and np.array_equal(va, np.array(vb, np.uint16))


# ---------------------------------------------------------------- P7
def pin_padding_rows():
    """batch_idx = 0 (any kv_len) or kv_len = 0 gives exactly (+0.0, -inf), even over a NaN pool."""
    case = make_decode_case(name="p7", seed=24, H_q=4, H_kv=2, D=16, page_size=8, num_pages=16,
                            num_slots=3, max_blocks=4, row_slots=[0, 1, 0, 2],
                            row_lens=[1, 20, 37, 5], layout="shuffled", fill="nan")
    kv_len = case.kv_len.copy()
    kv_len[3] = 0
    out, lse = oracle.decode(case.q, case.k_pool, case.v_pool, case.num_pages, case.page_size,
                             case.page_table, case.batch_idx, np.zeros(case.B, np.int32), kv_len,
                             case.scale)
    for r in (0, 2, 3):
        assert np.all(out[r] == 0.0) and not np.any(np.signbit(out[r]))
        assert np.all(lse[r] == -np.inf)
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- P8
def pin_merge_identity():
    """Merging partials over any split of [0, n) (empty pieces included) gives the full result."""
    case = make_decode_case(name="p8", seed=25, H_q=8, H_kv=4, D=16, page_size=8, num_pages=64,
                            num_slots=5, max_blocks=16, row_slots=[1, 0, 2, 4],
                            row_lens=[1, 9, 100, 127], layout="shuffled", fill="nan")
    full_o, full_l = _full_decode(case)
    rng = np.random.default_rng(3)
    for S in (1, 2, 3, 7):
        cuts = np.zeros((case.B, S + 1), np.int32)
        for r in range(case.B):
            n = int(case.kv_len[r])
            inner = np.sort(rng.integers(0, n + 1, size=S - 1))
            cuts[r] = np.concatenate([[0], inner, [n]])
        parts_o, parts_l = [], []
        for s in range(S):
            o, l = oracle.decode(case.q, case.k_pool, case.v_pool, case.num_pages,
                                 case.page_size, case.page_table, case.batch_idx,
                                 cuts[:, s].copy(), cuts[:, s + 1].copy(), case.scale)
            parts_o.append(o)
            parts_l.append(l)
        mo, ml = oracle.merge(np.stack(parts_o), np.stack(parts_l))
        assert np.allclose(mo, full_o, rtol=0, atol=1e-12)
        fin = np.isfinite(full_l)
        assert np.array_equal(fin, np.isfinite(ml))
        assert np.allclose(ml[fin], full_l[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P9
def pin_prefill_special_cases():
    """Length-1 documents, one document vs torch causal SDPA, document-order permutation."""
    # (a) documents of length 1: O_i = v_i, LSE_i = scale * q_i . k_i
    pc = make_prefill_case(name="p9a", seed=26, doc_lens=[1] * 6, H_q=4, H_kv=2, D=16,
                           page_size=4, num_pages=16, max_blocks=1)
    out, lse = oracle.prefill_case(pc)
    for i in range(pc.L):
        for h in range(pc.H_q):
            g = h // 2
            assert np.array_equal(out[i, h], _f64(pc.v[i, g]))
            want = float(pc.scale) * math.fsum(_f64(pc.q[i, h]) * _f64(pc.k[i, g]))
            assert abs(lse[i, h] - want) <= 1e-12 * max(1.0, abs(want))
    # (b) a single document: causal SDPA with GQA in float64
    pc = make_prefill_case(name="p9b", seed=27, doc_lens=[45], H_q=8, H_kv=2, D=32,
                           page_size=16, num_pages=8, max_blocks=3)
    out, lse = oracle.prefill_case(pc)
    Q = torch.from_numpy(_f64(pc.q)).permute(1, 0, 2)[None]   # [1, H_q, L, D]
    K = torch.from_numpy(_f64(pc.k)).permute(1, 0, 2)[None]
    V = torch.from_numpy(_f64(pc.v)).permute(1, 0, 2)[None]
    sc = float(pc.scale)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sc,
                                                           enable_gqa=True)
    assert np.allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    Ke = K.repeat_interleave(4, dim=1)
    sco = (Q @ Ke.transpose(-1, -2))[0] * sc
    mask = torch.ones(pc.L, pc.L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(sco.masked_fill(~mask, -math.inf), dim=-1)  # [H_q, L]
    assert np.allclose(lse, ref_lse.T.numpy(), rtol=0, atol=1e-12)
    # (c) permuting document order permutes rows identically
    pc = make_prefill_case(name="p9c", seed=28, doc_lens=[5, 12, 1, 9], H_q=4, H_kv=1, D=16,
                           page_size=4, num_pages=16, max_blocks=3)
    out, lse = oracle.prefill_case(pc)
    order = [2, 0, 3, 1]
    cu = pc.cu_seqlens
    idx = np.concatenate([np.arange(cu[d], cu[d + 1]) for d in order])
    lens = [cu[d + 1] - cu[d] for d in order]
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out2, lse2 = oracle.prefill(pc.q[idx], pc.k[idx], pc.v[idx], cu2, pc.scale)
    assert np.array_equal(out2, out[idx]) and np.array_equal(lse2, lse[idx])


# ---------------------------------------------------------------- P10
def pin_scatter():
    """Append equals numpy fancy-index assignment, byte for byte, with skips for slot/page 0."""
    pc = make_prefill_case(name="p10", seed=29, doc_lens=[7, 1, 19, 4], H_q=4, H_kv=2, D=8,
                           page_size=4, num_pages=24, max_blocks=5)
    kp0 = np.full((pc.H_kv, pc.num_pages * pc.page_size, pc.D), BF16_NAN, np.uint16)
    vp0 = kp0.copy()
    bi = pc.batch_idx.copy()
    pos = pc.input_pos.copy()
    pt = pc.page_table.copy()
    bi[3] = 0                      # a padding token
    pt[3, 1] = 0                   # doc 2 block 1 unmapped: its tokens must not be written
    ka, va = oracle.append_pages(kp0, vp0, pc.num_pages, pc.page_size, pt, bi, pos, pc.k, pc.v)
    ps = pc.page_size
    page = pt[bi, pos // ps]
    keep = (bi != 0) & (page != 0)
    rows = page[keep].astype(np.int64) * ps + pos[keep] % ps
    kr, vr = kp0.copy(), vp0.copy()
    kr[:, rows, :] = pc.k[keep].transpose(1, 0, 2)
    vr[:, rows, :] = pc.v[keep].transpose(1, 0, 2)
    assert keep.sum() < pc.L and np.any(~keep)
    assert np.array_equal(ka, kr) and np.array_equal(va, vr)
    assert np.all(ka[:, :ps] == BF16_NAN)  # page 0 never touched


# ---------------------------------------------------------------- P11
def pin_prefill_decode_consistency():
    """Append a document's K/V into shuffled pages, decode its last query: equals prefill's last row."""
    pc = make_prefill_case(name="p11", seed=30, doc_lens=[9, 40, 1, 23], H_q=8, H_kv=2, D=16,
                           page_size=8, num_pages=24, max_blocks=5)
    out, lse = oracle.prefill_case(pc)
    kp0 = np.full((pc.H_kv, pc.num_pages * pc.page_size, pc.D), BF16_NAN, np.uint16)
    kp, vp = oracle.append_pages(kp0, kp0, pc.num_pages, pc.page_size, pc.page_table,
                                 pc.batch_idx, pc.input_pos, pc.k, pc.v)
    last = pc.cu_seqlens[1:] - 1
    qd = pc.q[last]
    slots = np.arange(1, pc.n_docs + 1, dtype=np.int32)
    lens = pc.doc_lens().astype(np.int32)
    do, dl = oracle.decode(qd, kp, vp, pc.num_pages, pc.page_size, pc.page_table, slots,
                           np.zeros_like(lens), lens, pc.scale)
    assert np.allclose(do, out[last], rtol=0, atol=1e-12)
    assert np.allclose(dl, lse[last], rtol=0, atol=1e-12)


ALL_PINS = [
    pin_golden_two_keys,
    pin_dense_equivalence,
    pin_page_permutation_invariance,
    pin_single_key,
    pin_uniform_scores,
    pin_needles,
    pin_brute_force,
    pin_padding_rows,
    pin_merge_identity,
    pin_prefill_special_cases,
    pin_scatter,
    pin_prefill_decode_consistency,
]
