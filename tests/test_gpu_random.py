"""Seeded random sweep of the decode, fused decode, fused prefill and chunked prefill entry
points against the float64 oracle: shapes, GQA ratios, page sizes, layouts, schedules and
flags drawn together, so combinations the targeted tests do not name are covered too."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from workloads import make_chunked_prefill_case, make_decode_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_attention_23_amd as pkv  # noqa: E402
from gpu_util import check_close, dev_bf16, dev_i32, host_bits  # noqa: E402

# PKV_RANDOM_SWEEP=n multiplies the number of drawn cases per test (default 1).
SWEEP = max(1, int(os.environ.get("PKV_RANDOM_SWEEP", "1")))
GQA = [(8, 8), (16, 8), (32, 8), (12, 4), (16, 2), (16, 1), (32, 2)]


def _draw(rng):
    H_q, H_kv = GQA[rng.integers(len(GQA))]
    ps = int(rng.choice([16, 32, 64, 128, 256]))
    B = int(rng.integers(1, 40))
    lens = [int(x) for x in rng.integers(0, 700, B)]
    slots = [0 if rng.random() < 0.15 else r + 1 for r in range(B)]
    return H_q, H_kv, ps, B, lens, slots


@pytest.mark.parametrize("seed", range(12 * SWEEP))
def test_random_decode(seed):
    rng = np.random.default_rng(1000 + seed)
    H_q, H_kv, ps, B, lens, slots = _draw(rng)
    D = int(rng.choice([64, 128]))
    fused = bool(rng.random() < 0.5)
    layout = str(rng.choice(["shuffled", "sequential"]))
    sched = rng.integers(0, 4)   # 0: auto, 1: single, 2: per-row splits, 3: balanced
    flags = int(rng.choice([0, pkv.PKV_F_NO_CONTIG_DETECT]))
    print(f"random decode seed={seed} B={B} G={H_q // H_kv} D={D} ps={ps} fused={fused} "
          f"sched={sched}", flush=True)
    lens = [max(n, 1) if fused and s else n for n, s in zip(lens, slots)]
    need = sum(-(-n // ps) for n, s in zip(lens, slots) if s and n)
    mb = max([-(-n // ps) for n in lens] + [1])
    c = make_decode_case(name="rand", seed=seed, H_q=H_q, H_kv=H_kv, D=D, page_size=ps,
                         num_pages=need + 2, num_slots=B + 1, max_blocks=mb, row_slots=slots,
                         row_lens=lens, layout=layout, fill="nan", append_last=fused)
    kp, vp = c.k_pool, c.v_pool
    if fused:
        kp, vp = oracle.append_pages(kp, vp, c.num_pages, ps, c.page_table, c.app_batch_idx,
                                     c.app_input_pos, c.app_k, c.app_v)
    out_ref, lse_ref = oracle.decode_case(c, kp, vp)
    S = {0: 0, 1: 1, 2: int(rng.integers(2, 9)), 3: 0}[int(sched)]
    flags |= pkv.PKV_F_BALANCED if sched == 3 else 0
    kd, vd = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    args = (kd, vd, dev_i32(c.page_table), dev_i32(c.batch_idx), dev_i32(c.kv_len))
    kw = dict(page_size=ps, scale=float(c.scale), max_kv_len=int(max(lens)), num_splits=S,
              flags=flags)
    if fused:
        kn = np.zeros((B, H_kv, D), np.uint16)
        vn = np.zeros_like(kn)
        kn[c.active_rows()], vn[c.active_rows()] = c.app_k, c.app_v
        out, lse = pkv.paged_decode_attn_append(dev_bf16(c.q), dev_bf16(kn), dev_bf16(vn), *args, **kw)
    else:
        out, lse = pkv.paged_decode_attn(dev_bf16(c.q), *args, **kw)
    torch.cuda.synchronize()
    check_close(out, lse, out_ref, lse_ref, f"random decode seed{seed}")
    assert np.array_equal(host_bits(kd), kp) and np.array_equal(host_bits(vd), vp)


@pytest.mark.parametrize("seed", range(8 * SWEEP))
def test_random_chunked_prefill(seed):
    rng = np.random.default_rng(2000 + seed)
    H_q, H_kv, ps, B, _, slots = _draw(rng)
    B = min(B, 24)
    slots = slots[:B]
    prefix = [int(x) for x in rng.integers(0, 500, B)]
    chunk = [int(x) for x in rng.integers(0, 200, B)]
    if rng.random() < 0.3:
        prefix = [0] * B
    D = int(rng.choice([64, 128]))
    print(f"random chunked seed={seed} B={B} G={H_q // H_kv} D={D} ps={ps}", flush=True)
    c = make_chunked_prefill_case(name="rand", seed=seed, prefix_lens=prefix, chunk_lens=chunk,
                                  H_q=H_q, H_kv=H_kv, D=D, page_size=ps, slots=slots)
    if c.L == 0:
        pytest.skip("empty draw")
    kp, vp = oracle.append_pages(c.k_pool, c.v_pool, c.num_pages, ps, c.page_table, c.batch_idx,
                                 c.input_pos, c.k, c.v)
    out_ref, lse_ref = oracle.decode(c.q, kp, vp, c.num_pages, ps, c.page_table, c.batch_idx,
                                     np.zeros(c.L, np.int32), c.input_pos + 1, c.scale)
    kd, vd = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    out, lse = pkv.paged_prefill_attn(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v),
                                      dev_i32(c.cu_seqlens), dev_i32(c.prefix_lens),
                                      dev_i32(c.doc_slots), float(c.scale), kd, vd,
                                      dev_i32(c.page_table), ps)
    torch.cuda.synchronize()
    check_close(out, lse, out_ref, lse_ref, f"random chunked seed{seed}")
    assert np.array_equal(host_bits(kd), kp) and np.array_equal(host_bits(vd), vp)


@pytest.mark.parametrize("seed", range(8 * SWEEP))
def test_random_packed_prefill(seed):
    """Packed prefill, plain or with the fused scatter, over drawn document mixes (empty and
    single-token documents included), GQA ratios, head dims and page sizes."""
    from workloads import BF16_NAN, make_prefill_case
    rng = np.random.default_rng(3000 + seed)
    H_q, H_kv, ps, _, _, _ = _draw(rng)
    n = int(rng.integers(1, 40))
    lens = [int(x) for x in rng.integers(0, 600, n)]
    for i in rng.choice(n, size=min(n, 3), replace=False):
        lens[i] = int(rng.choice([0, 1, 2]))
    D = int(rng.choice([64, 128]))
    fused = bool(rng.random() < 0.5)
    print(f"random packed prefill seed={seed} docs={n} G={H_q // H_kv} D={D} ps={ps} "
          f"fused={fused}", flush=True)
    pc = make_prefill_case(name="rand", seed=seed, doc_lens=lens, H_q=H_q, H_kv=H_kv, D=D,
                           page_size=ps, num_pages=sum(-(-x // ps) for x in lens) + 2,
                           max_blocks=max([-(-x // ps) for x in lens] + [1]))
    if pc.L == 0:
        pytest.skip("empty draw")
    out_ref, lse_ref = oracle.prefill_case(pc)
    q, k, v, cu = dev_bf16(pc.q), dev_bf16(pc.k), dev_bf16(pc.v), dev_i32(pc.cu_seqlens)
    if not fused:
        out, lse = pkv.packed_prefill_attn(q, k, v, cu, float(pc.scale))
        torch.cuda.synchronize()
        check_close(out, lse, out_ref, lse_ref, f"random packed seed{seed}")
        return
    shape = (pc.H_kv, pc.num_pages * ps, D)
    kp0 = np.full(shape, BF16_NAN, np.uint16)
    kd, vd = dev_bf16(kp0), dev_bf16(kp0)
    slots = np.arange(1, pc.n_docs + 1, dtype=np.int32)
    out, lse = pkv.packed_prefill_attn_append(q, k, v, cu, float(pc.scale), kd, vd,
                                              dev_i32(pc.page_table), dev_i32(slots), ps)
    torch.cuda.synchronize()
    check_close(out, lse, out_ref, lse_ref, f"random fused prefill seed{seed}")
    kr, vr = oracle.append_pages(kp0, kp0.copy(), pc.num_pages, ps, pc.page_table, pc.batch_idx,
                                 pc.input_pos, pc.k, pc.v)
    assert np.array_equal(host_bits(kd), kr) and np.array_equal(host_bits(vd), vr)
