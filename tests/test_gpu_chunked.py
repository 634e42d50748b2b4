"""GPU parity of paged_prefill_attn (chunked prefill over a paged prefix) against the
float64 oracle: the oracle scatters the chunks into the pages, then decodes every chunk
row over positions 0..its own (the definition the C ABI states)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_chunked_prefill_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_attention_23_amd as pkv  # noqa: E402
from gpu_util import check_close, dev_bf16, dev_i32, host_bits  # noqa: E402


def _expected(c):
    kp, vp = oracle.append_pages(c.k_pool, c.v_pool, c.num_pages, c.page_size, c.page_table,
                                 c.batch_idx, c.input_pos, c.k, c.v)
    out, lse = oracle.decode(c.q, kp, vp, c.num_pages, c.page_size, c.page_table, c.batch_idx,
                             np.zeros(c.L, np.int32), c.input_pos + 1, c.scale)
    return kp, vp, out, lse


def _run(c, kd=None, vd=None):
    kd = dev_bf16(c.k_pool) if kd is None else kd
    vd = dev_bf16(c.v_pool) if vd is None else vd
    out, lse = pkv.paged_prefill_attn(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v),
                                      dev_i32(c.cu_seqlens), dev_i32(c.prefix_lens),
                                      dev_i32(c.doc_slots), float(c.scale), kd, vd,
                                      dev_i32(c.page_table), c.page_size)
    torch.cuda.synchronize()
    return out, lse, host_bits(kd), host_bits(vd)


CASES = [
    # (seed, prefix_lens, chunk_lens, H_q, H_kv, page_size, slots[, head_dim])
    (91, [0, 1, 63, 64, 65, 200, 700], [1, 33, 64, 100, 5, 128, 300], 32, 8, 16, None),
    (92, [5, 0, 130, 1000], [70, 9, 1, 40], 16, 2, 64, None),               # G = 8
    (93, [300, 40, 17], [0, 64, 200], 16, 1, 128, None),                    # G = 16, empty chunk
    (94, [100, 250, 31, 0], [50, 20, 100, 80], 32, 8, 32, [1, 0, 3, 4]),    # slot-0 sequence
    (95, [2000], [1], 32, 8, 128, None),                                    # decode-like chunk
    (96, [int(x) for x in np.random.default_rng(96).integers(0, 400, 70)],
     [int(x) for x in np.random.default_rng(97).integers(1, 40, 70)], 32, 8, 16, None),  # 70 seqs
    # prefixes past 64 pages of 64 tokens (page ids beyond the per-tile window of 64)
    (99, [4700, 4160, 4096, 4095], [40, 64, 3, 1], 16, 2, 64, None),
    (100, [700, 257, 256, 255], [33, 100, 1, 64], 32, 8, 256, None),        # page_size 256
    # head_dim 64: a stage pass covers 32 keys, i.e. two 16-token pages
    (191, [0, 1, 63, 64, 65, 200, 700], [1, 33, 64, 100, 5, 128, 300], 32, 8, 16, None, 64),
    (192, [1100, 1024, 1023, 40], [40, 64, 3, 1], 16, 2, 16, [1, 0, 3, 4], 64),  # past 64 pages
    (193, [700, 257, 256, 255], [33, 100, 1, 64], 32, 8, 256, None, 64),
]


@pytest.mark.parametrize("spec", CASES, ids=[f"seed{s[0]}" for s in CASES])
def test_chunked_prefill(spec):
    seed, prefix, chunk, H_q, H_kv, ps, slots = spec[:7]
    D = spec[7] if len(spec) > 7 else 128
    print(f"chunked prefill seed={seed} D={D}", flush=True)
    c = make_chunked_prefill_case(name="chunk", seed=seed, prefix_lens=prefix, chunk_lens=chunk,
                                  H_q=H_q, H_kv=H_kv, D=D, page_size=ps, slots=slots)
    kp, vp, out_ref, lse_ref = _expected(c)
    out, lse, kb, vb = _run(c)
    check_close(out, lse, out_ref, lse_ref, f"chunked seed{seed}")
    assert np.array_equal(kb, kp) and np.array_equal(vb, vp)
    out2, lse2, _, _ = _run(c)   # deterministic
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


def test_chunked_zero_prefix_is_fused_prefill():
    """With every prefix 0 the result is packed_prefill_attn_append's, bit for bit."""
    print("chunked prefix 0", flush=True)
    c = make_chunked_prefill_case(name="p0", seed=98, prefix_lens=[0] * 6,
                                  chunk_lens=[1, 64, 129, 300, 17, 90], H_q=32, H_kv=8, D=128,
                                  page_size=128)
    out, lse, kb, vb = _run(c)
    kd, vd = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    o2, l2 = pkv.packed_prefill_attn_append(dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v),
                                            dev_i32(c.cu_seqlens), float(c.scale), kd, vd,
                                            dev_i32(c.page_table), dev_i32(c.doc_slots),
                                            c.page_size)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    assert np.array_equal(kb, host_bits(kd)) and np.array_equal(vb, host_bits(vd))


def test_chunked_two_steps_equal_one():
    """Prefilling a sequence in two chunks (the second over the first's pages) gives the
    rows of the one-chunk prefill (within tolerance: different tiling)."""
    print("chunked two steps", flush=True)
    n1, n2 = 150, 110
    whole = make_chunked_prefill_case(name="w", seed=99, prefix_lens=[0], chunk_lens=[n1 + n2],
                                      H_q=32, H_kv=8, D=128, page_size=64)
    kd, vd = dev_bf16(whole.k_pool), dev_bf16(whole.v_pool)
    ref_out, ref_lse, _, _ = _run(whole)
    pt, slots = dev_i32(whole.page_table), dev_i32(whole.doc_slots)
    outs = []
    for lo, hi, pre in ((0, n1, 0), (n1, n1 + n2, n1)):
        o, l = pkv.paged_prefill_attn(
            dev_bf16(whole.q[lo:hi]), dev_bf16(whole.k[lo:hi]), dev_bf16(whole.v[lo:hi]),
            dev_i32(np.array([0, hi - lo], np.int32)), dev_i32(np.array([pre], np.int32)), slots,
            float(whole.scale), kd, vd, pt, whole.page_size)
        torch.cuda.synchronize()
        outs.append((o.clone(), l.clone()))
    o = torch.cat([outs[0][0], outs[1][0]]).float()
    l = torch.cat([outs[0][1], outs[1][1]])
    assert (o - ref_out.float()).abs().max().item() <= 2e-2
    assert (l - ref_lse).abs().max().item() <= 1e-3
