"""The prefill entry points captured in HIP graphs: every replay, with eager work and
synchronisation between replays, equals the eager call bit for bit (outputs and, for
the calls that write pages, the pools), and the eager call matches the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import BF16_NAN, make_chunked_prefill_case, make_prefill_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_attention_23_amd as pkv  # noqa: E402
from gpu_util import check_close, dev_bf16, dev_i32  # noqa: E402


def _capture(fn):
    """One warm-up call on a side stream, then fn captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _replays(g, outs, refs, reset):
    for rep in range(3):
        reset()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(_bits(o), _bits(r)), rep


@pytest.mark.parametrize("D", [128, 64])
def test_packed_and_fused_prefill_graphs(D):
    print(f"prefill graphs D={D}", flush=True)
    lens = [300, 1, 0, 129, 700, 33]
    ps = 64
    pc = make_prefill_case(name="pg", seed=401 + D, doc_lens=lens, H_q=32, H_kv=8, D=D, page_size=ps,
                           num_pages=sum(-(-n // ps) for n in lens) + 2, max_blocks=12)
    out_ref, lse_ref = oracle.prefill_case(pc)
    q, k, v, cu = dev_bf16(pc.q), dev_bf16(pc.k), dev_bf16(pc.v), dev_i32(pc.cu_seqlens)
    sc = float(pc.scale)
    # attention only
    eo, el = pkv.packed_prefill_attn(q, k, v, cu, sc)
    torch.cuda.synchronize()
    check_close(eo, el, out_ref, lse_ref, f"eager packed D={D}")
    out, lse = torch.empty_like(eo), torch.empty_like(el)
    g = _capture(lambda: pkv.packed_prefill_attn(q, k, v, cu, sc, out=out, lse=lse))
    _replays(g, [out, lse], [eo, el], lambda: (out.zero_(), lse.zero_()))
    # with the scatter into pages
    shape = (pc.H_kv, pc.num_pages * ps, D)
    kp0 = np.full(shape, BF16_NAN, np.uint16)
    pt, slots = dev_i32(pc.page_table), dev_i32(np.arange(1, pc.n_docs + 1, dtype=np.int32))
    ek, ev = dev_bf16(kp0), dev_bf16(kp0)
    eo, el = pkv.packed_prefill_attn_append(q, k, v, cu, sc, ek, ev, pt, slots, ps)
    torch.cuda.synchronize()
    check_close(eo, el, out_ref, lse_ref, f"eager fused D={D}")
    kd, vd = dev_bf16(kp0), dev_bf16(kp0)
    out, lse = torch.empty_like(eo), torch.empty_like(el)
    g = _capture(lambda: pkv.packed_prefill_attn_append(q, k, v, cu, sc, kd, vd, pt, slots, ps,
                                                       out=out, lse=lse))
    nan = dev_bf16(kp0)

    def reset():
        out.zero_()
        lse.zero_()
        kd.copy_(nan)
        vd.copy_(nan)
    _replays(g, [out, lse, kd, vd], [eo, el, ek, ev], reset)


def test_chunked_prefill_graph():
    print("chunked prefill graph", flush=True)
    c = make_chunked_prefill_case(name="cg", seed=411, prefix_lens=[700, 0, 65, 300],
                                  chunk_lens=[40, 129, 1, 64], H_q=32, H_kv=8, D=128, page_size=32)
    kp, vp = oracle.append_pages(c.k_pool, c.v_pool, c.num_pages, c.page_size, c.page_table,
                                 c.batch_idx, c.input_pos, c.k, c.v)
    out_ref, lse_ref = oracle.decode(c.q, kp, vp, c.num_pages, c.page_size, c.page_table,
                                     c.batch_idx, np.zeros(c.L, np.int32), c.input_pos + 1, c.scale)
    q, k, v = dev_bf16(c.q), dev_bf16(c.k), dev_bf16(c.v)
    cu, pl, sl, pt = (dev_i32(c.cu_seqlens), dev_i32(c.prefix_lens), dev_i32(c.doc_slots),
                      dev_i32(c.page_table))
    sc = float(c.scale)
    ek, ev = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    eo, el = pkv.paged_prefill_attn(q, k, v, cu, pl, sl, sc, ek, ev, pt, c.page_size)
    torch.cuda.synchronize()
    check_close(eo, el, out_ref, lse_ref, "eager chunked")
    k0, v0 = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    kd, vd = k0.clone(), v0.clone()
    out, lse = torch.empty_like(eo), torch.empty_like(el)
    g = _capture(lambda: pkv.paged_prefill_attn(q, k, v, cu, pl, sl, sc, kd, vd, pt, c.page_size,
                                                out=out, lse=lse))

    def reset():
        out.zero_()
        lse.zero_()
        kd.copy_(k0)
        vd.copy_(v0)
    _replays(g, [out, lse, kd, vd], [eo, el, ek, ev], reset)
