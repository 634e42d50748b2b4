"""GPU checks of the debug validation calls (pkv_validate_decode / _prefill).

Valid workloads give an empty report.  Planted violations (slot, length,
capacity, page id, document bounds) are reported with the right count, first
index, code and block.  These inputs are only ever passed to the validation
kernel, which reads every array within its stated length.
"""
from __future__ import annotations

import numpy as np
import pytest

from workloads import make_case, make_chunked_prefill_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_attention_23_amd as pkv  # noqa: E402
from gpu_util import dev_i32  # noqa: E402

C = pkv._binding._C
EMPTY = [0, -1, 0, -1]


def _decode_report(c, batch_idx=None, kv_len=None, page_table=None):
    bi = c.batch_idx if batch_idx is None else batch_idx
    kl = c.kv_len if kv_len is None else kv_len
    pt = c.page_table if page_table is None else page_table
    rep = pkv.validate_decode(dev_i32(pt), dev_i32(bi), dev_i32(kl), c.page_size, c.num_pages)
    torch.cuda.synchronize()
    return rep.cpu().tolist()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_validate_decode_clean(cfg):
    print(f"validate decode cfg{cfg}", flush=True)
    assert _decode_report(make_case(cfg, fill="zero")) == EMPTY


def test_validate_decode_violations():
    print("validate decode violations", flush=True)
    c = make_case(2, fill="zero")
    cap = c.max_blocks * c.page_size
    bi, kl, pt = c.batch_idx.copy(), c.kv_len.copy(), c.page_table.copy()
    bi[5] = c.num_slots                     # slot past the table
    assert _decode_report(c, batch_idx=bi) == [1, 5, C["PKV_V_SLOT"], -1]
    kl2 = kl.copy()
    kl2[3] = -1
    kl2[6] = cap + 1
    assert _decode_report(c, kv_len=kl2) == [2, 3, C["PKV_V_LEN"], -1]
    kl3 = kl.copy()
    kl3[6] = cap + 1
    assert _decode_report(c, kv_len=kl3) == [1, 6, C["PKV_V_CAPACITY"], -1]
    s = int(c.batch_idx[2])
    blk = int(kl[2] - 1) // c.page_size     # the row's last block
    pt2 = pt.copy()
    pt2[s, blk] = 0                         # the reserved padding page
    assert _decode_report(c, page_table=pt2) == [1, 2, C["PKV_V_PAGE"], blk]
    pt2[s, 0] = c.num_pages                 # past the pool: the first bad block is reported
    assert _decode_report(c, page_table=pt2) == [1, 2, C["PKV_V_PAGE"], 0]
    # padding rows are not checked beyond their slot: kv_len and pages are free
    bi4, kl4 = bi.copy(), kl.copy()
    bi4[5] = 0
    kl4[5] = cap + 100
    assert _decode_report(c, batch_idx=bi4, kv_len=kl4) == EMPTY


def _prefill_report(cu, total, **kw):
    rep = pkv.validate_prefill(dev_i32(np.asarray(cu, np.int32)), total, **kw)
    torch.cuda.synchronize()
    return rep.cpu().tolist()


def test_validate_prefill_bounds():
    print("validate prefill bounds", flush=True)
    pc = make_case(5)
    cu = pc.cu_seqlens
    assert _prefill_report(cu, pc.L) == EMPTY
    bad = cu.copy()
    bad[3] = bad[2] - 1                     # document 2 ends before it starts
    rep = _prefill_report(bad, pc.L)
    assert rep[1] == 2 and rep[2] == C["PKV_V_BOUNDS"] and rep[0] >= 1
    assert _prefill_report(cu, pc.L + 1)[1:3] == [pc.n_docs - 1, C["PKV_V_BOUNDS"]]
    bad = cu.copy()
    bad[0] = 1
    assert _prefill_report(bad, pc.L)[1:3] == [0, C["PKV_V_BOUNDS"]]
    assert _prefill_report([0], 0) == EMPTY            # no documents
    assert _prefill_report([3], 0) == [1, 0, C["PKV_V_BOUNDS"], -1]


def test_validate_prefill_pages():
    print("validate prefill pages", flush=True)
    rng = np.random.default_rng(77)
    cc = make_chunked_prefill_case(name="val", seed=77, prefix_lens=[300, 0, 129, 64],
                                   chunk_lens=[40, 17, 1, 90], H_q=8, H_kv=2, D=128,
                                   page_size=16, fill="zero", rng=rng)
    kw = dict(doc_slots=dev_i32(cc.doc_slots), prefix_lens=dev_i32(cc.prefix_lens),
              page_table=dev_i32(cc.page_table), page_size=cc.page_size,
              num_pages=cc.k_pool.shape[1] // cc.page_size)
    assert _prefill_report(cc.cu_seqlens, cc.L, **kw) == EMPTY
    # slots only (packed_prefill_attn_append): pages are not checked
    assert _prefill_report(cc.cu_seqlens, cc.L, doc_slots=kw["doc_slots"],
                           page_table=kw["page_table"], page_size=cc.page_size,
                           num_pages=kw["num_pages"]) == EMPTY
    pt = cc.page_table.copy()
    s = int(cc.doc_slots[2])
    pt[s, 3] = 0                            # inside document 2's 129-token prefix (blocks 0..8)
    rep = _prefill_report(cc.cu_seqlens, cc.L, **dict(kw, page_table=dev_i32(pt)))
    assert rep == [1, 2, C["PKV_V_PAGE"], 3]
    pl = cc.prefix_lens.copy()
    pl[1] = -4
    assert _prefill_report(cc.cu_seqlens, cc.L, **dict(kw, prefix_lens=dev_i32(pl))) == \
        [1, 1, C["PKV_V_LEN"], -1]
    ds = cc.doc_slots.copy()
    ds[3] = cc.page_table.shape[0]
    assert _prefill_report(cc.cu_seqlens, cc.L, **dict(kw, doc_slots=dev_i32(ds))) == \
        [1, 3, C["PKV_V_SLOT"], -1]
