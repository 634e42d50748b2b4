"""GPU tests of the per-bucket graph runner (DecodeGraphs): every replay equals the eager
fused call on the same padded inputs bit for bit, with eager work and synchronisation
between replays, and matches the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import make_decode_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_attention_23_amd as pkv  # noqa: E402
from paged_kv_attention_23_amd.graphs import DecodeGraphs  # noqa: E402
from gpu_util import assert_padding_exact, check_close, dev_bf16, dev_i32, host_bits  # noqa: E402


def _case(seed, B, ps=128):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 900, size=B)
    return make_decode_case(name="graphs", seed=seed, H_q=32, H_kv=8, D=128, page_size=ps,
                            num_pages=int(sum(-(-int(n) // ps) for n in lens)) + 4,
                            num_slots=B + 1, max_blocks=8, row_slots=list(range(1, B + 1)),
                            row_lens=lens, layout="shuffled", fill="nan", append_last=True)


@pytest.mark.parametrize("schedule", ["auto", "balanced"])
def test_decode_graphs_buckets(schedule):
    """Batches of 1, 3, 8, 17 and 50 rows through buckets 1..64 of one runner."""
    print(f"graphs {schedule}", flush=True)
    flags = pkv.PKV_F_BALANCED if schedule == "balanced" else 0
    c = _case(81, 50)
    kp_ref, vp_ref = oracle.append_pages(c.k_pool, c.v_pool, c.num_pages, c.page_size, c.page_table,
                                         c.app_batch_idx, c.app_input_pos, c.app_k, c.app_v)
    kd, vd, pt = dev_bf16(c.k_pool), dev_bf16(c.v_pool), dev_i32(c.page_table)
    runner = DecodeGraphs(kd, vd, pt, c.H_q, c.page_size, float(c.scale), max_batch=64,
                          max_kv_len=c.max_blocks * c.page_size, flags=flags)
    kn, vn = np.zeros((c.B, c.H_kv, c.D), np.uint16), np.zeros((c.B, c.H_kv, c.D), np.uint16)
    kn[c.active_rows()], vn[c.active_rows()] = c.app_k, c.app_v
    for n in (1, 3, 8, 17, 50):
        rows = np.arange(n)
        sub = dict(q=c.q[rows], kn=kn[rows], vn=vn[rows], bi=c.batch_idx[rows], kl=c.kv_len[rows])
        out_ref, lse_ref = oracle.decode(sub["q"], kp_ref, vp_ref, c.num_pages, c.page_size,
                                         c.page_table, sub["bi"], np.zeros(n, np.int32), sub["kl"],
                                         c.scale)
        b = runner.bucket_for(n)
        # eager reference on the same padded inputs the graph sees
        pad = b - n
        pq = np.concatenate([sub["q"], np.zeros((pad,) + sub["q"].shape[1:], np.uint16)])
        pk = np.concatenate([sub["kn"], np.zeros((pad,) + sub["kn"].shape[1:], np.uint16)])
        pv = np.concatenate([sub["vn"], np.zeros((pad,) + sub["vn"].shape[1:], np.uint16)])
        pbi = np.concatenate([sub["bi"], np.zeros(pad, np.int32)])
        pkl = np.concatenate([sub["kl"], np.zeros(pad, np.int32)])
        eo, el = pkv.paged_decode_attn_append(
            dev_bf16(pq), dev_bf16(pk), dev_bf16(pv), kd, vd, pt, dev_i32(pbi), dev_i32(pkl),
            page_size=c.page_size, scale=float(c.scale), max_kv_len=c.max_blocks * c.page_size,
            flags=flags)
        torch.cuda.synchronize()
        eo, el = eo[:n].clone(), el[:n].clone()
        for rep in range(3):
            if rep < 2:   # copy-in convenience call
                out, lse = runner(dev_bf16(sub["q"]), dev_bf16(sub["kn"]), dev_bf16(sub["vn"]),
                                  dev_i32(sub["bi"]), dev_i32(sub["kl"]))
            else:         # inputs written in place, then run
                views = runner.inputs(n)
                views["q"].copy_(dev_bf16(sub["q"]))
                views["k_new"].copy_(dev_bf16(sub["kn"]))
                views["v_new"].copy_(dev_bf16(sub["vn"]))
                views["batch_idx"].copy_(dev_i32(sub["bi"]))
                views["kv_len"].copy_(dev_i32(sub["kl"]))
                out, lse = runner.run(n)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eo.view(torch.int16)), (n, rep)
            assert torch.equal(lse, el), (n, rep)
            check_close(out, lse, out_ref, lse_ref, f"graphs n={n} rep={rep}")
            if b > n:  # the bucket's padding rows (slot 0): exactly (+0, -inf)
                assert_padding_exact(runner.out[n:b], runner.lse[n:b], f"graphs pad n={n}")
            _ = (torch.ones(1 << 20, device="cuda") * 2).sum().item()  # eager work between replays
    # the pools hold exactly the oracle's appended tokens (appends are idempotent)
    assert np.array_equal(host_bits(kd), kp_ref) and np.array_equal(host_bits(vd), vp_ref)
