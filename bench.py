"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
  decode: paged_kv_append of one new token per live sequence, then
          paged_decode_attn over the bucketed B=64 batch (50 live rows,
          14 padding rows in slot 0, contexts 512..1024, sequential pages,
          H_q=32, H_kv=8, D=128, page_size=128);
  prefill: paged_kv_append of the packed prompts' K/V into shuffled pages,
          then packed_prefill_attn (64 prompts of 64..512 tokens, L ~ 18k).
Every timed step starts after a cache-flush kernel reads 1 GiB (four times
the 256 MiB Infinity Cache), so the KV bytes come from HBM.  Device time of each
part is taken with HIP events on the stream the kernels run on and summed
over the K timed steps; the flush is outside the events.

Prints one JSON line.  value = decode KV bytes per step / decode device time
(GB/s); the prefill part is reported under "prefill".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, published
METRIC = "paged decode KV-read GB/s (% of HBM peak) at B=64; prefill TFLOP/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--num-splits", type=int, default=0, help="decode split count (0 = auto)")
    ap.add_argument("--flags", type=int, default=0, help="decode PKV_F_* flags")
    ap.add_argument("--no-flush", action="store_true", help="warm-cache timing (reported as such)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget for the CPU oracle baseline (0 = skip)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_23_amd as pkv
    from workloads import make_case

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import dev_bf16, dev_i32

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------- decode inputs (bucketed B=64)
    c = make_case(3, fill="zero")
    rng = np.random.default_rng(9303)
    act = c.active_rows()
    app_bi = c.batch_idx[act].astype(np.int32)
    app_pos = (c.kv_len[act] - 1).astype(np.int32)         # the step's new token is key n-1
    from workloads import f32_to_bf16_bits
    app_k = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
    app_v = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
    d_q, d_k, d_v = dev_bf16(c.q), dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    d_pt, d_bi, d_kl = dev_i32(c.page_table), dev_i32(c.batch_idx), dev_i32(c.kv_len)
    d_abi, d_apos = dev_i32(app_bi), dev_i32(app_pos)
    d_ak, d_av = dev_bf16(app_k), dev_bf16(app_v)
    max_kv = int(c.kv_len.max())
    S = args.num_splits or pkv.paged_decode_num_splits(c.B, c.H_kv, max_kv)
    ws_bytes = pkv.paged_decode_workspace_size(c.B, c.H_q, c.D, S)
    d_ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    d_out = torch.empty((c.B, c.H_q, c.D), dtype=torch.bfloat16, device=dev)
    d_lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device=dev)
    kv_bytes = c.kv_bytes()

    def decode_step():
        pkv.paged_kv_append(d_k, d_v, d_pt, d_abi, d_apos, d_ak, d_av, page_size=c.page_size)
        pkv.paged_decode_attn(d_q, d_k, d_v, d_pt, d_bi, d_kl, page_size=c.page_size,
                              scale=float(c.scale), max_kv_len=max_kv, num_splits=S,
                              flags=args.flags, workspace=d_ws, out=d_out, lse=d_lse)

    def decode_only():
        pkv.paged_decode_attn(d_q, d_k, d_v, d_pt, d_bi, d_kl, page_size=c.page_size,
                              scale=float(c.scale), max_kv_len=max_kv, num_splits=S,
                              flags=args.flags, workspace=d_ws, out=d_out, lse=d_lse)

    # Cache flush: read 1 GiB (4x the Infinity Cache) into a scalar.  A read
    # leaves only clean lines behind, so the timed kernel does not pay for
    # the flush's own write-backs.
    flush_buf = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, out=flush_sink)

    def timed(fn, n):
        """Sum of device times of n calls of fn, each after a flush."""
        total = 0.0
        times = []
        for _ in range(n):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            times.append(ms)
            total += ms
        return total, times

    # ---------------- prefill inputs (packed 64 prompts)
    prefill = None
    if not args.no_prefill:
        pc = make_case(5)
        p_q, p_k, p_v = dev_bf16(pc.q), dev_bf16(pc.k), dev_bf16(pc.v)
        p_cu = dev_i32(pc.cu_seqlens)
        p_pt, p_bi, p_ip = dev_i32(pc.page_table), dev_i32(pc.batch_idx), dev_i32(pc.input_pos)
        p_kpool = torch.zeros((pc.H_kv, pc.num_pages * pc.page_size, pc.D), dtype=torch.bfloat16,
                              device=dev)
        p_vpool = torch.zeros_like(p_kpool)
        p_out = torch.empty((pc.L, pc.H_q, pc.D), dtype=torch.bfloat16, device=dev)
        p_lse = torch.empty((pc.L, pc.H_q), dtype=torch.float32, device=dev)

        def prefill_attn():
            pkv.packed_prefill_attn(p_q, p_k, p_v, p_cu, scale=float(pc.scale), out=p_out, lse=p_lse)

        def prefill_step():
            pkv.paged_kv_append(p_kpool, p_vpool, p_pt, p_bi, p_ip, p_k, p_v, page_size=pc.page_size)
            prefill_attn()

        try:
            prefill_step()
            torch.cuda.synchronize()
            prefill = dict(case=pc, step=prefill_step, attn=prefill_attn)
        except RuntimeError as e:  # kernel not available in this build
            print(f"prefill skipped: {e}", file=sys.stderr)

    # ---------------- warmup
    for _ in range(args.warmup):
        decode_step()
        if prefill:
            prefill["step"]()
    torch.cuda.synchronize()

    # ---------------- timed steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec_total, dec_times = timed(decode_step, args.steps)
    pre_total, pre_times = (timed(prefill["step"], args.steps) if prefill else (0.0, []))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # decode kernel alone (the dominant kernel for the roofline) and the attention part of prefill
    dk_total, dk_times = timed(decode_only, args.steps)
    pa_total, pa_times = (timed(prefill["attn"], args.steps) if prefill else (0.0, []))

    dec_ms = dec_total / args.steps
    dk_ms = dk_total / args.steps
    value = kv_bytes / (dec_ms * 1e-3) / 1e9
    achieved = kv_bytes / (dk_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((dec_total + pre_total) / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "bucketed decode B=64 (50 live rows + 14 slot-0 padding rows), "
                        "H_q=32 H_kv=8 D=128 page_size=128, contexts U[512,1024], "
                        "sequential pages, + append of 1 token per live row",
            "global_batch": int(c.B),
            "kv_bytes_per_step": int(kv_bytes),
            "num_splits": int(S),
            "flags": int(args.flags),
            "cache": "warm" if args.no_flush else "flushed (1 GiB read before each step)",
            "decode_step_ms_median": round(float(np.median(dec_times)), 5),
            "decode_step_ms_best": round(float(np.min(dec_times)), 5),
            "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_attn (decode_kernel%s)" % (" + merge_kernel" if S > 1 else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_call_us": round(dk_ms * 1e3, 3),
            "algorithmic_bytes_per_call": int(kv_bytes),
        },
        "wall_s_timed_region": round(wall, 3),
    }
    if prefill:
        pc = prefill["case"]
        flops = pc.flops()
        pa_ms = pa_total / args.steps
        pre_ms = pre_total / args.steps
        out["prefill"] = {
            "workload": "packed prefill, 64 prompts U[64,512] (L=%d), H_q=32 H_kv=8 D=128, "
                        "document-causal, + append into shuffled 128-token pages" % pc.L,
            "flops_per_call": int(flops),
            "attn_ms": round(pa_ms, 5),
            "step_ms": round(pre_ms, 5),
            "tflops": round(flops / (pa_ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flops / (pa_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(c, kv_bytes, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline(c, kv_bytes, budget_s):
    """The float64 oracle timed on the host cores over the same decode workload."""
    import oracle

    B = c.B
    lo = np.zeros(B, np.int32)
    reps, t_total = 0, 0.0
    while t_total < budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.decode(c.q, c.k_pool, c.v_pool, c.num_pages, c.page_size, c.page_table,
                      c.batch_idx, lo, c.kv_len, c.scale)
        t_total += time.perf_counter() - t0
        reps += 1
    return {
        "value": round(kv_bytes * reps / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"the full B=64 decode step (50 live rows), repeated {reps}x "
                  f"in {t_total:.1f} s",
    }


if __name__ == "__main__":
    main()
