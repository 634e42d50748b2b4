"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
  decode:  the append of one new token per live sequence and the decode
           over the bucketed B=64 batch (50 live rows, 14 padding rows in
           slot 0, contexts 512..1024, sequential pages, H_q=32, H_kv=8,
           D=128, page_size=128), as one paged_decode_attn_append launch
           (--separate: paged_kv_append, then paged_decode_attn);
  prefill: the scatter of the packed prompts' K/V into shuffled pages and
           the document-causal attention (64 prompts of 64..512 tokens,
           L ~ 18k), as one packed_prefill_attn_append launch (--separate:
           paged_kv_append, then packed_prefill_attn).

Cold data without a flush: like the layers of a model, the benchmark keeps
several independent KV caches (and prefill inputs) and runs the steps back to
back, rotating through them, so every call reads data that was last touched
several calls (>1 GiB of other traffic) earlier and cannot still sit in the
256 MiB Infinity Cache.  The K timed steps are captured into one HIP graph
(as a serving loop captures its decode step per batch bucket, the pages'
CUDA-graph setup) and replayed once, bracketed by one pair of HIP events on
the stream they run on, after a synchronize on both sides; --eager launches
each call from Python instead.  (--flush times each call alone after a 1 GiB
read of another buffer.)

Prints one JSON line.  value = decode KV bytes per step / decode step time
(GB/s); the prefill part is reported under "prefill".
"""
from __future__ import annotations

import argparse
import hashlib
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
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "paged_kv_attention_23_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8,
                    help="independent KV caches rotated through by the decode steps")
    ap.add_argument("--prefill-layers", type=int, default=4,
                    help="independent prefill input sets rotated through")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="decode split count: 0 = automatic, 1 = single pass, >1 = per-row splits")
    ap.add_argument("--flags", type=int, default=0,
                    help="decode PKV_F_* flags (4 = balanced schedule, with --num-splits 0)")
    ap.add_argument("--separate", action="store_true",
                    help="steps as paged_kv_append + attention instead of the fused entry points")
    ap.add_argument("--eager", action="store_true",
                    help="launch every timed call from Python instead of replaying a HIP graph")
    ap.add_argument("--flush", action="store_true",
                    help="time each call alone after a 1 GiB read of another buffer")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill (paged prefix) measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size: the reference that scales the HBM byte counters."""
    import torch

    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4}), flush=True)


def decode_kernels(S: int, W: int) -> str:
    """The kernels one paged_decode_attn call launches for this schedule."""
    if W > 1:
        return "decode_balanced_kernel + merge_balanced_kernel"
    if S > 1:
        return "decode_rows_kernel + merge_rows_kernel"
    return "decode_rows_kernel"


def measured_traffic(kernel: str, source: str):
    """HBM bytes per launch from the committed counter runs, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)[kernel]
        with open(os.path.join(CSRC, source), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    return int(t["traffic_bytes"]) if t.get("source_sha256") == sha else None


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_23_amd as pkv
    from workloads import f32_to_bf16_bits, make_case

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import dev_bf16, dev_i32

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------- decode inputs (bucketed B=64), one KV cache per layer
    c = make_case(3, fill="zero")
    rng = np.random.default_rng(9303)
    act = c.active_rows()
    app_bi = c.batch_idx[act].astype(np.int32)
    app_pos = (c.kv_len[act] - 1).astype(np.int32)         # the step's new token is key n-1
    app_k = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
    app_v = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
    d_q = dev_bf16(c.q)
    k0, v0 = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
    NL = max(1, args.layers)
    d_k = [k0] + [k0.clone() for _ in range(NL - 1)]
    d_v = [v0] + [v0.clone() for _ in range(NL - 1)]
    d_pt, d_bi, d_kl = dev_i32(c.page_table), dev_i32(c.batch_idx), dev_i32(c.kv_len)
    d_abi, d_apos = dev_i32(app_bi), dev_i32(app_pos)
    d_ak, d_av = dev_bf16(app_k), dev_bf16(app_v)
    row_k = np.zeros((c.B, c.H_kv, c.D), np.uint16)   # the same tokens, indexed by row
    row_v = np.zeros_like(row_k)
    row_k[act], row_v[act] = app_k, app_v
    d_rk, d_rv = dev_bf16(row_k), dev_bf16(row_v)
    max_kv = int(c.kv_len.max())
    balanced = bool(args.flags & pkv.PKV_F_BALANCED)
    S = args.num_splits or (0 if balanced else pkv.paged_decode_num_splits(c.B, c.H_kv, max_kv))
    W = pkv.paged_decode_balanced_parts(c.B, c.H_kv, max_kv) if balanced else 0
    ws_bytes = pkv.paged_decode_workspace_size(c.B, c.H_q, c.H_kv, c.D, S, args.flags)
    d_ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    d_out = torch.empty((c.B, c.H_q, c.D), dtype=torch.bfloat16, device=dev)
    d_lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device=dev)
    kv_bytes = c.kv_bytes()

    def decode_only(i):
        pkv.paged_decode_attn(d_q, d_k[i % NL], d_v[i % NL], d_pt, d_bi, d_kl,
                              page_size=c.page_size, scale=float(c.scale), max_kv_len=max_kv,
                              num_splits=S, flags=args.flags, workspace=d_ws, out=d_out, lse=d_lse)

    def decode_step_separate(i):
        pkv.paged_kv_append(d_k[i % NL], d_v[i % NL], d_pt, d_abi, d_apos, d_ak, d_av,
                            page_size=c.page_size)
        decode_only(i)

    def decode_step_fused(i):
        pkv.paged_decode_attn_append(d_q, d_rk, d_rv, d_k[i % NL], d_v[i % NL], d_pt, d_bi, d_kl,
                                     page_size=c.page_size, scale=float(c.scale),
                                     max_kv_len=max_kv, num_splits=S, flags=args.flags,
                                     workspace=d_ws, out=d_out, lse=d_lse)

    decode_step = decode_step_separate if args.separate else decode_step_fused

    # ---------------- prefill inputs (packed 64 prompts), one input set per layer
    prefill = None
    if not args.no_prefill:
        pc = make_case(5)
        NP = max(1, args.prefill_layers)
        p_q = [dev_bf16(pc.q)]
        p_k = [dev_bf16(pc.k)]
        p_v = [dev_bf16(pc.v)]
        for _ in range(NP - 1):
            p_q.append(p_q[0].clone())
            p_k.append(p_k[0].clone())
            p_v.append(p_v[0].clone())
        p_cu = dev_i32(pc.cu_seqlens)
        p_pt, p_bi, p_ip = dev_i32(pc.page_table), dev_i32(pc.batch_idx), dev_i32(pc.input_pos)
        shape = (pc.H_kv, pc.num_pages * pc.page_size, pc.D)
        p_kpool = [torch.zeros(shape, dtype=torch.bfloat16, device=dev) for _ in range(NP)]
        p_vpool = [torch.zeros(shape, dtype=torch.bfloat16, device=dev) for _ in range(NP)]
        p_out = torch.empty((pc.L, pc.H_q, pc.D), dtype=torch.bfloat16, device=dev)
        p_lse = torch.empty((pc.L, pc.H_q), dtype=torch.float32, device=dev)

        def prefill_attn(i):
            j = i % NP
            pkv.packed_prefill_attn(p_q[j], p_k[j], p_v[j], p_cu, scale=float(pc.scale),
                                    out=p_out, lse=p_lse)

        p_slots = dev_i32(np.arange(1, pc.n_docs + 1, dtype=np.int32))

        def prefill_step_separate(i):
            j = i % NP
            pkv.paged_kv_append(p_kpool[j], p_vpool[j], p_pt, p_bi, p_ip, p_k[j], p_v[j],
                                page_size=pc.page_size)
            prefill_attn(i)

        def prefill_step_fused(i):
            j = i % NP
            pkv.packed_prefill_attn_append(p_q[j], p_k[j], p_v[j], p_cu, float(pc.scale),
                                           p_kpool[j], p_vpool[j], p_pt, p_slots, pc.page_size,
                                           out=p_out, lse=p_lse)

        prefill = dict(case=pc, layers=NP, attn=prefill_attn,
                       step=prefill_step_separate if args.separate else prefill_step_fused,
                       alt=prefill_step_fused if args.separate else prefill_step_separate)

    # ---------------- chunked prefill over a paged prefix (64 sequences), one pool set per layer
    chunked = None
    if not args.no_chunked:
        from workloads import make_chunked_prefill_case
        crng = np.random.default_rng(9305)
        cc = make_chunked_prefill_case(name="chunked", seed=9305,
                                       prefix_lens=crng.integers(256, 1025, 64),
                                       chunk_lens=crng.integers(64, 257, 64), H_q=32, H_kv=8,
                                       D=128, page_size=128, fill="empty", rng=crng)
        NC = max(1, args.prefill_layers)
        c_kp = [dev_bf16(cc.k_pool) for _ in range(NC)]
        c_vp = [dev_bf16(cc.v_pool) for _ in range(NC)]
        c_q, c_k, c_v = dev_bf16(cc.q), dev_bf16(cc.k), dev_bf16(cc.v)
        c_cu, c_pl = dev_i32(cc.cu_seqlens), dev_i32(cc.prefix_lens)
        c_sl, c_pt = dev_i32(cc.doc_slots), dev_i32(cc.page_table)
        c_out = torch.empty((cc.L, cc.H_q, cc.D), dtype=torch.bfloat16, device=dev)
        c_lse = torch.empty((cc.L, cc.H_q), dtype=torch.float32, device=dev)

        def chunked_step(i):
            j = i % NC
            pkv.paged_prefill_attn(c_q, c_k, c_v, c_cu, c_pl, c_sl, float(cc.scale), c_kp[j],
                                   c_vp[j], c_pt, cc.page_size, out=c_out, lse=c_lse)

        chunked = dict(case=cc, step=chunked_step, layers=NC)

    flush_buf = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) \
        if args.flush else None
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn, n, replays=None):
        """Device time (ms) of n steps fn(0..n-1).  With a list `replays`, the captured
        graph is replayed 5 more times and each replay's time (ms) is appended to it."""
        if args.flush:  # each call alone after a 1 GiB read (clean eviction)
            total = 0.0
            for i in range(n):
                torch.sum(flush_buf, dim=0, out=flush_sink)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn(i)
                e1.record(stream)
                e1.synchronize()
                total += e0.elapsed_time(e1)
            return total
        if args.eager:
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                fn(i)
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1)
        # The n steps are captured once into a HIP graph (as a serving loop
        # captures its decode step) and replayed: the timed region holds the
        # GPU work only, not Python's per-call launch cost.  All buffers are
        # allocated before the capture; no memset is recorded.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        graph.replay()                      # first replay uploads the graph
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        e1.synchronize()
        total = e0.elapsed_time(e1)
        if replays is not None:
            for _ in range(5):
                e0.record(stream)
                graph.replay()
                e1.record(stream)
                e1.synchronize()
                replays.append(e0.elapsed_time(e1))
        return total

    # ---------------- warmup
    for i in range(args.warmup):
        decode_step(i)
        if prefill:
            prefill["step"](i)
        if chunked:
            chunked["step"](i)
    torch.cuda.synchronize()

    # ---------------- timed steps
    K = args.steps
    t0 = time.perf_counter()
    dec_total = timed(decode_step, K)
    pre_total = timed(prefill["step"], K) if prefill else 0.0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the dominant kernels alone (roofline): decode attention, prefill attention
    dk_reps, pa_reps = [], []
    dk_total = timed(decode_only, K, dk_reps)
    alt_total = timed(decode_step_fused if args.separate else decode_step_separate, K)
    pa_total = timed(prefill["attn"], K, pa_reps) if prefill else 0.0
    palt_total = timed(prefill["alt"], K) if prefill else 0.0
    ch_total = timed(chunked["step"], K) if chunked else 0.0
    # warm, for context: every call reads the same cache (input set), which
    # then sits in the 256 MiB Infinity Cache; not an HBM figure
    dw_total = timed(lambda i: decode_only(0), K)
    pw_total = timed(lambda i: prefill["attn"](0), K) if prefill else 0.0

    dec_ms, dk_ms = dec_total / K, dk_total / K
    value = kv_bytes / (dec_ms * 1e-3) / 1e9
    achieved = kv_bytes / (dk_ms * 1e-3) / 1e9
    cache = ("flushed: 1 GiB read before each call" if args.flush else
             f"cold: {NL} KV caches (one per layer) read round-robin, "
             f"{(NL - 1) * kv_bytes / 1e9:.2f} GB of other KV between reuses")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round((dec_total + pre_total) / K, 5),
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
            "decode_step_ms": round(dec_ms, 5),
            "decode_step": ("paged_kv_append + paged_decode_attn" if args.separate else
                            "paged_decode_attn_append (append and decode fused in one launch)"),
            ("fused_step_ms" if args.separate else "separate_step_ms"): round(alt_total / K, 5),
            "schedule": (f"balanced: {W} workgroups per KV head" if balanced else
                         f"per-row: {S} split(s) per row"),
            "launch": "eager stream launches" if (args.eager or args.flush) else
                      f"one HIP graph of the {K} timed steps, replayed once",
            "flags": int(args.flags),
            "cache": cache,
            "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": decode_kernels(S, W) + " (one paged_decode_attn call)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode", "decode.hip"),
            "avg_call_us": round(dk_ms * 1e3, 3),
            "algorithmic_bytes_per_call": int(kv_bytes),
            "replays_us": ({"median": round(float(np.median(dk_reps)) / K * 1e3, 3),
                            "best": round(min(dk_reps) / K * 1e3, 3), "n": len(dk_reps)}
                           if dk_reps else None),
            "warm_call_us": round(dw_total / K * 1e3, 3),
            "warm_gbs": round(kv_bytes / (dw_total / K * 1e-3) / 1e9, 2),
            "warm": "the same KV cache every call (Infinity-Cache resident), context only",
        },
        "wall_s_timed_region": round(wall, 3),
    }
    if prefill:
        pc = prefill["case"]
        flops = pc.flops()
        pa_ms, pre_ms = pa_total / K, pre_total / K
        tflops = flops / (pa_ms * 1e-3) / 1e12
        p_bytes = (pc.L * (pc.H_q + 2 * pc.H_kv) * pc.D * 2 + pc.L * pc.H_q * pc.D * 2
                   + pc.L * pc.H_q * 4)
        out["prefill"] = {
            "workload": "packed prefill, 64 prompts U[64,512] (L=%d), H_q=32 H_kv=8 D=128, "
                        "document-causal, + append into shuffled 128-token pages" % pc.L,
            "flops_per_call": int(flops),
            "attn_us": round(pa_ms * 1e3, 3),
            "step_us": round(pre_ms * 1e3, 3),
            "step": ("paged_kv_append + packed_prefill_attn" if args.separate else
                     "packed_prefill_attn_append (scatter and attention fused in one launch)"),
            ("fused_step_us" if args.separate else "separate_step_us"): round(palt_total / K * 1e3, 3),
            "tflops": round(tflops, 2),
            "roofline": {
                "bound": "mfma",
                "kernel": "prefill_kernel (packed_prefill_attn)",
                "achieved": round(tflops, 2),
                "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("prefill", "prefill.hip"),
                # the same call against HBM: q, k, v read once, out and lse written once
                "compulsory_bytes": int(p_bytes),
                "hbm_achieved_gbs": round(p_bytes / (pa_ms * 1e-3) / 1e9, 2),
                "hbm_frac": round(p_bytes / (pa_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "replays_us": ({"median": round(float(np.median(pa_reps)) / K * 1e3, 3),
                                "best": round(min(pa_reps) / K * 1e3, 3), "n": len(pa_reps)}
                               if pa_reps else None),
                "warm_attn_us": round(pw_total / K * 1e3, 3),
                "warm_tflops": round(flops / (pw_total / K * 1e-3) / 1e12, 2),
                "warm": "the same input set every call (Infinity-Cache resident), context only",
            },
            "cache": f"cold: {prefill['layers']} input sets read round-robin",
        }
    if chunked:
        cc = chunked["case"]
        ch_ms = ch_total / K
        kv_prefix = int(cc.prefix_lens.astype(np.int64).sum()) * cc.H_kv * cc.D * 2 * 2
        out["chunked_prefill"] = {
            "workload": "chunked prefill over a paged prefix: 64 sequences with U[256,1024] "
                        "cached tokens, chunks U[64,256] (L=%d), H_q=32 H_kv=8 D=128, "
                        "page_size=128 shuffled; chunk K/V written into the pages" % cc.L,
            "call": "paged_prefill_attn",
            "us": round(ch_ms * 1e3, 3),
            "flops_per_call": int(cc.flops()),
            "tflops": round(cc.flops() / (ch_ms * 1e-3) / 1e12, 2),
            "prefix_kv_bytes": kv_prefix,
            "cache": f"cold: {chunked['layers']} pool sets read round-robin",
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
        "sample": f"the full B=64 decode step (50 live rows, {kv_bytes / 1e6:.1f} MB of KV), "
                  f"repeated {reps}x in {t_total:.1f} s",
    }


if __name__ == "__main__":
    main()
