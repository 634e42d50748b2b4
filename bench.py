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

Beside the headline step, every named workload gets its own entry under
"configs" (tiny decode; B=8 decode + append; the B=64 bucket, with the
contiguous-page path against the page-table walk; B=256 through the
automatic plan, split-K + merge and the balanced schedule; packed prefill),
each timed cold and warm, plus the float64 oracle timed on the host cores
(all threads, and one thread for the decode workloads).  "ceilings" holds
what plain kernels of the same shapes reach on this GPU: a streaming read,
a streaming read with the decode launch shape, a dense bf16 matrix-core
loop and a library bf16 GEMM.

Cold data without a flush: like the layers of a model, the benchmark keeps
several independent KV caches (and prefill inputs) and runs the steps back to
back, rotating through them, so every call reads data that was last touched
more than 512 MB of other traffic earlier and cannot still sit in the
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
import ctypes
import hashlib
import json
import math
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
CEIL_LIB = os.path.join(ROOT, "paged_kv_attention_23_amd", "measure", "libpkvceil.so")
COLD_DISTANCE = 600e6          # bytes of other traffic between two reads of the same data


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8,
                    help="independent KV caches rotated through by the headline decode steps")
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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload entries (configs 1, 2 and 4; the B=64 path A/B)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the reachable-rate probes")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None,
                    help="time only the decode or only the prefill attention call (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="budget per oracle measurement on the host (0 = skip)")
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Timer:
    """Device time of fn(0..n-1) on the current stream (graph-replayed unless eager/flush)."""

    def __init__(self, torch, stream, args, dev):
        self.torch, self.stream, self.args = torch, stream, args
        self.flush_buf = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) \
            if args.flush else None
        self.flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def events(self):
        t = self.torch
        return t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)

    def __call__(self, fn, n, replays=None):
        """Total ms of n steps.  With a list `replays`, the captured graph is replayed 5
        more times and each replay's total (ms) is appended to it."""
        torch, stream, args = self.torch, self.stream, self.args
        if args.flush:  # each call alone after a 1 GiB read (clean eviction)
            total = 0.0
            for i in range(n):
                torch.sum(self.flush_buf, dim=0, out=self.flush_sink)
                e0, e1 = self.events()
                e0.record(stream)
                fn(i)
                e1.record(stream)
                e1.synchronize()
                total += e0.elapsed_time(e1)
            return total
        if args.eager:
            torch.cuda.synchronize()
            e0, e1 = self.events()
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
        e0, e1 = self.events()
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
        del graph
        return total


def layers_for(nbytes: float, cap: int = 64) -> int:
    """Independent copies needed so that COLD_DISTANCE bytes pass between two reuses."""
    return int(min(cap, max(2, math.ceil(COLD_DISTANCE / max(nbytes, 1.0)) + 1)))


class DecodeBench:
    """One decode workload on the GPU: NL independent pool copies, rotated through."""

    def __init__(self, torch, pkv, case, dev, layers=None):
        from gpu_util import dev_bf16, dev_i32
        self.torch, self.pkv, self.c = torch, pkv, case
        c = case
        self.kv_bytes = c.kv_bytes()
        self.NL = layers if layers else layers_for(self.kv_bytes)
        k0, v0 = dev_bf16(c.k_pool), dev_bf16(c.v_pool)
        self.k = [k0] + [k0.clone() for _ in range(self.NL - 1)]
        self.v = [v0] + [v0.clone() for _ in range(self.NL - 1)]
        self.q = dev_bf16(c.q)
        self.pt, self.bi, self.kl = dev_i32(c.page_table), dev_i32(c.batch_idx), dev_i32(c.kv_len)
        self.max_kv = int(c.kv_len.max())
        self.out = torch.empty((c.B, c.H_q, c.D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device=dev)
        self.ws = {}
        self.dev = dev
        act = c.active_rows()
        self.act = act
        rng = np.random.default_rng(9303 + c.seed)
        from workloads import f32_to_bf16_bits
        row_k = np.zeros((c.B, c.H_kv, c.D), np.uint16)
        row_v = np.zeros_like(row_k)
        row_k[act] = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
        row_v[act] = f32_to_bf16_bits(rng.standard_normal((len(act), c.H_kv, c.D), dtype=np.float32))
        self.rk, self.rv = dev_bf16(row_k), dev_bf16(row_v)

    def workspace(self, S, flags):
        key = (S, flags)
        if key not in self.ws:
            c = self.c
            n = self.pkv.paged_decode_workspace_size(c.B, c.H_q, c.H_kv, c.D, S, flags)
            self.ws[key] = self.torch.empty(max(n, 16), dtype=self.torch.uint8, device=self.dev)
        return self.ws[key]

    def call(self, S=0, flags=0, rotate=True):
        c, pkv = self.c, self.pkv
        ws = self.workspace(S, flags)

        def fn(i):
            j = i % self.NL if rotate else 0
            pkv.paged_decode_attn(self.q, self.k[j], self.v[j], self.pt, self.bi, self.kl,
                                  page_size=c.page_size, scale=float(c.scale),
                                  max_kv_len=self.max_kv, num_splits=S, flags=flags,
                                  workspace=ws, out=self.out, lse=self.lse)
        return fn

    def fused(self, S=0, flags=0):
        c, pkv = self.c, self.pkv
        ws = self.workspace(S, flags)

        def fn(i):
            j = i % self.NL
            pkv.paged_decode_attn_append(self.q, self.rk, self.rv, self.k[j], self.v[j], self.pt,
                                         self.bi, self.kl, page_size=c.page_size,
                                         scale=float(c.scale), max_kv_len=self.max_kv,
                                         num_splits=S, flags=flags, workspace=ws, out=self.out,
                                         lse=self.lse)
        return fn

    def free(self):
        self.k = self.v = None
        self.ws = {}


def plan_name(pkv, c, S, flags, max_kv):
    if flags & pkv.PKV_F_BALANCED or (S == 0 and pkv.paged_decode_auto_balanced(c.B, c.H_kv, max_kv)):
        W = pkv.paged_decode_balanced_parts(c.B, c.H_kv, max_kv)
        return f"balanced: {W} workgroups per KV head", 1, W
    s = S or pkv.paged_decode_num_splits(c.B, c.H_kv, max_kv)
    return f"per-row: {s} split(s) per row", s, 0


def time_decode(timer, db, K, S=0, flags=0, warm=True, replays=False):
    """Cold (rotating copies) and warm (one copy) per-call times of one decode plan."""
    reps = [] if replays else None
    cold_ms = timer(db.call(S, flags), K, reps) / K
    r = {"cold_us": round(cold_ms * 1e3, 3),
         "gbs": round(db.kv_bytes / (cold_ms * 1e-3) / 1e9, 2),
         "frac_of_hbm_peak": round(db.kv_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if reps:
        r["replays_us"] = {"median": round(float(np.median(reps)) / K * 1e3, 3),
                           "best": round(min(reps) / K * 1e3, 3), "n": len(reps)}
    if warm:
        warm_ms = timer(db.call(S, flags, rotate=False), K) / K
        r["warm_us"] = round(warm_ms * 1e3, 3)
    return r, cold_ms


def oracle_rate(fn, units, budget_s, threads=None):
    """Repeat the oracle call until budget_s has passed (at least once); units per second."""
    import oracle
    prev = oracle.num_threads()
    if threads:
        oracle.set_threads(threads)
    try:
        used = oracle.num_threads()
        reps, total = 0, 0.0
        while total < budget_s or reps == 0:
            t0 = time.perf_counter()
            fn()
            total += time.perf_counter() - t0
            reps += 1
    finally:
        oracle.set_threads(prev)
    return units * reps / total, used, reps, total


def cpu_decode_baseline(c, budget_s, single=True):
    import oracle
    lo = np.zeros(c.B, np.int32)
    kvb = c.kv_bytes()

    def fn():
        oracle.decode(c.q, c.k_pool, c.v_pool, c.num_pages, c.page_size, c.page_table,
                      c.batch_idx, lo, c.kv_len, c.scale)
    gbs, cores, reps, t = oracle_rate(fn, kvb / 1e9, budget_s)
    r = {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
         "sample": f"the whole decode call ({kvb / 1e6:.1f} MB of KV), {reps}x in {t:.2f} s"}
    if single:
        g1, _, reps1, t1 = oracle_rate(fn, kvb / 1e9, budget_s, threads=1)
        r["one_thread"] = {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"{reps1}x in {t1:.2f} s"}
    return r


def cpu_prefill_baseline(pc, budget_s):
    import oracle
    flops = pc.flops()
    docs = min(pc.n_docs, 16)  # a bounded sample: the first documents of the packing
    cu = pc.cu_seqlens[:docs + 1].astype(np.int32)
    end = int(cu[-1])
    n = np.diff(cu.astype(np.int64))
    sflops = 4 * pc.D * pc.H_q * int((n * (n + 1) // 2).sum())

    def fn():
        oracle.prefill(pc.q[:end], pc.k[:end], pc.v[:end], cu, pc.scale)
    gf, cores, reps, t = oracle_rate(fn, sflops / 1e9, budget_s)
    return {"value": round(gf / 1e3, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {docs} of the {pc.n_docs} documents ({end} rows, "
                      f"{sflops / 1e9:.2f} of the call's {flops / 1e9:.1f} GFLOP), "
                      f"{reps}x in {t:.2f} s"}


def load_ceil():
    if not os.path.exists(CEIL_LIB):
        return None
    L = ctypes.CDLL(CEIL_LIB)
    L.ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    L.ceil_stream_units.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.ceil_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.ceil_prefill_shape.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    P, I, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
    L.ceil_paged_units.argtypes = [P, P, ctypes.c_uint64, U, I, P, I, I, I, I, P, P, I, P, P]
    return L


def ceilings(torch, timer, dev, db3, K, prefill=None):
    """What plain kernels of the attention kernels' shapes reach on this GPU."""
    L = load_ceil()
    out = {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def st():  # the stream current at call time (a capture stream inside a graph capture)
        return torch.cuda.current_stream().cuda_stream

    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    if L is not None:
        big = torch.ones(2 * 1024 ** 3 // 4, dtype=torch.float32, device=dev)
        nb = big.numel() * 4
        best = None
        for grid in (cus * 4, cus * 8, cus * 16):
            def fn(i, grid=grid):
                assert L.ceil_stream_read(big.data_ptr(), nb, grid, sink.data_ptr(), st()) == 0
            ms = timer(fn, 4) / 4
            gbs = nb / (ms * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, grid, ms)
        out["stream_read"] = {"gbs": round(best[0], 1), "bytes": nb, "grid": best[1],
                              "us": round(best[2] * 1e3, 2),
                              "frac_of_hbm_peak": round(best[0] / HBM_PEAK_GBS, 4),
                              "kernel": "grid-strided non-temporal 16-byte loads, 256 threads"}
        # the same bytes as one B=64 decode call, in windows of a 2 GiB buffer read in turn
        w = (db3.kv_bytes + 255) // 256 * 256
        nwin = nb // w

        def fw(i):
            off = (i % nwin) * w
            assert L.ceil_stream_read(big.data_ptr() + off, w, best[1], sink.data_ptr(), st()) == 0
        ms = timer(fw, K) / K
        out["stream_read_decode_bytes"] = {
            "us": round(ms * 1e3, 3), "bytes": int(w), "gbs": round(w / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(w / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "one grid-strided read of as many bytes as the B=64 decode call, cold"}
        del big
        # the decode launch shape, streaming only: one unit per (row, KV head), its K and V
        # rows a contiguous run (the workload's sequential pages), 4 waves, one 32-key tile
        # in flight per wave; padding rows have no keys
        c = db3.c
        if c.contiguous:
            units = np.zeros((c.B * c.H_kv, 2), np.int32)
            plane_rows = c.num_pages * c.page_size
            for r in range(c.B):
                s, n = int(c.batch_idx[r]), int(c.kv_len[r])
                if s == 0 or n <= 0:
                    continue
                row0 = int(c.page_table[s, 0]) * c.page_size
                assert 0 <= row0 and row0 + n <= plane_rows
                units[r * c.H_kv:(r + 1) * c.H_kv] = (row0, n)
            du = torch.from_numpy(units.reshape(-1)).to(dev)
            plane_bytes = plane_rows * c.D * 2

            def fu(i):
                j = i % db3.NL
                assert L.ceil_stream_units(db3.k[j].data_ptr(), db3.v[j].data_ptr(), plane_bytes,
                                           c.H_kv, du.data_ptr(), c.B * c.H_kv, sink.data_ptr(),
                                           st()) == 0
            ms = timer(fu, K) / K
            out["decode_shape_stream"] = {
                "us": round(ms * 1e3, 3), "bytes": int(db3.kv_bytes),
                "gbs": round(db3.kv_bytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(db3.kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "the B=64 decode's launch shape and bytes with no arithmetic: "
                        f"{c.B * c.H_kv} workgroups of 4 waves (one per row and KV head), cold"}
        # the same launch shape reaching its keys the way paged decode does: slot and length,
        # then the page-id window, then K/V through the page ids (the dependent-load chain
        # without any arithmetic)
        if c.max_blocks <= 64 and c.D == 128:
            plane_bytes = c.num_pages * c.page_size * c.D * 2
            shift = int(c.page_size).bit_length() - 1

            def fp(i):
                j = i % db3.NL
                assert L.ceil_paged_units(db3.k[j].data_ptr(), db3.v[j].data_ptr(), plane_bytes,
                                          c.D * 2, c.H_kv, db3.pt.data_ptr(), c.max_blocks, shift,
                                          c.num_pages, c.num_slots, db3.bi.data_ptr(),
                                          db3.kl.data_ptr(), c.B, sink.data_ptr(), st()) == 0
            ms = timer(fp, K) / K
            out["decode_shape_paged"] = {
                "us": round(ms * 1e3, 3), "bytes": int(db3.kv_bytes),
                "gbs": round(db3.kv_bytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(db3.kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "decode_shape_stream with the paged lookups: batch_idx and kv_len, one "
                        "page-id window per unit, K/V rows through the page ids; no arithmetic"}
        # the packed prefill's launch shape and memory traffic without its arithmetic
        if prefill is not None and prefill["case"].D == 128:
            pc, tz, NP = prefill["case"], prefill["tensors"], prefill["layers"]

            def fpre(i):
                j = i % NP
                assert L.ceil_prefill_shape(tz["q"][j].data_ptr(), tz["k"][j].data_ptr(),
                                            tz["v"][j].data_ptr(), tz["cu"].data_ptr(), pc.n_docs,
                                            pc.L, pc.H_q, pc.H_kv, tz["out"].data_ptr(),
                                            tz["lse"].data_ptr(), st()) == 0
            ms = timer(fpre, K) / K
            fl = pc.flops()
            out["prefill_shape_stream"] = {
                "us": round(ms * 1e3, 3), "flops_of_the_call": int(fl),
                "tflops_if_at_this_time": round(fl / (ms * 1e-3) / 1e12, 1),
                "frac_of_bf16_peak_if_at_this_time": round(fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "note": "the packed prefill's grid and tile order, tile search, Q rows read once, "
                        "each document's K/V streamed in 32-key stages (one in flight), output "
                        "rows and LSEs written, at the prefill's occupancy (three workgroups per CU); "
                        "no arithmetic. Cold: the same rotating input sets"}
        fsink = torch.zeros(1024, dtype=torch.float32, device=dev)
        iters, grid = 4000, 2 * cus

        def fm(i):
            assert L.ceil_mfma(grid, iters, fsink.data_ptr(), st()) == 0
        ms = timer(fm, 4) / 4
        flops = grid * 4 * iters * 16 * (16 * 16 * 32 * 2)
        out["mfma_bf16"] = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                            "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                            "kernel": "v_mfma_f32_16x16x32_bf16, 16 independent accumulators "
                                      "per wave, 2 waves per SIMD"}
    # a plain device copy: reads and writes the same number of bytes (mixed traffic, as in
    # prefill, whose compulsory bytes are 61% reads and 39% writes)
    csrc = torch.ones(1024 ** 3 // 4, dtype=torch.float32, device=dev)  # past the Infinity Cache
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    torch.cuda.synchronize()
    e0, e1 = timer.events()
    e0.record()
    for _ in range(10):
        cdst.copy_(csrc)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / 10
    cb = 2 * csrc.numel() * 4
    out["copy_read_write"] = {"gbs": round(cb / (ms * 1e-3) / 1e9, 1), "bytes_moved": cb,
                              "frac_of_hbm_peak": round(cb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "note": "torch device copy of 1 GiB: bytes read plus bytes written "
                                      "per second"}
    del csrc, cdst
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    b = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    cbuf = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.matmul(a, b, out=cbuf)
    torch.cuda.synchronize()
    e0, e1 = timer.events()
    e0.record()
    for _ in range(5):
        torch.matmul(a, b, out=cbuf)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / 5
    out["torch_matmul_bf16"] = {"tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1),
                                "shape": [n, n, n],
                                "frac_of_peak": round(2 * n ** 3 / (ms * 1e-3) / 1e12
                                                      / BF16_PEAK_TFLOPS, 4)}
    return out


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
    from workloads import make_case

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import dev_bf16, dev_i32

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream, args, dev)
    K = args.steps

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------- decode inputs (bucketed B=64), one KV cache per layer
    c = make_case(3, fill="zero")
    db = DecodeBench(torch, pkv, c, dev, layers=max(1, args.layers))
    balanced = bool(args.flags & pkv.PKV_F_BALANCED)
    sched, S_eff, W = plan_name(pkv, c, args.num_splits, args.flags, db.max_kv)
    S = args.num_splits
    kv_bytes = db.kv_bytes
    app_bi = dev_i32(c.batch_idx[db.act].astype(np.int32))
    app_pos = dev_i32((c.kv_len[db.act] - 1).astype(np.int32))
    app_k = db.rk[torch.from_numpy(db.act).to(dev)].contiguous()
    app_v = db.rv[torch.from_numpy(db.act).to(dev)].contiguous()
    decode_only = db.call(S, args.flags)
    decode_step_fused = db.fused(S, args.flags)

    def decode_step_separate(i):
        j = i % db.NL
        pkv.paged_kv_append(db.k[j], db.v[j], db.pt, app_bi, app_pos, app_k, app_v,
                            page_size=c.page_size)
        decode_only(i)

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
                       tensors=dict(q=p_q, k=p_k, v=p_v, cu=p_cu, out=p_out, lse=p_lse),
                       step=prefill_step_separate if args.separate else prefill_step_fused,
                       alt=prefill_step_fused if args.separate else prefill_step_separate)

    # ---------------- chunked prefill over a paged prefix (64 sequences), one pool set per layer
    chunked = None
    if not args.no_chunked and args.only is None:
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

    # ---------------- context: the same prefill kernel on two 8192-token documents, where
    # the per-tile start-up and the launch tail are small next to the key loop
    long_pf = None
    if not args.no_prefill and args.only is None:
        from workloads import make_prefill_case
        lc = make_prefill_case(name="long", seed=9306, doc_lens=[8192, 8192], H_q=32, H_kv=8,
                               D=128, page_size=128, num_pages=130, max_blocks=64)
        NLP = 2
        l_q = [dev_bf16(lc.q) for _ in range(NLP)]
        l_k = [dev_bf16(lc.k) for _ in range(NLP)]
        l_v = [dev_bf16(lc.v) for _ in range(NLP)]
        l_cu = dev_i32(lc.cu_seqlens)
        l_out = torch.empty((lc.L, lc.H_q, lc.D), dtype=torch.bfloat16, device=dev)
        l_lse = torch.empty((lc.L, lc.H_q), dtype=torch.float32, device=dev)

        def long_step(i):
            j = i % NLP
            pkv.packed_prefill_attn(l_q[j], l_k[j], l_v[j], l_cu, scale=float(lc.scale),
                                    out=l_out, lse=l_lse)

        long_pf = dict(case=lc, step=long_step, layers=NLP)

    # ---------------- profiling runs: one attention call type only
    if args.only is not None:
        fn = decode_only if args.only == "decode" else prefill["attn"]
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ms = timer(fn, K) / K
        print(json.dumps({"only": args.only, "avg_call_us": round(ms * 1e3, 3), "steps": K}),
              flush=True)
        return

    # ---------------- warmup
    for i in range(args.warmup):
        decode_step(i)
        if prefill:
            prefill["step"](i)
        if chunked:
            chunked["step"](i)
    torch.cuda.synchronize()
    progress("warmup done")

    # ---------------- timed steps
    t0 = time.perf_counter()
    dec_total = timer(decode_step, K)
    pre_total = timer(prefill["step"], K) if prefill else 0.0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the dominant kernels alone (roofline): decode attention, prefill attention
    dk_reps, pa_reps = [], []
    dk_total = timer(decode_only, K, dk_reps)
    alt_total = timer(decode_step_fused if args.separate else decode_step_separate, K)
    pa_total = timer(prefill["attn"], K, pa_reps) if prefill else 0.0
    palt_total = timer(prefill["alt"], K) if prefill else 0.0
    ch_total = timer(chunked["step"], K) if chunked else 0.0
    lp_total = timer(long_pf["step"], K) if long_pf else 0.0
    # warm, for context: every call reads the same cache (input set), which
    # then sits in the 256 MiB Infinity Cache; not an HBM figure
    dw_total = timer(db.call(S, args.flags, rotate=False), K)
    pw_total = timer(lambda i: prefill["attn"](0), K) if prefill else 0.0
    progress("headline steps timed")

    dec_ms, dk_ms = dec_total / K, dk_total / K
    value = kv_bytes / (dec_ms * 1e-3) / 1e9
    achieved = kv_bytes / (dk_ms * 1e-3) / 1e9
    cache = ("flushed: 1 GiB read before each call" if args.flush else
             f"cold: {db.NL} KV caches (one per layer) read round-robin, "
             f"{(db.NL - 1) * kv_bytes / 1e9:.2f} GB of other KV between reuses")
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
            "schedule": sched,
            "launch": "eager stream launches" if (args.eager or args.flush) else
                      f"one HIP graph of the {K} timed steps, replayed once",
            "flags": int(args.flags),
            "cache": cache,
            "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": decode_kernels(S_eff, W) + " (one paged_decode_attn call)",
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
                # the binding roof at this intensity: min(matrix peak, intensity x HBM peak)
                "intensity_flop_per_byte": round(flops / p_bytes, 1),
                "frac_of_intensity_roof": round(
                    tflops / min(BF16_PEAK_TFLOPS, flops / p_bytes * HBM_PEAK_GBS / 1e3), 4),
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
    if long_pf:
        lc = long_pf["case"]
        lp_ms = lp_total / K
        out["prefill_long_documents"] = {
            "workload": "packed prefill of 2 documents of 8192 tokens (L=16384), H_q=32 H_kv=8 "
                        "D=128, document-causal; context for the kernel's rate once per-tile "
                        "start-up and the launch tail are small",
            "call": "packed_prefill_attn",
            "us": round(lp_ms * 1e3, 3),
            "flops_per_call": int(lc.flops()),
            "tflops": round(lc.flops() / (lp_ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(lc.flops() / (lp_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "cache": f"cold: {long_pf['layers']} input sets read round-robin",
        }

    # ---------------- every named workload on its own
    cases = {3: c}
    if not args.no_configs:
        cfgs = {}
        # B=64 bucket: the contiguous-page path against the page-table walk, same layout
        ab = {}
        for name, fl in (("detect (default)", 0), ("walk (PKV_F_NO_CONTIG_DETECT)",
                                                   pkv.PKV_F_NO_CONTIG_DETECT),
                         ("assume (PKV_F_ASSUME_CONTIGUOUS)", pkv.PKV_F_ASSUME_CONTIGUOUS)):
            r, _ = time_decode(timer, db, K, S, args.flags | fl, warm=False, replays=True)
            ab[name] = r
        cfgs["3"] = {"workload": out["config"]["workload"] + " (decode call alone)",
                     "kv_bytes": int(kv_bytes), "schedule": sched,
                     "contiguous_path": ab,
                     "note": "same sequential pages, same schedule; cold rotating caches"}
        progress("config 3 paths timed")
        # tiny decode: launch-bound, context only
        c1 = cases[1] = make_case(1, fill="zero")
        d1 = DecodeBench(torch, pkv, c1, dev, layers=2)
        r1 = {}
        for S1, fl1, nm in ((0, 0, "auto"), (2, 0, "split 2"), (0, pkv.PKV_F_BALANCED, "balanced")):
            rr, _ = time_decode(timer, d1, K, S1, fl1)
            r1[nm + " (" + plan_name(pkv, c1, S1, fl1, d1.max_kv)[0] + ")"] = rr
        cfgs["1"] = {"workload": "tiny decode B=3 (slot 0 padding), H_q=4 H_kv=2 D=64 "
                                 "page_size=16, 37 and 70 keys", "kv_bytes": int(d1.kv_bytes),
                     "schedules": r1, "note": "launch-bound; context only"}
        d1.free()
        # B=8 Qwen3-4B decode + append
        c2 = cases[2] = make_case(2, fill="zero")
        d2 = DecodeBench(torch, pkv, c2, dev)
        r2 = {}
        for S2, fl2, nm in ((0, 0, "auto"), (1, 0, "single pass"),
                            (0, pkv.PKV_F_BALANCED, "balanced")):
            rr, _ = time_decode(timer, d2, K, S2, fl2, replays=(nm == "auto"))
            r2[nm + " (" + plan_name(pkv, c2, S2, fl2, d2.max_kv)[0] + ")"] = rr
        app_ms = timer(d2.fused(0, 0), K) / K
        cfgs["2"] = {"workload": "Qwen3-4B decode B=8, H_q=32 H_kv=8 D=128 page_size=128, "
                                 "contexts U[256,1536], shuffled pages",
                     "kv_bytes": int(d2.kv_bytes), "layers": d2.NL, "schedules": r2,
                     "fused_append_step_us": round(app_ms * 1e3, 3)}
        d2.free()
        progress("config 2 timed")
        # B=256, 4096-page pool: automatic plan, split-K + merge, balanced
        c4 = cases[4] = make_case(4, fill="zero")
        d4 = DecodeBench(torch, pkv, c4, dev)
        r4 = {}
        for S4, fl4, nm in ((0, 0, "auto"), (2, 0, "split-K 2 + merge"),
                            (4, 0, "split-K 4 + merge"), (0, pkv.PKV_F_BALANCED, "balanced")):
            rr, _ = time_decode(timer, d4, max(4, K // 4), S4, fl4, replays=(nm == "auto"))
            r4[nm + " (" + plan_name(pkv, c4, S4, fl4, d4.max_kv)[0] + ")"] = rr
        cfgs["4"] = {"workload": "large-batch decode B=256, H_q=32 H_kv=8 D=128 page_size=128, "
                                 "contexts U[1024,2048], 4096-page pool, shuffled pages",
                     "kv_bytes": int(d4.kv_bytes), "layers": d4.NL, "schedules": r4}
        d4.free()
        progress("config 4 timed")
        if prefill:
            cfgs["5"] = {"workload": out["prefill"]["workload"],
                         "see": "prefill (attention call) and prefill.roofline"}
        out["configs"] = cfgs

    if not args.no_ceilings:
        out["ceilings"] = ceilings(torch, timer, dev, db, K, prefill)
        progress("ceilings measured")

    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_decode_baseline(c, args.cpu_seconds, single=False)
        out["cpu_baseline"]["cpu_model"] = cpu_model()
        if not args.no_configs:
            per = {}
            for k in (1, 2, 3, 4):
                per[str(k)] = cpu_decode_baseline(cases[k], args.cpu_seconds)
            if prefill:
                per["5"] = cpu_prefill_baseline(prefill["case"], args.cpu_seconds)
            out["cpu_baselines"] = {"cpu_model": cpu_model(), "nproc": os.cpu_count(),
                                    "per_config": per}
        progress("oracle timed")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
