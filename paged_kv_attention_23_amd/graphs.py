"""Graph-captured decode per batch bucket.

The flex commit page ("Why this works", point 3) captures one CUDA graph
per batch-size bucket (1, 2, 4, 8, 16, 32, ...) during warmup, dispatches
every decode step to the nearest bucket at or above the live batch and pads
the missing rows with batch slot 0, the reserved no-op slot; it names graph
replay as the lever that closes the gap to vLLM (the inference script of the
qwen3_flex_inference.py page does it in its decode-step and graph-capture
functions).  DecodeGraphs does the same for one attention layer on MI355X:
one HIP graph per bucket of paged_decode_attn_append (append of each row's
new token + decode, plus the split merge when the plan has one) over fixed
pools and static input buffers.

The library calls allocate nothing and never synchronise, so capture needs
no special mode: all buffers (inputs, outputs, split workspace) are
allocated here before capture, and no memset is recorded (padding rows are
cleared with torch fill kernels outside the graph).  The page table is read
by the kernels at replay time, so its contents may change between steps; the
pools and the page table must stay at the same addresses.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _binding as B


def default_buckets(max_batch: int) -> list:
    """[1, 2, 4, 8] and then multiples of 16 up to max_batch (max_batch always included)."""
    out = [b for b in (1, 2, 4, 8) if b <= max_batch]
    out += list(range(16, max_batch + 1, 16))
    if not out or out[-1] != max_batch:
        out.append(max_batch)
    return sorted(set(out))


class DecodeGraphs:
    """One captured fused append+decode step per batch bucket, for fixed pools.

    max_kv_len bounds every row's kv_len over the runner's lifetime; the
    split plan of each bucket is fixed at capture from it (a loose bound costs
    speed, never correctness).
    """

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
                 num_q_heads: int, page_size: int, scale: float, max_batch: int,
                 max_kv_len: int, buckets: Optional[Sequence[int]] = None, num_splits: int = 0,
                 flags: int = 0):
        if max_batch <= 0:
            raise ValueError("max_batch must be positive")
        self.k_pool, self.v_pool, self.page_table = k_pool, v_pool, page_table
        self.page_size, self.scale = int(page_size), float(scale)
        self.max_kv_len, self.num_splits, self.flags = int(max_kv_len), int(num_splits), int(flags)
        self.buckets = sorted(set(int(b) for b in (buckets or default_buckets(max_batch))))
        if self.buckets[0] <= 0 or self.buckets[-1] < max_batch:
            raise ValueError("buckets must be positive and reach max_batch")
        H_kv, _, D = k_pool.shape
        Bmax = self.buckets[-1]
        dev = k_pool.device
        self.q = torch.zeros((Bmax, num_q_heads, D), dtype=torch.bfloat16, device=dev)
        self.k_new = torch.zeros((Bmax, H_kv, D), dtype=torch.bfloat16, device=dev)
        self.v_new = torch.zeros((Bmax, H_kv, D), dtype=torch.bfloat16, device=dev)
        self.batch_idx = torch.zeros((Bmax,), dtype=torch.int32, device=dev)
        self.kv_len = torch.zeros((Bmax,), dtype=torch.int32, device=dev)
        self.out = torch.zeros((Bmax, num_q_heads, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.zeros((Bmax, num_q_heads), dtype=torch.float32, device=dev)
        ws = max(B.paged_decode_workspace_size(b, num_q_heads, H_kv, D, self.num_splits,
                                               self.flags) for b in self.buckets)
        self.workspace = torch.empty((max(ws, 16),), dtype=torch.uint8, device=dev)
        self.graphs: Dict[int, torch.cuda.CUDAGraph] = {}
        torch.cuda.synchronize(dev)
        for b in reversed(self.buckets):  # largest first, as the reference captures
            self._step(b)                  # eager run: plans and checks arguments
            torch.cuda.synchronize(dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._step(b)
            self.graphs[b] = g
        torch.cuda.synchronize(dev)

    def _step(self, b: int) -> None:
        B.paged_decode_attn_append(
            self.q[:b], self.k_new[:b], self.v_new[:b], self.k_pool, self.v_pool, self.page_table,
            self.batch_idx[:b], self.kv_len[:b], page_size=self.page_size, scale=self.scale,
            max_kv_len=self.max_kv_len, num_splits=self.num_splits, flags=self.flags,
            workspace=self.workspace, out=self.out[:b], lse=self.lse[:b])

    def bucket_for(self, batch: int) -> int:
        for b in self.buckets:
            if b >= batch:
                return b
        raise ValueError(f"batch {batch} exceeds the largest bucket {self.buckets[-1]}")

    def inputs(self, batch: int) -> Dict[str, torch.Tensor]:
        """Static input views for a batch of `batch` rows (q, k_new, v_new, batch_idx, kv_len).
        Write the step's inputs into them in place, then call run(batch)."""
        self.bucket_for(batch)
        return {"q": self.q[:batch], "k_new": self.k_new[:batch], "v_new": self.v_new[:batch],
                "batch_idx": self.batch_idx[:batch], "kv_len": self.kv_len[:batch]}

    def run(self, batch: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """Replay the bucket of `batch` rows on the static inputs; rows past `batch` up to the
        bucket become padding (slot 0, no keys).  Returns views (out [batch, H_q, D],
        lse [batch, H_q]) valid until the next step."""
        b = self.bucket_for(batch)
        if b > batch:  # padding rows: slot 0, no keys (fill kernels, outside the graph)
            self.batch_idx[batch:b].zero_()
            self.kv_len[batch:b].zero_()
        self.graphs[b].replay()
        return self.out[:batch], self.lse[:batch]

    def __call__(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                 batch_idx: torch.Tensor, kv_len: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        """Copy one step's inputs into the static buffers and run it (see inputs/run)."""
        n = q.shape[0]
        views = self.inputs(n)
        for name, src in (("q", q), ("k_new", k_new), ("v_new", v_new), ("batch_idx", batch_idx),
                          ("kv_len", kv_len)):
            views[name].copy_(src)
        return self.run(n)
