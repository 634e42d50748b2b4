"""Seeded synthetic workloads for GQA attention over a paged KV cache.

The cache format follows the flex paged-attention commit page ("Why this
works", point 1): one bfloat16 pool per K and per V, shaped
[H_kv, num_pages * page_size, D], and a page table that maps
(batch slot, logical block) to a physical page. Slot 0 and page 0 are the
reserved padding entries (same page, point 3).

Everything here is input construction: random draws, rounding of those draws
to bfloat16 bit patterns, and writing them into pages. There is no attention
arithmetic in this module; the CPU reference and the GPU library both read
the arrays it returns.

Random draws use numpy's PCG64 generator.  Order of draws for one case:
lengths (by the config builders), the page permutation (shuffled layouts
only), q, K values, V values, then the appended tokens' K and V.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BF16_NAN = 0x7FC0  # quiet NaN; fills every cache byte that holds no valid key


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits.

    A bfloat16 is the upper half of an IEEE binary32.  Rounding adds
    0x7FFF plus the lowest kept bit, then truncates.  Inputs here are finite
    normal draws, so no NaN/Inf special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32 (shift into the top half)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclass
class DecodeCase:
    """One decode step: a paged cache, a page table and one query per row."""

    name: str
    seed: int
    H_q: int
    H_kv: int
    D: int
    page_size: int
    num_pages: int
    num_slots: int
    max_blocks: int
    scale: np.float32
    q: np.ndarray            # uint16 [B, H_q, D]
    k_pool: np.ndarray       # uint16 [H_kv, num_pages*page_size, D]
    v_pool: np.ndarray       # uint16 [H_kv, num_pages*page_size, D]
    page_table: np.ndarray   # int32 [num_slots, max_blocks]; 0 = no page
    batch_idx: np.ndarray    # int32 [B]; 0 = padding row
    kv_len: np.ndarray       # int32 [B]; valid keys of the row, appended token included
    contiguous: bool         # pages of every active row were handed out consecutively
    # Tokens to append before the decode (one per active row, at position kv_len-1),
    # or None when the pool already holds every valid key.
    app_batch_idx: Optional[np.ndarray] = None   # int32 [N]
    app_input_pos: Optional[np.ndarray] = None   # int32 [N]
    app_k: Optional[np.ndarray] = None           # uint16 [N, H_kv, D]
    app_v: Optional[np.ndarray] = None           # uint16 [N, H_kv, D]
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    def active_rows(self) -> np.ndarray:
        return np.nonzero((self.batch_idx != 0) & (self.kv_len > 0))[0]

    def kv_bytes(self) -> int:
        """Bytes of K and V that the valid keys occupy (the decode's compulsory read)."""
        n = int(self.kv_len[self.active_rows()].astype(np.int64).sum())
        return n * self.H_kv * self.D * 2 * 2


@dataclass
class PrefillCase:
    """Packed prompts (document-causal attention) plus the scatter of their K/V into pages."""

    name: str
    seed: int
    H_q: int
    H_kv: int
    D: int
    scale: np.float32
    q: np.ndarray            # uint16 [L, H_q, D]
    k: np.ndarray            # uint16 [L, H_kv, D]
    v: np.ndarray            # uint16 [L, H_kv, D]
    cu_seqlens: np.ndarray   # int32 [n_docs+1]
    # paged destination for the scatter of k/v
    page_size: int
    num_pages: int
    num_slots: int
    max_blocks: int
    page_table: np.ndarray   # int32 [num_slots, max_blocks]
    batch_idx: np.ndarray    # int32 [L]; document d lives in slot d+1
    input_pos: np.ndarray    # int32 [L]; position inside the document
    meta: dict = field(default_factory=dict)

    @property
    def L(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_docs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def doc_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    def flops(self) -> int:
        """4*D*H_q per unmasked (query, key) pair, diagonal included."""
        n = self.doc_lens()
        pairs = int((n * (n + 1) // 2).sum())
        return 4 * self.D * self.H_q * pairs


def _assign_pages(rng, row_slots, row_blocks, num_pages, layout):
    """Physical page ids for each active row's blocks, in row then block order."""
    need = int(sum(row_blocks))
    if need > num_pages - 1:
        raise ValueError(f"{need} pages needed, pool has {num_pages - 1} usable")
    if layout == "shuffled":
        order = rng.permutation(np.arange(1, num_pages, dtype=np.int64))
    elif layout == "sequential":
        order = np.arange(1, num_pages, dtype=np.int64)
    else:
        raise ValueError(layout)
    out, pos = [], 0
    for nb in row_blocks:
        out.append(order[pos:pos + nb].astype(np.int32))
        pos += nb
    return out


def make_decode_case(*, name: str, seed: int, H_q: int, H_kv: int, D: int, page_size: int,
                     num_pages: int, num_slots: int, max_blocks: int,
                     row_slots: Sequence[int], row_lens: Sequence[int],
                     layout: str = "shuffled", fill: str = "nan",
                     append_last: bool = False, rng: Optional[np.random.Generator] = None,
                     scale: Optional[float] = None) -> DecodeCase:
    """Build one decode step.

    row_slots[r] is the batch slot of row r (0 = padding) and row_lens[r] its
    number of valid keys.  Active rows must use distinct slots.  `fill` picks
    what the cache holds where no valid key lives: 'nan' (bf16 quiet NaN, so a
    stray read shows up), 'zero', or 'empty' (np.zeros, for timing runs).
    With append_last the last key of every active row is held back from the
    pool and returned as a token to append at position kv_len-1.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    row_slots = np.asarray(row_slots, dtype=np.int32)
    row_lens = np.asarray(row_lens, dtype=np.int32)
    B = int(row_slots.shape[0])
    active = [r for r in range(B) if row_slots[r] != 0 and row_lens[r] > 0]
    slots_used = [int(row_slots[r]) for r in active]
    if len(set(slots_used)) != len(slots_used):
        raise ValueError("active rows must use distinct slots")
    if any(s >= num_slots for s in slots_used):
        raise ValueError("slot id beyond num_slots")
    blocks = [-(-int(row_lens[r]) // page_size) for r in active]
    if any(b > max_blocks for b in blocks):
        raise ValueError("row longer than max_blocks*page_size")
    pages = _assign_pages(rng, slots_used, blocks, num_pages, layout)
    pt = np.zeros((num_slots, max_blocks), dtype=np.int32)
    for s, pg in zip(slots_used, pages):
        pt[s, :len(pg)] = pg
    contiguous = all(bool(np.all(np.diff(pg) == 1)) for pg in pages)

    q = _normal_bf16(rng, (B, H_q, D))

    rows_total = num_pages * page_size
    if fill == "nan":
        k_pool = np.full((H_kv, rows_total, D), BF16_NAN, dtype=np.uint16)
        v_pool = np.full((H_kv, rows_total, D), BF16_NAN, dtype=np.uint16)
    elif fill in ("zero", "empty"):
        k_pool = np.zeros((H_kv, rows_total, D), dtype=np.uint16)
        v_pool = np.zeros((H_kv, rows_total, D), dtype=np.uint16)
    else:
        raise ValueError(fill)

    # physical row of every valid key, rows in order, keys in order
    phys = []
    for r, pg in zip(active, pages):
        n = int(row_lens[r])
        j = np.arange(n, dtype=np.int64)
        phys.append(pg[j // page_size].astype(np.int64) * page_size + j % page_size)
    phys_all = np.concatenate(phys) if phys else np.zeros(0, dtype=np.int64)
    nkeys = int(phys_all.shape[0])
    kv_k = _normal_bf16(rng, (nkeys, H_kv, D))
    kv_v = _normal_bf16(rng, (nkeys, H_kv, D))

    app = dict(app_batch_idx=None, app_input_pos=None, app_k=None, app_v=None)
    if append_last:
        # the last key of each active row is the token the decode step appends
        ends = np.cumsum([int(row_lens[r]) for r in active]) - 1
        keep = np.ones(nkeys, dtype=bool)
        keep[ends] = False
        app = dict(app_batch_idx=np.asarray(slots_used, dtype=np.int32),
                   app_input_pos=np.asarray([int(row_lens[r]) - 1 for r in active], dtype=np.int32),
                   app_k=np.ascontiguousarray(kv_k[ends]), app_v=np.ascontiguousarray(kv_v[ends]))
        phys_w, k_w, v_w = phys_all[keep], kv_k[keep], kv_v[keep]
    else:
        phys_w, k_w, v_w = phys_all, kv_k, kv_v
    for h in range(H_kv):
        k_pool[h, phys_w, :] = k_w[:, h, :]
        v_pool[h, phys_w, :] = v_w[:, h, :]

    sc = np.float32(scale if scale is not None else 1.0 / np.sqrt(D))
    return DecodeCase(name=name, seed=seed, H_q=H_q, H_kv=H_kv, D=D, page_size=page_size,
                      num_pages=num_pages, num_slots=num_slots, max_blocks=max_blocks,
                      scale=sc, q=q, k_pool=k_pool, v_pool=v_pool, page_table=pt,
                      batch_idx=row_slots.copy(), kv_len=row_lens.copy(), contiguous=contiguous,
                      meta=dict(layout=layout, fill=fill), **app)


def make_prefill_case(*, name: str, seed: int, doc_lens: Sequence[int], H_q: int, H_kv: int,
                      D: int, page_size: int = 128, num_pages: int = 2048, max_blocks: int = 16,
                      layout: str = "shuffled", rng: Optional[np.random.Generator] = None,
                      scale: Optional[float] = None) -> PrefillCase:
    """Pack documents into one sequence; document d owns batch slot d+1.

    The paged destination gives slot d+1 ceil(n_d/page_size) pages drawn in
    document order from the layout's page order.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(doc_lens, dtype=np.int64)
    n_docs = int(lens.shape[0])
    cu = np.zeros(n_docs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    L = int(cu[-1])
    num_slots = n_docs + 1
    blocks = [-(-int(n) // page_size) for n in lens]
    if any(b > max_blocks for b in blocks):
        raise ValueError("document longer than max_blocks*page_size")
    pages = _assign_pages(rng, list(range(1, n_docs + 1)), blocks, num_pages, layout)
    pt = np.zeros((num_slots, max_blocks), dtype=np.int32)
    for d, pg in enumerate(pages):
        pt[d + 1, :len(pg)] = pg
    q = _normal_bf16(rng, (L, H_q, D))
    k = _normal_bf16(rng, (L, H_kv, D))
    v = _normal_bf16(rng, (L, H_kv, D))
    bidx = np.repeat(np.arange(1, n_docs + 1, dtype=np.int32), lens)
    ipos = np.concatenate([np.arange(int(n), dtype=np.int32) for n in lens]) if n_docs else \
        np.zeros(0, dtype=np.int32)
    sc = np.float32(scale if scale is not None else 1.0 / np.sqrt(D))
    return PrefillCase(name=name, seed=seed, H_q=H_q, H_kv=H_kv, D=D, scale=sc, q=q, k=k, v=v,
                       cu_seqlens=cu, page_size=page_size, num_pages=num_pages,
                       num_slots=num_slots, max_blocks=max_blocks, page_table=pt,
                       batch_idx=bidx, input_pos=ipos.astype(np.int32), meta=dict(layout=layout))


@dataclass
class ChunkedPrefillCase:
    """Prompt chunks continuing sequences whose first tokens are already cached in pages."""

    name: str
    seed: int
    H_q: int
    H_kv: int
    D: int
    scale: np.float32
    q: np.ndarray            # uint16 [L, H_q, D], the chunks packed
    k: np.ndarray            # uint16 [L, H_kv, D]
    v: np.ndarray            # uint16 [L, H_kv, D]
    cu_seqlens: np.ndarray   # int32 [n+1], chunk bounds
    prefix_lens: np.ndarray  # int32 [n], cached tokens before each chunk
    doc_slots: np.ndarray    # int32 [n], batch slot of each sequence (0 = padding)
    page_size: int
    num_pages: int
    num_slots: int
    max_blocks: int
    page_table: np.ndarray   # int32 [num_slots, max_blocks]
    k_pool: np.ndarray       # uint16 [H_kv, num_pages*page_size, D], the cached prefixes
    v_pool: np.ndarray
    batch_idx: np.ndarray    # int32 [L], slot of each chunk token
    input_pos: np.ndarray    # int32 [L], position of each chunk token in its sequence
    meta: dict = field(default_factory=dict)

    @property
    def L(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_docs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def flops(self) -> int:
        """4*D*H_q per (query, key) pair a live chunk row attends to (prefix + causal chunk)."""
        live = self.doc_slots[self.batch_idx_doc()] != 0
        return 4 * self.D * self.H_q * int((self.input_pos[live].astype(np.int64) + 1).sum())

    def batch_idx_doc(self) -> np.ndarray:
        """Document of each chunk token."""
        return np.repeat(np.arange(self.n_docs), np.diff(self.cu_seqlens.astype(np.int64)))


def make_chunked_prefill_case(*, name: str, seed: int, prefix_lens: Sequence[int],
                              chunk_lens: Sequence[int], H_q: int, H_kv: int, D: int,
                              page_size: int, slots: Optional[Sequence[int]] = None,
                              num_pages: Optional[int] = None, max_blocks: Optional[int] = None,
                              layout: str = "shuffled", fill: str = "nan",
                              rng: Optional[np.random.Generator] = None,
                              scale: Optional[float] = None) -> ChunkedPrefillCase:
    """Build one chunked-prefill step.

    Sequence d lives in slot slots[d] (default d+1; 0 = padding) and owns
    ceil((prefix_d + chunk_d) / page_size) pages, assigned in the layout's
    order; its prefix K/V (positions 0..prefix_d-1) are drawn and written into
    the pools, whose other bytes hold `fill` ('nan', 'zero' or 'empty').
    Draw order: page permutation, prefix K, prefix V, chunk q, k, v.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    chunk = np.asarray(chunk_lens, dtype=np.int32)
    n = int(prefix.shape[0])
    slots = np.asarray(slots if slots is not None else np.arange(1, n + 1), dtype=np.int32)
    live = [d for d in range(n) if slots[d] != 0]
    if len(set(int(slots[d]) for d in live)) != len(live):
        raise ValueError("live sequences must use distinct slots")
    blocks = [-(-int(prefix[d] + chunk[d]) // page_size) for d in live]
    mb = max_blocks if max_blocks is not None else max(blocks + [1])
    if any(b > mb for b in blocks):
        raise ValueError("sequence longer than max_blocks*page_size")
    P = num_pages if num_pages is not None else sum(blocks) + 2
    pages = _assign_pages(rng, [int(slots[d]) for d in live], blocks, P, layout)
    num_slots = int(slots.max()) + 1 if n else 1
    pt = np.zeros((num_slots, mb), dtype=np.int32)
    for d, pg in zip(live, pages):
        pt[slots[d], :len(pg)] = pg
    rows_total = P * page_size
    if fill == "nan":
        k_pool = np.full((H_kv, rows_total, D), BF16_NAN, dtype=np.uint16)
    elif fill in ("zero", "empty"):
        k_pool = np.zeros((H_kv, rows_total, D), dtype=np.uint16)
    else:
        raise ValueError(fill)
    v_pool = k_pool.copy()
    phys = []
    for d, pg in zip(live, pages):
        j = np.arange(int(prefix[d]), dtype=np.int64)
        phys.append(pg[j // page_size].astype(np.int64) * page_size + j % page_size)
    phys_all = np.concatenate(phys) if phys else np.zeros(0, dtype=np.int64)
    pk = _normal_bf16(rng, (phys_all.shape[0], H_kv, D))
    pv = _normal_bf16(rng, (phys_all.shape[0], H_kv, D))
    for h in range(H_kv):
        k_pool[h, phys_all, :] = pk[:, h, :]
        v_pool[h, phys_all, :] = pv[:, h, :]
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunk)
    L = int(cu[-1])
    q = _normal_bf16(rng, (L, H_q, D))
    k = _normal_bf16(rng, (L, H_kv, D))
    v = _normal_bf16(rng, (L, H_kv, D))
    bidx = np.repeat(slots, chunk).astype(np.int32)
    ipos = np.concatenate([int(prefix[d]) + np.arange(int(chunk[d]), dtype=np.int32)
                           for d in range(n)]).astype(np.int32) if n else np.zeros(0, np.int32)
    sc = np.float32(scale if scale is not None else 1.0 / np.sqrt(D))
    return ChunkedPrefillCase(name=name, seed=seed, H_q=H_q, H_kv=H_kv, D=D, scale=sc, q=q, k=k,
                              v=v, cu_seqlens=cu, prefix_lens=prefix, doc_slots=slots,
                              page_size=page_size, num_pages=P, num_slots=num_slots,
                              max_blocks=mb, page_table=pt, k_pool=k_pool, v_pool=v_pool,
                              batch_idx=bidx, input_pos=ipos, meta=dict(layout=layout, fill=fill))


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds are 2300 + config number.  "Uniform in
# [a, b]" means integers, both ends included.
# ---------------------------------------------------------------------------

def _cfg1(fill="nan"):
    # Tiny decode: slot 0 is the padding row; slots 1 and 2 hold 37 and 70 keys.
    seed = 2301
    return make_decode_case(name="tiny decode B=3 Hq=4 Hkv=2 D=64 ps=16", seed=seed, H_q=4, H_kv=2,
                            D=64, page_size=16, num_pages=16, num_slots=3, max_blocks=8,
                            row_slots=[0, 1, 2], row_lens=[1, 37, 70], layout="shuffled", fill=fill)


def _cfg2(fill="nan"):
    # Qwen3-4B-shaped decode, one layer, plus the append of one token per sequence.
    seed = 2302
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(256, 1536, size=8, endpoint=True)
    return make_decode_case(name="qwen3-4b decode B=8 Hq=32 Hkv=8 D=128 ps=128 + append", seed=seed,
                            H_q=32, H_kv=8, D=128, page_size=128, num_pages=2048, num_slots=9,
                            max_blocks=16, row_slots=list(range(1, 9)), row_lens=lens,
                            layout="shuffled", fill=fill, append_last=True, rng=rng)


def _cfg3(fill="nan"):
    # Bucketed decode: 50 live sequences padded to a bucket of 64 rows with slot 0.
    seed = 2303
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 1024, size=50, endpoint=True)
    slots = list(range(1, 51)) + [0] * 14
    row_lens = list(lens) + [1] * 14
    return make_decode_case(name="bucketed decode B=64 (50 active) Hq=32 Hkv=8 D=128 ps=128 sequential pages",
                            seed=seed, H_q=32, H_kv=8, D=128, page_size=128, num_pages=2048,
                            num_slots=65, max_blocks=16, row_slots=slots, row_lens=row_lens,
                            layout="sequential", fill=fill, rng=rng)


def _cfg4(fill="nan"):
    # Large-batch decode over a 4096-page pool with shuffled pages.
    seed = 2304
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1024, 2048, size=256, endpoint=True)
    return make_decode_case(name="large-batch decode B=256 Hq=32 Hkv=8 D=128 ps=128 shuffled",
                            seed=seed, H_q=32, H_kv=8, D=128, page_size=128, num_pages=4096,
                            num_slots=257, max_blocks=16, row_slots=list(range(1, 257)),
                            row_lens=lens, layout="shuffled", fill=fill, rng=rng)


def _cfg5(fill="nan"):
    # Packed prefill: 64 prompts of 64..512 tokens, document-causal.
    del fill
    seed = 2305
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(64, 512, size=64, endpoint=True)
    return make_prefill_case(name="packed prefill 64 docs Hq=32 Hkv=8 D=128", seed=seed,
                             doc_lens=lens, H_q=32, H_kv=8, D=128, page_size=128,
                             num_pages=2048, max_blocks=16, layout="shuffled", rng=rng)


CONFIGS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


def make_case(config: int, fill: str = "nan"):
    """Build named workload 1..5 (see the builders above for shapes)."""
    return CONFIGS[config](fill=fill)
