"""CPU-only checks of the C ABI: the library loads, exports what include/pkv.h
declares, and rejects bad arguments on the host before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")
LIB = os.path.join(ROOT, "paged_kv_attention_23_amd", "libpkv.so")

from paged_kv_attention_23_amd import _binding as B  # noqa: E402


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) >= {"paged_kv_append", "paged_decode_attn", "packed_prefill_attn",
                          "paged_decode_attn_append",
                          "paged_decode_workspace_size", "paged_decode_num_splits",
                          "paged_decode_balanced_parts",
                          "pkv_last_error"}
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in pkv.h but not exported"


def test_header_constants_parsed():
    assert B._C["PKV_OK"] == 0 and B._C["PKV_E_HIP"] == -6
    assert B.PKV_F_ASSUME_CONTIGUOUS == 1 and B.PKV_F_NO_CONTIG_DETECT == 2
    assert B.PKV_F_BALANCED == 4
    assert B.PKV_MAX_SPLITS == 64


FAKE = 0x100000  # a 16-byte-aligned non-null value: only ever seen by host checks


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, num_pages=8, page_size=16, H_kv=2, D=128, pt=FAKE,
             num_slots=3, max_blocks=4, bi=FAKE, kl=FAKE, batch=2, H_q=4, scale=0.125,
             max_kv_len=64, splits=1, flags=0, ws=0, ws_bytes=0, out=FAKE, lse=FAKE, stream=0)
    a.update(kw)
    return lib.paged_decode_attn(a["q"], a["k"], a["v"], a["num_pages"], a["page_size"], a["H_kv"],
                                 a["D"], a["pt"], a["num_slots"], a["max_blocks"], a["bi"], a["kl"],
                                 a["batch"], a["H_q"], a["scale"], a["max_kv_len"], a["splits"],
                                 a["flags"], a["ws"], a["ws_bytes"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=96), -2, "head_dim"),
    (dict(page_size=24), -2, "page_size"),
    (dict(page_size=8), -2, "page_size"),
    (dict(H_q=5), -2, "multiple"),
    (dict(H_q=34, H_kv=2), -2, "16 query heads"),
    (dict(batch=-1), -2, "batch"),
    (dict(num_pages=0), -2, "num_pages"),
    (dict(max_blocks=0), -2, "max_blocks"),
    (dict(scale=float("nan")), -2, "scale"),
    (dict(scale=-0.125), -2, "scale"),
    (dict(scale=0.0), -2, "scale"),
    (dict(splits=65), -5, "num_splits"),
    (dict(splits=-1), -5, "num_splits"),
    (dict(flags=8), -2, "flag"),
    (dict(q=0), -1, "NULL"),
    (dict(lse=0), -1, "NULL"),
    (dict(q=FAKE + 2), -3, "aligned"),
    (dict(out=FAKE + 8), -3, "aligned"),
    (dict(kl=FAKE + 2), -3, "aligned"),
    (dict(splits=2), -4, "workspace"),
    (dict(splits=2, flags=4), -5, "num_splits"),
    (dict(splits=0, flags=4), -4, "workspace"),
    (dict(splits=0, max_kv_len=4096, max_blocks=300), -4, "balanced"),   # automatic, long context
    (dict(splits=0, batch=128, H_kv=8, H_q=32), -4, "balanced"),        # automatic, 4 units per CU
    (dict(splits=2, ws=FAKE, ws_bytes=100), -4, "workspace"),
    (dict(splits=2, ws=FAKE + 4, ws_bytes=1 << 20), -3, "workspace"),
])
def test_decode_rejects(lib, kw, code, msg):
    rc = _decode(lib, **kw)
    assert rc == code, (rc, B.last_error())
    assert msg in B.last_error()


def _fused(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, num_pages=8, page_size=16, H_kv=2, D=128,
             pt=FAKE, num_slots=3, max_blocks=4, bi=FAKE, kl=FAKE, batch=2, H_q=4, scale=0.125,
             max_kv_len=64, splits=1, flags=0, ws=0, ws_bytes=0, out=FAKE, lse=FAKE, stream=0)
    a.update(kw)
    return lib.paged_decode_attn_append(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["num_pages"],
                                        a["page_size"], a["H_kv"], a["D"], a["pt"],
                                        a["num_slots"], a["max_blocks"], a["bi"], a["kl"],
                                        a["batch"], a["H_q"], a["scale"], a["max_kv_len"],
                                        a["splits"], a["flags"], a["ws"], a["ws_bytes"], a["out"],
                                        a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(kn=0), -1, "NULL"),
    (dict(vn=0), -1, "NULL"),
    (dict(kn=FAKE + 2), -3, "aligned"),
    (dict(vn=FAKE + 8), -3, "aligned"),
    (dict(D=96), -2, "head_dim"),
    (dict(splits=2), -4, "workspace"),
])
def test_fused_rejects(lib, kw, code, msg):
    rc = _fused(lib, **kw)
    assert rc == code, (rc, B.last_error())
    assert msg in B.last_error()
    if code != -2:
        assert "paged_decode_attn_append" in B.last_error()


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, batch=0, q=0, k=0, v=0, pt=0, bi=0, kl=0, out=0, lse=0) == 0


def test_append_checks(lib):
    f = lib.paged_kv_append
    assert f(0, 0, 8, 16, 2, 128, 0, 3, 4, 0, 0, 0, 0, 0, 0) == 0          # no tokens: no-op
    assert f(FAKE, FAKE, 8, 16, 2, 128, FAKE, 3, 4, FAKE, FAKE, -1, FAKE, FAKE, 0) == -2
    assert f(FAKE, FAKE, 8, 12, 2, 128, FAKE, 3, 4, FAKE, FAKE, 1, FAKE, FAKE, 0) == -2
    assert f(FAKE, 0, 8, 16, 2, 128, FAKE, 3, 4, FAKE, FAKE, 1, FAKE, FAKE, 0) == -1
    assert f(FAKE, FAKE, 8, 16, 2, 128, FAKE, 3, 4, FAKE, FAKE, 1, FAKE + 2, FAKE, 0) == -3
    assert f(FAKE, FAKE, 8, 16, 2, 100, FAKE, 3, 4, FAKE, FAKE, 1, FAKE, FAKE, 0) == -2
    assert "head_dim" in B.last_error()


def test_prefill_checks(lib):
    f = lib.packed_prefill_attn
    assert f(0, 0, 0, 0, 0, 0, 32, 8, 128, 0.1, 0, 0, 0) == 0               # empty: no-op
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 10, 32, 8, 96, 0.1, FAKE, FAKE, 0) == -2      # head_dim
    assert "head_dim" in B.last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 10, 30, 8, 128, 0.1, FAKE, FAKE, 0) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 10, 32, 8, 128, 0.1, FAKE, FAKE, 0) == -2
    assert f(FAKE, 0, FAKE, FAKE, 1, 10, 32, 8, 128, 0.1, FAKE, FAKE, 0) == -1
    assert f(FAKE, FAKE, FAKE, FAKE + 1, 1, 10, 32, 8, 128, 0.1, FAKE, FAKE, 0) == -3
    assert f(FAKE, FAKE, FAKE, FAKE, 1, -5, 32, 8, 128, 0.1, FAKE, FAKE, 0) == -2
    # one token's K row (num_kv_heads*head_dim*2 bytes) must stay below 2^24
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 10, 65536, 65536, 128, 0.1, FAKE, FAKE, 0) == -2
    assert "2^24" in B.last_error()
    # a grid of more than 2^32 workgroups (tiles of 8 rows at 16 query heads per KV head)
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2**31 - 1, 512, 32, 128, 0.1, FAKE, FAKE, 0) == -2
    assert "2^32 workgroups" in B.last_error()


def test_validate_checks(lib):
    """The debug validation calls reject bad shapes and pointers on the host."""
    f = lib.pkv_validate_decode
    assert f(FAKE, 8, 16, 3, 4, FAKE, FAKE, -1, FAKE, 0) == -2                  # batch < 0
    assert f(FAKE, 8, 24, 3, 4, FAKE, FAKE, 2, FAKE, 0) == -2                   # page_size
    assert f(FAKE, 0, 16, 3, 4, FAKE, FAKE, 2, FAKE, 0) == -2                   # num_pages
    assert f(FAKE, 8, 16, 3, 4, FAKE, FAKE, 2, 0, 0) == -1                      # report
    assert f(0, 8, 16, 3, 4, FAKE, FAKE, 2, FAKE, 0) == -1                      # page_table
    assert f(FAKE, 8, 16, 3, 4, FAKE + 2, FAKE, 2, FAKE, 0) == -3               # alignment
    g = lib.pkv_validate_prefill
    assert g(FAKE, -1, 10, 0, 0, 0, 1, 16, 1, 1, FAKE, 0) == -2                 # num_docs < 0
    assert g(0, 1, 10, 0, 0, 0, 1, 16, 1, 1, FAKE, 0) == -1                     # cu_seqlens
    assert g(FAKE, 1, 10, 0, FAKE, 0, 1, 16, 1, 1, FAKE, 0) == -1               # prefix w/o slots
    assert g(FAKE, 1, 10, FAKE, 0, 0, 8, 16, 3, 4, FAKE, 0) == -1               # slots w/o table
    assert g(FAKE, 1, 10, FAKE, 0, FAKE, 8, 20, 3, 4, FAKE, 0) == -2            # page_size
    assert g(FAKE + 1, 1, 10, 0, 0, 0, 1, 16, 1, 1, FAKE, 0) == -3              # alignment
    assert "pkv_validate_prefill" in B.last_error()
    assert B._C["PKV_V_SLOT"] == 1 and B._C["PKV_V_BOUNDS"] == 5


def test_workspace_size(lib):
    ws = lib.paged_decode_workspace_size
    assert ws(4, 32, 8, 128, 1, 0) == 0
    rows = 3 * 2 * 4
    o_bytes = (rows * 128 * 4 + 255) // 256 * 256
    assert ws(2, 4, 2, 128, 3, 0) == o_bytes + rows * 4
    assert ws(0, 4, 2, 128, 3, 0) == 0
    assert ws(2, 5, 2, 128, 3, 0) == 0                 # H_q not a multiple of H_kv
    # balanced: partials for 2 slots per (KV head, workgroup), independent of the batch
    w8 = lib.paged_decode_balanced_parts(100000, 8, 1 << 20)      # the cap: 2*CUs/H_kv
    assert w8 >= 1
    b = ws(64, 32, 8, 128, 0, 4)
    assert b == ws(7, 32, 8, 128, 0, 4) > 0
    rows = 8 * w8 * 2 * 4
    assert b == (rows * 128 * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256 + 8 * w8 * 16
    # automatic: covers the largest per-row split count the heuristic can pick and the
    # balanced schedule, which it takes for long contexts
    s_max = lib.paged_decode_num_splits(2, 2, 1 << 30)
    rows = s_max * 2 * 4
    per_row = (rows * 128 * 4 + 255) // 256 * 256 + rows * 4
    assert ws(2, 4, 2, 128, 0, 0) == max(per_row, ws(2, 4, 2, 128, 0, 4))
    assert ws(512, 32, 8, 128, 0, 0) == ws(512, 32, 8, 128, 0, 4)  # single pass, or balanced


def test_auto_splits(lib):
    ns = lib.paged_decode_num_splits
    assert ns(64, 8, 1024) == 1                        # 512 units fill the chip
    assert ns(8, 8, 1536) == min(1536 // 256, round(256 / 64))
    assert ns(1, 1, 100) == 1                          # too short to split
    assert 1 <= ns(1, 1, 1 << 20) <= 64


def test_balanced_parts(lib):
    bp = lib.paged_decode_balanced_parts
    wmax = bp(100000, 8, 1 << 20)
    assert bp(100000, 1, 1 << 20) == min(8 * wmax, 4096)
    assert bp(3, 2, 100) == 3                        # at least one workgroup per row
    assert bp(1, 2, 5000) == -(-157 // 4)            # 157 tiles, four per workgroup
    assert bp(64, 8, 1024) == wmax                   # enough tiles: the cap
    assert bp(0, 8, 1024) == 1


def test_graph_buckets():
    """Bucket list of the graph runner: 1, 2, 4, 8, then multiples of 16, then max_batch."""
    from paged_kv_attention_23_amd.graphs import default_buckets
    assert default_buckets(64) == [1, 2, 4, 8, 16, 32, 48, 64]
    assert default_buckets(50) == [1, 2, 4, 8, 16, 32, 48, 50]
    assert default_buckets(3) == [1, 2, 3]


def test_noalloc_host_checks(lib):
    """paged_decode_attn_noalloc: an empty batch is a no-op, a plan whose partials exceed
    the fixed scratch is refused before any HIP call, and bad shapes fail as in
    paged_decode_attn."""
    f = lib.paged_decode_attn_noalloc

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, num_pages=8, page_size=16, H_kv=8, D=128, pt=FAKE,
                 num_slots=3, max_blocks=4, bi=FAKE, kl=FAKE, batch=2, H_q=32, scale=0.125,
                 max_kv_len=64, splits=1, flags=0, out=FAKE, lse=FAKE, stream=0)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["num_pages"], a["page_size"], a["H_kv"], a["D"],
                 a["pt"], a["num_slots"], a["max_blocks"], a["bi"], a["kl"], a["batch"], a["H_q"],
                 a["scale"], a["max_kv_len"], a["splits"], a["flags"], a["out"], a["lse"],
                 a["stream"])

    assert call(batch=0, q=0, k=0, v=0, pt=0, bi=0, kl=0, out=0, lse=0) == 0
    rc = call(batch=4096, splits=64)  # 64 * 4096 * 32 * 129 * 4 bytes of partials
    assert rc == B._C["PKV_E_WORKSPACE"], (rc, B.last_error())
    assert "scratch" in B.last_error() and "paged_decode_attn_noalloc" in B.last_error()
    assert call(D=96) == -2
    assert call(splits=65) == B._C["PKV_E_SPLITS"]
