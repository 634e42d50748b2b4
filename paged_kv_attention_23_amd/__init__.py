"""GQA attention over a paged KV cache for AMD MI355X (gfx950).

Three operations, each a hand-written HIP kernel path behind the C ABI of
libpkv.so (include/pkv.h):

  paged_kv_append      scatter new tokens' K/V into their pages
  paged_decode_attn    one query token per row over its paged keys
                       (single pass, per-row or balanced split-K + merge,
                       contiguous-page fast path)
  paged_decode_attn_noalloc
                       paged_decode_attn for callers that cannot allocate:
                       split partials in a fixed per-GPU scratch array
  paged_decode_attn_append
                       the two above fused: each row's new token is
                       attended from registers and written into its page
  packed_prefill_attn  document-causal attention over packed prompts
  packed_prefill_attn_append
                       the prefill plus the scatter of the prompts' K/V
                       into their pages, in one launch
  paged_prefill_attn   chunked prefill: chunks attend to their sequence's
                       cached prefix (pages) and to themselves causally
  validate_decode, validate_prefill
                       debug checks of the device-side index inputs

This package is the thin Python binding: it marshals torch tensors into the
C calls and nothing else.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    PKV_F_ASSUME_CONTIGUOUS,
    PKV_F_BALANCED,
    PKV_F_NO_CONTIG_DETECT,
    PKV_MAX_SPLITS,
    last_error,
    load_library,
    packed_prefill_attn,
    packed_prefill_attn_append,
    paged_decode_attn,
    paged_decode_attn_append,
    paged_decode_attn_noalloc,
    paged_decode_auto_balanced,
    paged_decode_balanced_parts,
    paged_decode_num_splits,
    paged_decode_workspace_size,
    paged_kv_append,
    paged_prefill_attn,
    validate_decode,
    validate_prefill,
)
