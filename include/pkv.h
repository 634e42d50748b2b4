/*
 * pkv.h - grouped-query attention over a paged KV cache on AMD MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Every tensor argument is a plain DEVICE pointer owned by
 * the caller; the library allocates no memory, keeps no state between calls
 * (apart from a cached device-property query, and the fixed scratch array of
 * paged_decode_attn_noalloc), never synchronises, and only
 * enqueues work on the HIP stream passed in `stream` (a hipStream_t; NULL is
 * the default stream).  bf16 tensors are raw bfloat16 bit patterns, densely
 * packed (row-major, innermost dimension contiguous), 16-byte aligned.
 *
 * Cache format (flex paged-attention commit page, "Why this works", points
 * 1 and 3): one pool per K and per V of shape
 *     [num_kv_heads][num_pages * page_size][head_dim]   (bf16)
 * and a page table [num_slots][max_blocks] (int32) mapping (batch slot,
 * logical block) to a physical page.  Batch slot 0 and page 0 are reserved
 * padding: a row in slot 0 has no valid key.
 *
 * Error behaviour: every entry point returns PKV_OK (0) once its kernels are
 * enqueued, or a negative PKV_E* code, with a message in pkv_last_error().
 * All argument checks are host-side and happen before any HIP call.  Values
 * that live in device memory (page ids, slots, lengths, positions) are not
 * checked by the host; the kernels clamp them so that no access leaves the
 * buffers described by the size arguments, and results for out-of-contract
 * values are unspecified.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_E_NULL (-1)      /* a required pointer is NULL */
#define PKV_E_SHAPE (-2)     /* a size argument is out of range or inconsistent */
#define PKV_E_ALIGN (-3)     /* a bf16 tensor pointer is not 16-byte aligned */
#define PKV_E_WORKSPACE (-4) /* workspace missing or smaller than required */
#define PKV_E_SPLITS (-5)    /* num_splits out of range */
#define PKV_E_HIP (-6)       /* a HIP launch failed; message has hipGetErrorString */

/* paged_decode_attn flags */
#define PKV_F_ASSUME_CONTIGUOUS (1u << 0) /* caller promises each row's pages are consecutive ids */
#define PKV_F_NO_CONTIG_DETECT (1u << 1)  /* always walk the page table block by block */
#define PKV_F_BALANCED (1u << 2)          /* balanced split points across rows (num_splits = 0) */

#define PKV_MAX_SPLITS 64

/*
 * paged_kv_append - write new tokens' K and V into their pages.
 *
 * Defined by the cache update that runs before attention in the attention
 * forward of the qwen3_flex_inference.py page (update(input_pos, k, v,
 * batch_idx)).  Token t (0 <= t < num_tokens) with slot s = batch_idx[t] and
 * logical position p = input_pos[t] is written, for every KV head h, to pool
 * row  page_table[s][p / page_size] * page_size + p % page_size.  The copy is
 * bit-exact.  A token is skipped (nothing written) when s == 0, when its
 * block maps to page 0, or when s, p / page_size or the page lies outside
 * [1, num_slots), [0, max_blocks), [1, num_pages).  Two tokens naming the same
 * (slot, position) in one call is undefined.
 *
 *   k_pool, v_pool   bf16 [num_kv_heads][num_pages*page_size][head_dim], written
 *   page_table       int32 [num_slots][max_blocks]
 *   batch_idx        int32 [num_tokens]
 *   input_pos        int32 [num_tokens]
 *   k_new, v_new     bf16 [num_tokens][num_kv_heads][head_dim]
 *
 * num_tokens == 0 is a valid no-op.  head_dim must be 64 or 128, page_size a
 * power of two >= 16.
 */
int paged_kv_append(void *k_pool, void *v_pool, int32_t num_pages, int32_t page_size,
                    int32_t num_kv_heads, int32_t head_dim, const int32_t *page_table,
                    int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                    const int32_t *input_pos, int32_t num_tokens, const void *k_new,
                    const void *v_new, void *stream);

/*
 * paged_decode_workspace_size - bytes of workspace paged_decode_attn needs
 * for these num_splits and flags (the same values as in the call).  For
 * num_splits == 0 without PKV_F_BALANCED it covers both automatic choices
 * (the largest per-row split count for this batch, and the balanced
 * schedule); with PKV_F_BALANCED it
 * depends on the shape and the current device's compute-unit count, not on
 * the batch or the context lengths.  0 when no workspace is needed or for
 * invalid shapes.  Host function.
 */
size_t paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t num_splits, uint32_t flags);

/*
 * paged_decode_num_splits - the per-row split count paged_decode_attn
 * chooses for num_splits == 0 (without PKV_F_BALANCED) on the current device
 * when that automatic choice is the per-row schedule (see
 * paged_decode_auto_balanced).  Host function.
 */
int32_t paged_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len);

/*
 * paged_decode_auto_balanced - 1 when paged_decode_attn with num_splits == 0
 * (and no PKV_F_BALANCED) takes the balanced schedule on the current device
 * for this batch and key bound max_kv_len: a key bound above 2048, or at
 * least 4 (row, KV head) units per compute unit; 0 when it takes the per-row
 * schedule, and for non-positive arguments.  A scheduling choice of this
 * library: the decode block mask of the qwen3_flex_inference.py page fixes
 * what is attended, not how the work is split.  Host function.
 */
int32_t paged_decode_auto_balanced(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len);

/*
 * paged_decode_balanced_parts - the number W of workgroups per KV head that
 * the balanced schedule (PKV_F_BALANCED) uses on the current device for this
 * batch and max_kv_len; W == 1 means a single pass with no merge.  Host
 * function.
 */
int32_t paged_decode_balanced_parts(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len);

/*
 * paged_decode_attn - one query token per row attends to its row's cached keys.
 *
 * Defined by the decode attention of the qwen3_flex_inference.py page: the
 * block mask's causal offset lets row r see logical keys 0..input_pos, so the
 * row has kv_len[r] = input_pos + 1 valid keys (the token just appended
 * included), reached through the page table; flex_attention runs with
 * scale and enable_gqa.  Query head h reads KV head h / (num_q_heads /
 * num_kv_heads).  For row r with slot s = batch_idx[r] and n = kv_len[r]:
 *     x_j   = scale * q[r][h] . K[s, j]           j < n
 *     O     = sum_j softmax(x)_j V[s, j]          (fp32 accumulation, bf16 result)
 *     LSE   = ln sum_j exp(x_j)                   (fp32)
 * A row with s == 0 or n == 0 (a padding row, flex_vs_vllm.md page, "What
 * broke correctness") returns O = +0.0 and LSE = -inf, never NaN.  Pool
 * bytes outside the row's valid keys never influence the result.
 *
 *   q            bf16 [batch][num_q_heads][head_dim]
 *   k_pool,v_pool bf16 [num_kv_heads][num_pages*page_size][head_dim]
 *   page_table   int32 [num_slots][max_blocks]
 *   batch_idx    int32 [batch]
 *   kv_len       int32 [batch]; values above max_blocks*page_size are clamped
 *   max_kv_len   host upper bound of kv_len used to plan the key splits (<= 0
 *                or above max_blocks*page_size means max_blocks*page_size); a
 *                loose bound costs speed, never correctness
 *   num_splits   split-K (flash-decoding; the pages leave the decode kernel's
 *                work split open, so the schedules are the library's own):
 *                0 = automatic: the balanced schedule below when the key
 *                    bound (max_kv_len, else max_blocks*page_size) is above
 *                    2048 (long or skewed contexts) or when batch *
 *                    num_kv_heads is at least 4 per compute unit (large
 *                    batches); otherwise the per-row schedule with
 *                    paged_decode_num_splits splits,
 *                1 = one workgroup per (row, KV head), single pass,
 *                2..PKV_MAX_SPLITS = each row's keys in that many equal parts,
 *                    merged by log-sum-exp in a second kernel.
 *                Must be 0 with PKV_F_BALANCED.
 *   flags        PKV_F_* above.  PKV_F_BALANCED selects the balanced schedule:
 *                for each KV head the 32-key tiles of all rows, row after row,
 *                are dealt in equal contiguous shares to W workgroups
 *                (paged_decode_balanced_parts), cutting rows where a share
 *                ends; cut rows leave fp32 partials that a second kernel
 *                merges.  Every workgroup then streams the same number of
 *                keys whatever the mix of context lengths (one long row among
 *                short ones is spread over the whole chip).
 *   workspace    device buffer of at least paged_decode_workspace_size(...)
 *                bytes for the same num_splits and flags (may be NULL when
 *                that size is 0); contents on entry do not matter and are
 *                left undefined
 *   out          bf16 [batch][num_q_heads][head_dim]
 *   lse          fp32 [batch][num_q_heads]
 *
 * Results are bitwise reproducible for identical inputs, schedule and device
 * (the balanced schedule's cut points depend on the compute-unit count).
 * batch == 0 is a valid no-op.  Requirements: head_dim 64 or 128,
 * num_q_heads a multiple of num_kv_heads with at most 16 query heads per
 * KV head, page_size a power of two >= 16, scale finite and > 0.
 */
int paged_decode_attn(const void *q, const void *k_pool, const void *v_pool, int32_t num_pages,
                      int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                      const int32_t *page_table, int32_t num_slots, int32_t max_blocks,
                      const int32_t *batch_idx, const int32_t *kv_len, int32_t batch,
                      int32_t num_q_heads, float scale, int32_t max_kv_len, int32_t num_splits,
                      uint32_t flags, void *workspace, size_t workspace_bytes, void *out,
                      float *lse, void *stream);

/*
 * paged_decode_attn_noalloc - paged_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Arguments, schedule choice and results are those of paged_decode_attn with
 * the same num_splits and flags; there is no workspace argument.  The split
 * partials and descriptors go to a fixed scratch array inside the library,
 * 16 MiB per GPU (held by each GPU the library runs on until the process
 * ends).  A plan whose paged_decode_workspace_size exceeds 16 MiB is rejected
 * with PKV_E_WORKSPACE before anything is launched; every automatic plan on
 * head_dim <= 128 with at most 16 query heads per KV head fits.  The call
 * allocates nothing: the scratch address is looked up once per device
 * (hipGetSymbolAddress, with that device current) on the first call on it
 * whose plan writes partials; a failed lookup returns PKV_E_HIP.
 * Nothing in the scratch needs clearing between calls (every partial a call
 * reads is written by that call).  All calls on one GPU share its scratch:
 * calls that overlap in time on one GPU (different streams, or host threads)
 * race and give undefined results; serialise them on one stream.
 */
int paged_decode_attn_noalloc(const void *q, const void *k_pool, const void *v_pool,
                              int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                              int32_t head_dim, const int32_t *page_table, int32_t num_slots,
                              int32_t max_blocks, const int32_t *batch_idx, const int32_t *kv_len,
                              int32_t batch, int32_t num_q_heads, float scale, int32_t max_kv_len,
                              int32_t num_splits, uint32_t flags, void *out, float *lse,
                              void *stream);

/*
 * paged_decode_attn_append - paged_kv_append of each row's new token
 * followed by paged_decode_attn, in one launch.
 *
 * The decode step of the attention forward on the qwen3_flex_inference.py
 * page updates the cache with the step's token, then attends over the cache
 * including it.  Here row r's new token, at logical position kv_len[r] - 1,
 * is k_new[r] / v_new[r] (bf16 [batch][num_kv_heads][head_dim]); kv_len
 * counts it.  The workgroup that owns that key attends to it straight from
 * k_new / v_new and writes it into its page, so no key is read back from the
 * pool in the same launch.  Equivalent to
 *     paged_kv_append(tokens = live rows, input_pos = kv_len - 1) ;
 *     paged_decode_attn(same arguments)
 * with these exact rules: padding rows (slot 0, kv_len <= 0) write nothing
 * and return (+0, -inf); a row whose kv_len exceeds max_blocks*page_size has
 * no new token in range, so nothing is written and the row attends to its
 * first max_blocks*page_size keys; the write is skipped (the token still
 * attended) when the token's block maps to page 0 or to no page of the pool.
 * The pool bytes written are bit-exact copies of k_new / v_new.  Other
 * arguments, the schedule and the workspace are as in paged_decode_attn;
 * k_pool and v_pool are written.
 */
int paged_decode_attn_append(const void *q, const void *k_new, const void *v_new, void *k_pool,
                             void *v_pool, int32_t num_pages, int32_t page_size,
                             int32_t num_kv_heads, int32_t head_dim, const int32_t *page_table,
                             int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                             const int32_t *kv_len, int32_t batch, int32_t num_q_heads,
                             float scale, int32_t max_kv_len, int32_t num_splits, uint32_t flags,
                             void *workspace, size_t workspace_bytes, void *out, float *lse,
                             void *stream);

/*
 * packed_prefill_attn - document-causal attention over packed prompts.
 *
 * Defined by the prefill of the qwen3_flex_inference.py page: prompts are
 * concatenated into one sequence and masked so that each token sees only
 * tokens of its own document up to itself; GQA and scale as in decode.
 * Documents are the row ranges [cu_seqlens[d], cu_seqlens[d+1]); row i of
 * document d attends to keys j in [cu_seqlens[d], i].  K and V are read from
 * the packed arrays (write them into pages separately with paged_kv_append).
 *
 *   q            bf16 [total_len][num_q_heads][head_dim]
 *   k, v         bf16 [total_len][num_kv_heads][head_dim]
 *   cu_seqlens   int32 [num_docs+1], device; cu[0] = 0, non-decreasing,
 *                cu[num_docs] = total_len (zero-length documents allowed)
 *   out          bf16 [total_len][num_q_heads][head_dim]
 *   lse          fp32 [total_len][num_q_heads] (natural log)
 *
 * total_len == 0 is a valid no-op.  Requirements: head_dim 64 or 128, num_q_heads a
 * multiple of num_kv_heads with at most 16 query heads per KV head, scale
 * finite and > 0, and (total_len/8 + num_docs) * num_kv_heads below 2^32 (one
 * workgroup per query tile and KV head).  A violation returns PKV_E_SHAPE.
 */
int packed_prefill_attn(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                        int32_t num_docs, int32_t total_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale, void *out,
                        float *lse, void *stream);

/*
 * packed_prefill_attn_append - packed_prefill_attn plus the scatter of every
 * document's K/V into its pages, in one launch.
 *
 * The prefill of the qwen3_flex_inference.py page fills the paged cache with
 * the prompts' K/V (the cache update of the attention forward) and attends
 * over the packed prompts.  Document d (rows [cu_seqlens[d], cu_seqlens[d+1]))
 * lives in batch slot doc_slots[d], token j of it at logical position j (no
 * cached prefix).  Equivalent to
 *     paged_kv_append(k_pool, v_pool, ..., batch_idx = slot of each token,
 *                     input_pos = position in its document, k, v) ;
 *     packed_prefill_attn(q, k, v, cu_seqlens, ...)
 * with paged_kv_append's skip rules (slot 0 or out of range, block past
 * max_blocks, page 0 or out of range: nothing written for that token).  The
 * workgroup holding a document's longest key range writes that document's
 * rows while it streams them through LDS, so the scatter reads no extra HBM.
 *
 *   q, k, v, cu_seqlens, out, lse as in packed_prefill_attn
 *   k_pool, v_pool   bf16 [num_kv_heads][num_pages*page_size][head_dim], written
 *   page_table       int32 [num_slots][max_blocks]
 *   doc_slots        int32 [num_docs], device
 *
 * Requirements: those of packed_prefill_attn and paged_kv_append.
 */
int packed_prefill_attn_append(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, int32_t num_docs, int32_t total_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float scale, void *out, float *lse, void *k_pool, void *v_pool,
                               int32_t num_pages, int32_t page_size, const int32_t *page_table,
                               int32_t num_slots, int32_t max_blocks, const int32_t *doc_slots,
                               void *stream);

/*
 * paged_prefill_attn - chunked prefill over a paged prefix.
 *
 * The results write-up (flex_vs_vllm.md, "What's left on the table") names
 * chunked prefill, where new prompt chunks are processed against sequences
 * whose earlier tokens are already cached, as the main remaining penalty for
 * large batches.  Document d is a chunk of n_d = cu_seqlens[d+1] -
 * cu_seqlens[d] new tokens (those rows of q, k, v) continuing the sequence in
 * batch slot doc_slots[d], whose first prefix_lens[d] tokens are already in
 * the pools.  Chunk token j has position prefix_lens[d] + j: it is written
 * into its page as paged_kv_append would, and it attends to positions
 * 0 .. prefix_lens[d] + j of its sequence (the cached prefix through the
 * page table, the chunk causally; GQA and scale as in decode).  Equivalent to
 *     paged_kv_append(chunk tokens at their positions) ;
 *     for every chunk row: paged_decode_attn with kv_len = position + 1
 * Rows of a document whose slot is 0 or not below num_slots return
 * (+0, -inf).  With every prefix 0 the result is packed_prefill_attn_append.
 *
 *   q                bf16 [total_len][num_q_heads][head_dim]
 *   k, v             bf16 [total_len][num_kv_heads][head_dim], the chunks' K/V
 *   cu_seqlens       int32 [num_docs+1] as in packed_prefill_attn
 *   prefix_lens      int32 [num_docs], device; clamped to [0, max_blocks*page_size]
 *   doc_slots        int32 [num_docs], device
 *   k_pool, v_pool   bf16 [num_kv_heads][num_pages*page_size][head_dim];
 *                    read (prefix) and written (chunk)
 *   page_table       int32 [num_slots][max_blocks]
 *   out, lse         as in packed_prefill_attn
 *
 * The pages of a sequence's positions 0 .. prefix + n_d - 1 must be mapped
 * (pages 1..num_pages-1) and lie within max_blocks*page_size; otherwise
 * results are unspecified (no access leaves the buffers).  Requirements:
 * those of packed_prefill_attn and paged_kv_append.
 */
int paged_prefill_attn(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                       const int32_t *prefix_lens, const int32_t *doc_slots, int32_t num_docs,
                       int32_t total_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, float scale, void *k_pool, void *v_pool,
                       int32_t num_pages, int32_t page_size, const int32_t *page_table,
                       int32_t num_slots, int32_t max_blocks, void *out, float *lse,
                       void *stream);

/* Violation codes written by pkv_validate_decode / pkv_validate_prefill. */
#define PKV_V_SLOT 1     /* batch slot outside [0, num_slots) */
#define PKV_V_LEN 2      /* negative kv_len or prefix length */
#define PKV_V_CAPACITY 3 /* a live row's keys exceed max_blocks*page_size */
#define PKV_V_PAGE 4     /* a page id of a live block outside [1, num_pages) */
#define PKV_V_BOUNDS 5   /* cu_seqlens not 0 at the start, decreasing, or not total_len at the end */

/*
 * pkv_validate_decode - debug check of the device-side inputs of
 * paged_decode_attn and paged_decode_attn_append.
 *
 * The attention kernels take these values on trust and clamp them so that no
 * access leaves the buffers (results for out-of-contract values are
 * unspecified); this call reports them instead.  It is meant for debug
 * builds and tests, not the serving loop.  Row r is checked for:
 *   batch_idx[r] in [0, num_slots)                               (PKV_V_SLOT)
 *   kv_len[r] >= 0                                               (PKV_V_LEN)
 * and, for a live row (batch_idx[r] > 0, kv_len[r] > 0), the conditions of
 * the decode step of the qwen3_flex_inference.py page (its valid keys are
 * positions 0 .. kv_len-1, mapped through the page table):
 *   kv_len[r] <= max_blocks * page_size                          (PKV_V_CAPACITY)
 *   page_table[batch_idx[r]][j] in [1, num_pages) for every block j holding
 *   a valid key (page 0 is the reserved padding page)            (PKV_V_PAGE)
 *
 *   page_table          int32 [num_slots][max_blocks], device
 *   batch_idx, kv_len   int32 [batch], device
 *   report              int32 [4], device, written (nothing needs clearing):
 *                       { number of violating rows, first violating row or -1,
 *                         its PKV_V_* code or 0, the block for PKV_V_PAGE or -1 }
 *
 * One small kernel is enqueued on `stream`; read `report` after it.  Shapes
 * follow paged_decode_attn (page_size a power of two >= 16); batch == 0
 * writes an empty report.
 */
int pkv_validate_decode(const int32_t *page_table, int32_t num_pages, int32_t page_size,
                        int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                        const int32_t *kv_len, int32_t batch, int32_t *report, void *stream);

/*
 * pkv_validate_prefill - debug check of the device-side inputs of
 * packed_prefill_attn, packed_prefill_attn_append and paged_prefill_attn.
 *
 * Document d (d < num_docs) is checked for:
 *   cu_seqlens[0] == 0, cu_seqlens[d+1] >= cu_seqlens[d],
 *   cu_seqlens[num_docs] == total_len                            (PKV_V_BOUNDS)
 * with doc_slots (NULL: not checked):
 *   doc_slots[d] in [0, num_slots)                               (PKV_V_SLOT)
 * with prefix_lens as well (NULL: no cached prefix), for paged_prefill_attn:
 *   prefix_lens[d] >= 0                                          (PKV_V_LEN)
 * and for a document in a slot > 0:
 *   prefix_lens[d] + n_d <= max_blocks * page_size               (PKV_V_CAPACITY)
 *   the page ids of the blocks holding the cached prefix lie in [1, num_pages)
 *   (the chunk's own rows are written with paged_kv_append's skip rules)
 *                                                                (PKV_V_PAGE)
 *
 *   cu_seqlens    int32 [num_docs+1], device
 *   doc_slots     int32 [num_docs], device, or NULL
 *   prefix_lens   int32 [num_docs], device, or NULL (needs doc_slots)
 *   page_table    int32 [num_slots][max_blocks], device; needed with doc_slots
 *   report        int32 [4] as in pkv_validate_decode, documents in place of rows
 *
 * Without doc_slots the page arguments are ignored.
 */
int pkv_validate_prefill(const int32_t *cu_seqlens, int32_t num_docs, int32_t total_len,
                         const int32_t *doc_slots, const int32_t *prefix_lens,
                         const int32_t *page_table, int32_t num_pages, int32_t page_size,
                         int32_t num_slots, int32_t max_blocks, int32_t *report, void *stream);

/* Text for the most recent non-zero status returned on this thread. */
const char *pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
