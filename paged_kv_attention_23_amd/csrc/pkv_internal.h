// Host-side launch interfaces between the C ABI (pkv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
  uint16_t *k_pool, *v_pool;       // [H_kv][num_pages*page_size][D]
  const int32_t *page_table;       // [num_slots][max_blocks]
  const int32_t *batch_idx, *input_pos;  // [num_tokens]
  const uint16_t *k_new, *v_new;   // [num_tokens][H_kv][D]
  int64_t plane_rows;              // num_pages * page_size
  int32_t num_pages, page_shift, num_slots, max_blocks;
  int32_t num_tokens, H_kv, D;
};

struct DecodeArgs {
  const uint16_t *q;               // [B][H_q][D]
  const uint16_t *k_pool, *v_pool; // [H_kv][plane_rows][D]
  const int32_t *page_table;       // [num_slots][max_blocks]
  const int32_t *batch_idx, *kv_len;  // [B]
  int64_t plane_rows;
  int32_t num_pages, page_shift, num_slots, max_blocks;
  int32_t B, H_q, H_kv, G, D;
  float scale_log2;                // scale * log2(e)
  int32_t balanced;                // 1: balanced schedule, 0: per-row splits
  int32_t num_splits;              // per-row: splits per row; balanced: workgroups per KV head (W)
  int32_t contig_mode;             // 0 detect per row, 1 assume contiguous, 2 never
  int32_t stream_nt;               // per-row schedule: non-temporal K/V loads
  // Partials.  Per-row: [S][B][H_q][D] and [S][B][H_q].  Balanced: [H_kv][W][2][G][D],
  // [H_kv][W][2][G] and one descriptor per (KV head, workgroup) in desc.
  float *o_part, *lse_part;
  int4 *desc;
  uint16_t *out;                   // [B][H_q][D] bf16
  float *lse;                      // [B][H_q]
  // Fused append (paged_decode_attn_append): each live row's new token, at
  // position kv_len - 1, comes from k_new/v_new [B][H_kv][D] and is written
  // into the pools through k_pool_w/v_pool_w.  All NULL for plain decode.
  const uint16_t *k_new, *v_new;
  uint16_t *k_pool_w, *v_pool_w;
};

struct PrefillArgs {
  const uint16_t *q;               // [L][H_q][D]
  const uint16_t *k, *v;           // [L][H_kv][D]
  const int32_t *cu_seqlens;       // [num_docs+1]
  int32_t num_docs, L, H_q, H_kv, G;
  float scale_log2;
  uint16_t *out;                   // [L][H_q][D]
  float *lse;                      // [L][H_q]
  // Fused scatter (packed_prefill_attn_append): token j of document d goes to
  // slot doc_slots[d], position j of the paged pools.  k_pool NULL: none.
  uint16_t *k_pool, *v_pool;       // [H_kv][plane_rows][D]
  const int32_t *page_table;       // [num_slots][max_blocks]
  const int32_t *doc_slots;        // [num_docs]
  const int32_t *prefix_lens;      // [num_docs] cached tokens before each chunk; NULL: none
  int64_t plane_rows;
  int32_t num_pages, page_shift, num_slots, max_blocks;
  int32_t D;                       // head_dim: 64 or 128
};

// Debug checks (pkv_validate_decode / pkv_validate_prefill).  Decode: rows
// r < batch with batch_idx/kv_len.  Prefill (cu_seqlens non-NULL): documents
// d < batch, with doc_slots and prefix_lens optional (NULL).
struct ValidateArgs {
  const int32_t *page_table;       // [num_slots][max_blocks], or NULL when no page is checked
  const int32_t *batch_idx, *kv_len;
  const int32_t *cu_seqlens, *doc_slots, *prefix_lens;
  int32_t batch, total_len;
  int32_t num_pages, page_shift, num_slots, max_blocks;
  int32_t *report;                 // [4]: count, first index, code, block
};

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t stream);
hipError_t launch_validate(const ValidateArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

}  // namespace pkv
