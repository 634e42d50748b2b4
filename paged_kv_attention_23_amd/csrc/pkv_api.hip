// C ABI of libpkv.so (declared in include/pkv.h): argument checks, split
// planning and kernel dispatch.  Every check runs on the host before any HIP
// call, so the error paths work (and are tested) without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int log2_exact(int32_t v) {  // log2 of a power of two, else -1
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) != v) ++s;
  return s;
}

int check_pool(int32_t num_pages, int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
               int32_t num_slots, int32_t max_blocks) {
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_SHAPE, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (num_kv_heads <= 0) return fail(PKV_E_SHAPE, "num_kv_heads must be positive (got %d)", num_kv_heads);
  if (log2_exact(page_size) < 4 || page_size > (1 << 20))
    return fail(PKV_E_SHAPE, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
  if (num_pages <= 0) return fail(PKV_E_SHAPE, "num_pages must be positive (got %d)", num_pages);
  if ((int64_t)num_pages * page_size > INT32_MAX)
    return fail(PKV_E_SHAPE, "num_pages*page_size exceeds 2^31-1 rows");
  if (num_slots <= 0 || max_blocks <= 0)
    return fail(PKV_E_SHAPE, "num_slots and max_blocks must be positive (got %d, %d)", num_slots,
                max_blocks);
  if ((int64_t)max_blocks * page_size > INT32_MAX)
    return fail(PKV_E_SHAPE, "max_blocks*page_size exceeds 2^31-1 keys");
  if ((int64_t)num_pages * page_size * head_dim * 2 > (int64_t)UINT32_MAX)
    return fail(PKV_E_SHAPE, "one KV head plane (num_pages*page_size*head_dim*2 bytes) must be below 4 GiB");
  return PKV_OK;
}

int launch_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, cached per device id.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

constexpr int kMinSplitKeys = 256;
// Above this key bound the automatic choice uses the balanced schedule
// (measured: per-row wins up to 2048 keys, balanced from 2-4k keys on, and by
// 2-7x when one long row sits among short ones).
constexpr int32_t kAutoBalancedKeys = 2048;
// At or above this many (row, KV head) units per compute unit the automatic
// choice also uses the balanced schedule: rows of unequal length then leave
// some CUs with more keys than others, which the equal shares even out
// (measured at B=256 over 8 KV heads, contexts U[1024,2048]: 268 vs 281 us;
// at B=64, 400 units, the per-row schedule stays faster).
constexpr int64_t kAutoBalancedUnitsPerCu = 4;

// Per-row schedule, automatic split count.  One workgroup per (row, KV head)
// already fills the chip when there are at least as many units as compute
// units; splitting then only adds the merge pass.  Below that, split so that
// roughly one unit lands on every CU, keeping at least kMinSplitKeys keys per
// split.
int32_t auto_splits(int32_t batch, int32_t num_kv_heads, int32_t kv_bound, int cus) {
  const int64_t units = (int64_t)batch * num_kv_heads;
  if (units <= 0 || kv_bound <= 0 || units >= cus) return 1;
  int64_t s = (cus + units / 2) / units;
  const int64_t by_len = kv_bound / kMinSplitKeys;
  if (s > by_len) s = by_len;
  if (s > PKV_MAX_SPLITS) s = PKV_MAX_SPLITS;
  if (s < 1) s = 1;
  return (int32_t)s;
}

// Balanced schedule: workgroups per KV head.  Two decode workgroups fit on a
// compute unit, so 2*CUs workgroups in all fill the chip in one wave; fewer
// when the batch cannot give each at least a few tiles (four 32-key tiles, one
// per wave), but never fewer than one per row.
int32_t balanced_max_parts(int32_t num_kv_heads, int cus) {
  int64_t w = (2 * (int64_t)cus) / num_kv_heads;
  if (w > 4096) w = 4096;
  return (int32_t)(w < 1 ? 1 : w);
}

int32_t balanced_parts(int32_t batch, int32_t num_kv_heads, int32_t kv_bound, int cus) {
  const int64_t wmax = balanced_max_parts(num_kv_heads, cus);
  const int64_t tiles = (int64_t)batch * ((kv_bound + 31) / 32);
  int64_t w = (tiles + 3) / 4;
  if (w < batch) w = batch;
  if (w > wmax) w = wmax;
  return (int32_t)(w < 1 ? 1 : w);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The automatic choice (num_splits 0, no schedule flag) takes the balanced
// schedule for long contexts, where one long row would otherwise hold a few
// workgroups busy long after the rest of the batch is done, and for large
// batches, where rows of unequal length load the CUs unequally.
bool auto_balanced(int32_t batch, int32_t num_kv_heads, int32_t kv_bound) {
  return kv_bound > kAutoBalancedKeys ||
         (int64_t)batch * num_kv_heads >= kAutoBalancedUnitsPerCu * device_cus();
}

}  // namespace

extern "C" {

const char *pkv_last_error(void) { return g_err; }

// Shape checks of the page arguments shared by the two validation calls.
static int check_pages(const char *who, int32_t num_pages, int32_t page_size, int32_t num_slots,
                       int32_t max_blocks) {
  if (log2_exact(page_size) < 4 || page_size > (1 << 20))
    return fail(PKV_E_SHAPE, "%s: page_size must be a power of two in [16, 2^20] (got %d)", who,
                page_size);
  if (num_pages <= 0 || num_slots <= 0 || max_blocks <= 0)
    return fail(PKV_E_SHAPE, "%s: num_pages, num_slots and max_blocks must be positive (got %d, %d, %d)",
                who, num_pages, num_slots, max_blocks);
  return PKV_OK;
}

int pkv_validate_decode(const int32_t *page_table, int32_t num_pages, int32_t page_size,
                        int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                        const int32_t *kv_len, int32_t batch, int32_t *report, void *stream) {
  const char *who = "pkv_validate_decode";
  if (batch < 0) return fail(PKV_E_SHAPE, "%s: batch must be >= 0 (got %d)", who, batch);
  int rc = check_pages(who, num_pages, page_size, num_slots, max_blocks);
  if (rc) return rc;
  if (!report || (batch > 0 && (!page_table || !batch_idx || !kv_len)))
    return fail(PKV_E_NULL, "%s: a required pointer is NULL", who);
  if (!aligned4(report) || !aligned4(page_table) || !aligned4(batch_idx) || !aligned4(kv_len))
    return fail(PKV_E_ALIGN, "%s: int32 arrays must be 4-byte aligned", who);
  pkv::ValidateArgs a = {};
  a.page_table = page_table;
  a.batch_idx = batch_idx;
  a.kv_len = kv_len;
  a.batch = batch;
  a.num_pages = num_pages;
  a.page_shift = log2_exact(page_size);
  a.num_slots = num_slots;
  a.max_blocks = max_blocks;
  a.report = report;
  return launch_status(pkv::launch_validate(a, (hipStream_t)stream), who);
}

int pkv_validate_prefill(const int32_t *cu_seqlens, int32_t num_docs, int32_t total_len,
                         const int32_t *doc_slots, const int32_t *prefix_lens,
                         const int32_t *page_table, int32_t num_pages, int32_t page_size,
                         int32_t num_slots, int32_t max_blocks, int32_t *report, void *stream) {
  const char *who = "pkv_validate_prefill";
  if (num_docs < 0 || total_len < 0)
    return fail(PKV_E_SHAPE, "%s: num_docs and total_len must be >= 0 (got %d, %d)", who, num_docs,
                total_len);
  if (!cu_seqlens || !report) return fail(PKV_E_NULL, "%s: a required pointer is NULL", who);
  if (prefix_lens && !doc_slots)
    return fail(PKV_E_NULL, "%s: prefix_lens needs doc_slots", who);
  if (doc_slots) {
    int rc = check_pages(who, num_pages, page_size, num_slots, max_blocks);
    if (rc) return rc;
    if (!page_table) return fail(PKV_E_NULL, "%s: doc_slots needs page_table", who);
  }
  if (!aligned4(cu_seqlens) || !aligned4(report) || !aligned4(doc_slots) ||
      !aligned4(prefix_lens) || !aligned4(page_table))
    return fail(PKV_E_ALIGN, "%s: int32 arrays must be 4-byte aligned", who);
  pkv::ValidateArgs a = {};
  a.cu_seqlens = cu_seqlens;
  a.doc_slots = doc_slots;
  a.prefix_lens = prefix_lens;
  a.page_table = doc_slots ? page_table : nullptr;
  a.batch = num_docs;
  a.total_len = total_len;
  if (doc_slots) {
    a.num_pages = num_pages;
    a.page_shift = log2_exact(page_size);
    a.num_slots = num_slots;
    a.max_blocks = max_blocks;
  }
  a.report = report;
  return launch_status(pkv::launch_validate(a, (hipStream_t)stream), who);
}

int paged_kv_append(void *k_pool, void *v_pool, int32_t num_pages, int32_t page_size,
                    int32_t num_kv_heads, int32_t head_dim, const int32_t *page_table,
                    int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                    const int32_t *input_pos, int32_t num_tokens, const void *k_new,
                    const void *v_new, void *stream) {
  if (num_tokens < 0) return fail(PKV_E_SHAPE, "num_tokens must be >= 0 (got %d)", num_tokens);
  int rc = check_pool(num_pages, page_size, num_kv_heads, head_dim, num_slots, max_blocks);
  if (rc) return rc;
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !page_table || !batch_idx || !input_pos || !k_new || !v_new)
    return fail(PKV_E_NULL, "paged_kv_append: a required pointer is NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_E_ALIGN, "paged_kv_append: bf16 tensors must be 16-byte aligned");
  if (!aligned4(page_table) || !aligned4(batch_idx) || !aligned4(input_pos))
    return fail(PKV_E_ALIGN, "paged_kv_append: int32 tensors must be 4-byte aligned");
  pkv::AppendArgs a;
  a.k_pool = (uint16_t *)k_pool;
  a.v_pool = (uint16_t *)v_pool;
  a.page_table = page_table;
  a.batch_idx = batch_idx;
  a.input_pos = input_pos;
  a.k_new = (const uint16_t *)k_new;
  a.v_new = (const uint16_t *)v_new;
  a.plane_rows = (int64_t)num_pages * page_size;
  a.num_pages = num_pages;
  a.page_shift = log2_exact(page_size);
  a.num_slots = num_slots;
  a.max_blocks = max_blocks;
  a.num_tokens = num_tokens;
  a.H_kv = num_kv_heads;
  a.D = head_dim;
  return launch_status(pkv::launch_kv_append(a, (hipStream_t)stream), "paged_kv_append launch");
}

size_t paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t num_splits, uint32_t flags) {
  if (num_splits < 0 || batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const size_t parts = (size_t)num_kv_heads * balanced_max_parts(num_kv_heads, device_cus()) * 2;
  const size_t brows = parts * (size_t)(num_q_heads / num_kv_heads);
  const size_t balanced_bytes = align256(brows * (size_t)head_dim * sizeof(float)) +
                                align256(brows * sizeof(float)) + parts / 2 * 4 * sizeof(int32_t);
  if (flags & PKV_F_BALANCED) return balanced_bytes;
  // automatic: the largest count auto_splits can pick for this batch, whatever the lengths
  const int32_t S = num_splits ? num_splits : auto_splits(batch, num_kv_heads, INT32_MAX, device_cus());
  const size_t rows = (size_t)S * (size_t)batch * (size_t)num_q_heads;
  const size_t per_row_bytes =
      S <= 1 ? 0 : align256(rows * (size_t)head_dim * sizeof(float)) + rows * sizeof(float);
  // the automatic choice may also pick the balanced schedule (long contexts)
  return num_splits ? per_row_bytes : std::max(per_row_bytes, balanced_bytes);
}

int32_t paged_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len) {
  return auto_splits(batch, num_kv_heads, max_kv_len, device_cus());
}
int32_t paged_decode_auto_balanced(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len) {
  if (batch <= 0 || num_kv_heads <= 0 || max_kv_len <= 0) return 0;
  return auto_balanced(batch, num_kv_heads, max_kv_len) ? 1 : 0;
}

int32_t paged_decode_balanced_parts(int32_t batch, int32_t num_kv_heads, int32_t max_kv_len) {
  if (batch <= 0 || num_kv_heads <= 0) return 1;
  return balanced_parts(batch, num_kv_heads, max_kv_len > 0 ? max_kv_len : 1, device_cus());
}

// Scratch of paged_decode_attn_noalloc: the split partials and descriptors
// live in this fixed device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a stand-in, so its device address is taken
// once per device with hipGetSymbolAddress and used everywhere instead.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

static int scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PKV_E_SHAPE, "device %d is beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return PKV_OK;
}

static int decode_common(const char *who, const void *q, const void *k_new, const void *v_new,
                         const void *k_pool, const void *v_pool, bool fused, int32_t num_pages,
                         int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                         const int32_t *page_table, int32_t num_slots, int32_t max_blocks,
                         const int32_t *batch_idx, const int32_t *kv_len, int32_t batch,
                         int32_t num_q_heads, float scale, int32_t max_kv_len, int32_t num_splits,
                         uint32_t flags, void *workspace, size_t workspace_bytes, void *out,
                         float *lse, void *stream, bool noalloc = false) {
  if (batch < 0) return fail(PKV_E_SHAPE, "batch must be >= 0 (got %d)", batch);
  int rc = check_pool(num_pages, page_size, num_kv_heads, head_dim, num_slots, max_blocks);
  if (rc) return rc;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_E_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_E_SHAPE, "at most 16 query heads per KV head are supported (got %d)",
                num_q_heads / num_kv_heads);
  if (!(scale > 0.f) || isinf(scale)) return fail(PKV_E_SHAPE, "scale must be finite and positive");
  if (num_splits < 0 || num_splits > PKV_MAX_SPLITS)
    return fail(PKV_E_SPLITS, "num_splits must be in [0, %d] (got %d)", PKV_MAX_SPLITS, num_splits);
  if (flags & ~(uint32_t)(PKV_F_ASSUME_CONTIGUOUS | PKV_F_NO_CONTIG_DETECT | PKV_F_BALANCED))
    return fail(PKV_E_SHAPE, "unknown flag bits 0x%x", flags);
  if ((int64_t)batch * num_kv_heads * PKV_MAX_SPLITS > INT32_MAX)
    return fail(PKV_E_SHAPE, "batch*num_kv_heads too large (got %d*%d)", batch, num_kv_heads);
  if (batch == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !page_table || !batch_idx || !kv_len || !out || !lse ||
      (fused && (!k_new || !v_new)))
    return fail(PKV_E_NULL, "%s: a required pointer is NULL", who);
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      (fused && (!aligned16(k_new) || !aligned16(v_new))))
    return fail(PKV_E_ALIGN, "%s: bf16 tensors must be 16-byte aligned", who);
  if (!aligned4(page_table) || !aligned4(batch_idx) || !aligned4(kv_len) || !aligned4(lse))
    return fail(PKV_E_ALIGN, "%s: int32/fp32 tensors must be 4-byte aligned", who);

  const int32_t cap = max_blocks * page_size;
  const int32_t kv_bound = (max_kv_len <= 0 || max_kv_len > cap) ? cap : max_kv_len;
  if ((flags & PKV_F_BALANCED) && num_splits != 0)
    return fail(PKV_E_SPLITS, "PKV_F_BALANCED chooses its own split points: num_splits must be 0 (got %d)",
                num_splits);
  const bool balanced = (flags & PKV_F_BALANCED) != 0 ||
                        (num_splits == 0 && auto_balanced(batch, num_kv_heads, kv_bound));
  int32_t S;
  if (balanced) {
    S = balanced_parts(batch, num_kv_heads, kv_bound, device_cus());
    // The balanced plan forms products (tiles in the list) * (workgroups) in int64.
    if ((double)batch * ((cap + 31) / 32) * S > 4.0e18)
      return fail(PKV_E_SHAPE, "batch*max_blocks*page_size too large for the balanced schedule");
  } else {
    S = num_splits ? num_splits : auto_splits(batch, num_kv_heads, kv_bound, device_cus());
  }

  pkv::DecodeArgs a;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.desc = nullptr;
  if (S > 1) {
    const size_t need = paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                    balanced ? 0 : S, flags);
    if (noalloc) {  // partials in the fixed scratch instead of a caller workspace
      if (need > kNoAllocScratchBytes)
        return fail(PKV_E_WORKSPACE,
                    "%s: this plan needs %zu bytes of scratch, above the fixed maximum of %zu",
                    who, need, kNoAllocScratchBytes);
      int rc2 = scratch_address(&workspace);
      if (rc2) return rc2;
      workspace_bytes = kNoAllocScratchBytes;
    }
    if (!workspace || workspace_bytes < need)
      return fail(PKV_E_WORKSPACE, "%s: %s needs %zu workspace bytes (got %zu%s)", who,
                  balanced ? "the balanced schedule" : "this split count", need, workspace_bytes,
                  workspace ? "" : ", NULL");
    if (!aligned16(workspace))
      return fail(PKV_E_ALIGN, "%s: workspace must be 16-byte aligned", who);
    char *ws = (char *)workspace;
    if (balanced) {
      const size_t rows = (size_t)num_kv_heads *
                          balanced_max_parts(num_kv_heads, device_cus()) * 2 *
                          (size_t)(num_q_heads / num_kv_heads);
      a.o_part = (float *)ws;
      a.lse_part = (float *)(ws + align256(rows * head_dim * sizeof(float)));
      a.desc = (int4 *)(ws + align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float)));
    } else {
      const size_t rows = (size_t)S * batch * num_q_heads;
      a.o_part = (float *)ws;
      a.lse_part = (float *)(ws + align256(rows * head_dim * sizeof(float)));
    }
  }
  a.q = (const uint16_t *)q;
  a.k_pool = (const uint16_t *)k_pool;
  a.v_pool = (const uint16_t *)v_pool;
  a.page_table = page_table;
  a.batch_idx = batch_idx;
  a.kv_len = kv_len;
  a.plane_rows = (int64_t)num_pages * page_size;
  a.num_pages = num_pages;
  a.page_shift = log2_exact(page_size);
  a.num_slots = num_slots;
  a.max_blocks = max_blocks;
  a.B = batch;
  a.H_q = num_q_heads;
  a.H_kv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.D = head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.balanced = (balanced && S > 1) ? 1 : 0;
  // Non-temporal K/V loads when the (row, KV head) units fill the chip
  // (measured: B=256 286 -> 267 us; at B=8 they cost 13.0 -> 13.6 us).
  a.stream_nt = ((int64_t)batch * num_kv_heads >= device_cus()) ? 1 : 0;
  a.num_splits = S;
  a.contig_mode = (flags & PKV_F_NO_CONTIG_DETECT) ? 2 : (flags & PKV_F_ASSUME_CONTIGUOUS) ? 1 : 0;
  a.out = (uint16_t *)out;
  a.lse = lse;
  a.k_new = fused ? (const uint16_t *)k_new : nullptr;
  a.v_new = fused ? (const uint16_t *)v_new : nullptr;
  a.k_pool_w = fused ? (uint16_t *)k_pool : nullptr;
  a.v_pool_w = fused ? (uint16_t *)v_pool : nullptr;
  return launch_status(pkv::launch_decode(a, (hipStream_t)stream), who);
}

int paged_decode_attn(const void *q, const void *k_pool, const void *v_pool, int32_t num_pages,
                      int32_t page_size, int32_t num_kv_heads, int32_t head_dim,
                      const int32_t *page_table, int32_t num_slots, int32_t max_blocks,
                      const int32_t *batch_idx, const int32_t *kv_len, int32_t batch,
                      int32_t num_q_heads, float scale, int32_t max_kv_len, int32_t num_splits,
                      uint32_t flags, void *workspace, size_t workspace_bytes, void *out,
                      float *lse, void *stream) {
  return decode_common("paged_decode_attn", q, nullptr, nullptr, k_pool, v_pool, false, num_pages,
                       page_size, num_kv_heads, head_dim, page_table, num_slots, max_blocks,
                       batch_idx, kv_len, batch, num_q_heads, scale, max_kv_len, num_splits, flags,
                       workspace, workspace_bytes, out, lse, stream);
}

int paged_decode_attn_noalloc(const void *q, const void *k_pool, const void *v_pool,
                              int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                              int32_t head_dim, const int32_t *page_table, int32_t num_slots,
                              int32_t max_blocks, const int32_t *batch_idx, const int32_t *kv_len,
                              int32_t batch, int32_t num_q_heads, float scale, int32_t max_kv_len,
                              int32_t num_splits, uint32_t flags, void *out, float *lse,
                              void *stream) {
  return decode_common("paged_decode_attn_noalloc", q, nullptr, nullptr, k_pool, v_pool, false,
                       num_pages, page_size, num_kv_heads, head_dim, page_table, num_slots,
                       max_blocks, batch_idx, kv_len, batch, num_q_heads, scale, max_kv_len,
                       num_splits, flags, nullptr, 0, out, lse, stream, true);
}

int paged_decode_attn_append(const void *q, const void *k_new, const void *v_new, void *k_pool,
                             void *v_pool, int32_t num_pages, int32_t page_size,
                             int32_t num_kv_heads, int32_t head_dim, const int32_t *page_table,
                             int32_t num_slots, int32_t max_blocks, const int32_t *batch_idx,
                             const int32_t *kv_len, int32_t batch, int32_t num_q_heads,
                             float scale, int32_t max_kv_len, int32_t num_splits, uint32_t flags,
                             void *workspace, size_t workspace_bytes, void *out, float *lse,
                             void *stream) {
  return decode_common("paged_decode_attn_append", q, k_new, v_new, k_pool, v_pool, true,
                       num_pages, page_size, num_kv_heads, head_dim, page_table, num_slots,
                       max_blocks, batch_idx, kv_len, batch, num_q_heads, scale, max_kv_len,
                       num_splits, flags, workspace, workspace_bytes, out, lse, stream);
}

static int prefill_common(const char *who, const void *q, const void *k, const void *v,
                          const int32_t *cu_seqlens, int32_t num_docs, int32_t total_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                          void *out, float *lse, bool fused, void *k_pool, void *v_pool,
                          int32_t num_pages, int32_t page_size, const int32_t *page_table,
                          int32_t num_slots, int32_t max_blocks, const int32_t *doc_slots,
                          const int32_t *prefix_lens, void *stream) {
  if (total_len < 0 || num_docs < 0)
    return fail(PKV_E_SHAPE, "total_len and num_docs must be >= 0 (got %d, %d)", total_len, num_docs);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_SHAPE, "%s: head_dim must be 64 or 128 (got %d)", who, head_dim);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_E_SHAPE, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_E_SHAPE, "at most 16 query heads per KV head are supported (got %d)",
                num_q_heads / num_kv_heads);
  if (!(scale > 0.f) || isinf(scale)) return fail(PKV_E_SHAPE, "scale must be finite and positive");
  if ((int64_t)num_kv_heads * head_dim * 2 >= (1 << 24))  // one token's K row in bytes, a 24-bit product
    return fail(PKV_E_SHAPE, "%s: num_kv_heads*head_dim*2 must be below 2^24 (got %d heads)", who,
                num_kv_heads);
  // One workgroup per (query tile, KV head); a tile holds at least 8 rows.
  if (((int64_t)total_len + 7) / 8 + num_docs > (int64_t)UINT32_MAX / num_kv_heads)
    return fail(PKV_E_SHAPE, "%s: total_len %d with %d KV heads needs more than 2^32 workgroups",
                who, total_len, num_kv_heads);
  if (fused) {
    int rc = check_pool(num_pages, page_size, num_kv_heads, head_dim, num_slots, max_blocks);
    if (rc) return rc;
  }
  if (total_len == 0) return PKV_OK;
  if (num_docs == 0) return fail(PKV_E_SHAPE, "total_len > 0 needs at least one document");
  if (!q || !k || !v || !cu_seqlens || !out || !lse ||
      (fused && (!k_pool || !v_pool || !page_table || !doc_slots)) ||
      (prefix_lens && !fused))
    return fail(PKV_E_NULL, "%s: a required pointer is NULL", who);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (fused && (!aligned16(k_pool) || !aligned16(v_pool))))
    return fail(PKV_E_ALIGN, "%s: bf16 tensors must be 16-byte aligned", who);
  if (!aligned4(cu_seqlens) || !aligned4(lse) ||
      (fused && (!aligned4(page_table) || !aligned4(doc_slots))) ||
      (prefix_lens && !aligned4(prefix_lens)))
    return fail(PKV_E_ALIGN, "%s: int32/fp32 tensors must be 4-byte aligned", who);
  pkv::PrefillArgs a;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.cu_seqlens = cu_seqlens;
  a.num_docs = num_docs;
  a.L = total_len;
  a.H_q = num_q_heads;
  a.H_kv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.D = head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.out = (uint16_t *)out;
  a.lse = lse;
  a.k_pool = fused ? (uint16_t *)k_pool : nullptr;
  a.v_pool = fused ? (uint16_t *)v_pool : nullptr;
  a.page_table = fused ? page_table : nullptr;
  a.doc_slots = fused ? doc_slots : nullptr;
  a.prefix_lens = fused ? prefix_lens : nullptr;
  a.plane_rows = fused ? (int64_t)num_pages * page_size : 0;
  a.num_pages = num_pages;
  a.page_shift = fused ? log2_exact(page_size) : 0;
  a.num_slots = num_slots;
  a.max_blocks = max_blocks;
  return launch_status(pkv::launch_prefill(a, (hipStream_t)stream), who);
}

int packed_prefill_attn(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                        int32_t num_docs, int32_t total_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale, void *out,
                        float *lse, void *stream) {
  return prefill_common("packed_prefill_attn", q, k, v, cu_seqlens, num_docs, total_len,
                        num_q_heads, num_kv_heads, head_dim, scale, out, lse, false, nullptr,
                        nullptr, 0, 0, nullptr, 0, 0, nullptr, nullptr, stream);
}

int packed_prefill_attn_append(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, int32_t num_docs, int32_t total_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float scale, void *out, float *lse, void *k_pool, void *v_pool,
                               int32_t num_pages, int32_t page_size, const int32_t *page_table,
                               int32_t num_slots, int32_t max_blocks, const int32_t *doc_slots,
                               void *stream) {
  return prefill_common("packed_prefill_attn_append", q, k, v, cu_seqlens, num_docs, total_len,
                        num_q_heads, num_kv_heads, head_dim, scale, out, lse, true, k_pool, v_pool,
                        num_pages, page_size, page_table, num_slots, max_blocks, doc_slots,
                        nullptr, stream);
}

int paged_prefill_attn(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                       const int32_t *prefix_lens, const int32_t *doc_slots, int32_t num_docs,
                       int32_t total_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, float scale, void *k_pool, void *v_pool,
                       int32_t num_pages, int32_t page_size, const int32_t *page_table,
                       int32_t num_slots, int32_t max_blocks, void *out, float *lse,
                       void *stream) {
  if (total_len > 0 && !prefix_lens)
    return fail(PKV_E_NULL, "paged_prefill_attn: a required pointer is NULL");
  return prefill_common("paged_prefill_attn", q, k, v, cu_seqlens, num_docs, total_len,
                        num_q_heads, num_kv_heads, head_dim, scale, out, lse, true, k_pool, v_pool,
                        num_pages, page_size, page_table, num_slots, max_blocks, doc_slots,
                        prefix_lens, stream);
}

}  // extern "C"
