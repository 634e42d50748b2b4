// KV append: scatter new tokens' K and V rows into their pages.
//
// The cache update of the attention forward on the qwen3_flex_inference.py
// page writes each new token through the page table before attention runs.
// A token's rows are 2 * H_kv * D/8 pieces of 16 bytes (K rows, then V
// rows).  A workgroup of 256 threads takes 256 / pieces tokens (one token,
// looping over its pieces, when a token has more), so a token's slot,
// position and page are loaded once per token and the index arithmetic stays
// in 32 bits; every thread then moves one 16-byte piece.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendArgs a, int tokens_per_wg) {
  const int row_shift = a.D == 128 ? 4 : 3;             // log2 of 16-byte pieces per head row
  const int half = a.H_kv << row_shift;                  // pieces of one tensor per token
  const int per_token = 2 * half;
  const int tl = (int)(threadIdx.x / (unsigned)per_token);  // token of this thread in the workgroup
  if (tl >= tokens_per_wg) return;
  const int64_t t = (int64_t)blockIdx.x * tokens_per_wg + tl;
  if (t >= a.num_tokens) return;

  const int s = a.batch_idx[t];
  const int p = a.input_pos[t];
  if (s <= 0 || s >= a.num_slots || p < 0) return;     // padding slot / no such slot
  const int blk = p >> a.page_shift;
  if (blk >= a.max_blocks) return;
  const int page = a.page_table[(int64_t)s * a.max_blocks + blk];
  if (page <= 0 || page >= a.num_pages) return;          // reserved page 0 / not a page
  const int64_t row = ((int64_t)page << a.page_shift) + (p & ((1 << a.page_shift) - 1));

  const int first = (int)threadIdx.x - tl * per_token;
  const int step = tokens_per_wg == 1 ? kAppendThreads : per_token;  // one token: loop over its pieces
  for (int q = first; q < per_token; q += step) {
    const bool is_v = q >= half;
    const int r = is_v ? q - half : q;
    const int h = r >> row_shift;
    const int piece = r & ((1 << row_shift) - 1);
    const uint16_t *src = (is_v ? a.v_new : a.k_new) + (t * a.H_kv + h) * a.D + piece * 8;
    uint16_t *dst = (is_v ? a.v_pool : a.k_pool) + ((int64_t)h * a.plane_rows + row) * a.D + piece * 8;
    // Each byte is read once and written once: stream it past the caches.
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
  }
}

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int per_token = 2 * a.H_kv * (a.D / 8);
  const int tokens_per_wg = per_token >= kAppendThreads ? 1 : kAppendThreads / per_token;
  const int64_t blocks = ((int64_t)a.num_tokens + tokens_per_wg - 1) / tokens_per_wg;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, a,
                     tokens_per_wg);
  return hipGetLastError();
}

}  // namespace pkv
