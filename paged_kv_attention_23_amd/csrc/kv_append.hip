// KV append: scatter new tokens' K and V rows into their pages.
//
// The cache update of the attention forward on the qwen3_flex_inference.py
// page writes each new token through the page table before attention runs.
// Here every thread moves one 16-byte piece of one (token, head) row of K or
// V; the page-table lookup is repeated per piece (it hits in cache), which
// keeps the kernel a flat, fully coalesced copy.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int pieces_per_row = a.D >> 3;                       // 16-byte pieces per head row
  const int64_t per_tensor = (int64_t)a.num_tokens * a.H_kv * pieces_per_row;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * per_tensor) return;
  const bool is_v = i >= per_tensor;
  const int64_t j = is_v ? i - per_tensor : i;
  const int piece = (int)(j % pieces_per_row);
  const int64_t th = j / pieces_per_row;                     // token * H_kv + head
  const int h = (int)(th % a.H_kv);
  const int t = (int)(th / a.H_kv);

  const int s = a.batch_idx[t];
  const int p = a.input_pos[t];
  if (s <= 0 || s >= a.num_slots || p < 0) return;           // padding slot / no such slot
  const int blk = p >> a.page_shift;
  if (blk >= a.max_blocks) return;
  const int page = a.page_table[(int64_t)s * a.max_blocks + blk];
  if (page <= 0 || page >= a.num_pages) return;              // reserved page 0 / not a page
  const int64_t row = ((int64_t)page << a.page_shift) + (p & ((1 << a.page_shift) - 1));

  const uint16_t *src = (is_v ? a.v_new : a.k_new) + th * a.D + piece * 8;
  uint16_t *dst = (is_v ? a.v_pool : a.k_pool) + ((int64_t)h * a.plane_rows + row) * a.D + piece * 8;
  *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
}

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)a.num_tokens * a.H_kv * (a.D >> 3);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
