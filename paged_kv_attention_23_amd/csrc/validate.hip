// Debug checks of the device-side inputs that the attention kernels take on
// trust (they clamp out-of-contract values instead of checking them).
//
// One workgroup walks every row (decode) or document (prefill); each thread
// takes rows t, t + 256, ... in increasing order and keeps its first
// violation.  The count and the smallest violating index are combined in LDS;
// the thread that owns that index then writes its code and block.  The
// kernel reads page_table[s][j] only for s in [0, num_slots) and
// j in [0, max_blocks), and cu_seqlens / doc_slots / prefix_lens only within
// their stated lengths, so any input values are safe to check.
#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kValThreads = 256;

// Pages of the first nblk blocks of slot s: the first block whose page id
// lies outside [1, num_pages), or -1.
__device__ int first_bad_page(const ValidateArgs &a, int s, int64_t nblk) {
  const int32_t *row = a.page_table + (int64_t)s * a.max_blocks;
  for (int64_t j = 0; j < nblk; ++j) {
    const int p = row[j];
    if (p <= 0 || p >= a.num_pages) return (int)j;
  }
  return -1;
}

// The first violation of decode row r: PKV_V_* code, block in *blk.
__device__ int check_decode_row(const ValidateArgs &a, int r, int *blk) {
  const int s = a.batch_idx[r];
  const int n = a.kv_len[r];
  if (s < 0 || s >= a.num_slots) return PKV_V_SLOT;
  if (n < 0) return PKV_V_LEN;
  if (s == 0 || n == 0) return 0;  // padding row
  if ((int64_t)n > ((int64_t)a.max_blocks << a.page_shift)) return PKV_V_CAPACITY;
  const int64_t nblk = ((int64_t)n + (1 << a.page_shift) - 1) >> a.page_shift;
  *blk = first_bad_page(a, s, nblk);
  return *blk >= 0 ? PKV_V_PAGE : 0;
}

// The first violation of prefill document d.
__device__ int check_prefill_doc(const ValidateArgs &a, int d, int *blk) {
  const int lo = a.cu_seqlens[d], hi = a.cu_seqlens[d + 1];
  if ((d == 0 && lo != 0) || hi < lo || (d == a.batch - 1 && hi != a.total_len)) return PKV_V_BOUNDS;
  if (!a.doc_slots) return 0;
  const int s = a.doc_slots[d];
  if (s < 0 || s >= a.num_slots) return PKV_V_SLOT;
  if (!a.prefix_lens) return 0;
  const int p = a.prefix_lens[d];
  if (p < 0) return PKV_V_LEN;
  if (s == 0) return 0;  // padding document
  const int64_t cap = (int64_t)a.max_blocks << a.page_shift;
  if ((int64_t)p + ((int64_t)hi - lo) > cap) return PKV_V_CAPACITY;
  // the cached prefix is read through the page table; the chunk's own rows
  // are written with the append's skip rules, so only prefix blocks count
  const int64_t nblk = ((int64_t)p + (1 << a.page_shift) - 1) >> a.page_shift;
  *blk = first_bad_page(a, s, nblk);
  return *blk >= 0 ? PKV_V_PAGE : 0;
}

__global__ __launch_bounds__(kValThreads) void validate_kernel(ValidateArgs a) {
  __shared__ int count;
  __shared__ int first;
  if (threadIdx.x == 0) {
    count = 0;
    first = INT32_MAX;
  }
  __syncthreads();
  int mine = -1, mine_code = 0, mine_blk = -1, n_bad = 0;
  if (a.cu_seqlens && a.batch == 0 && threadIdx.x == 0 && a.cu_seqlens[0] != a.total_len) {
    n_bad = 1;  // no documents: cu_seqlens[0] must equal total_len (both 0)
    mine = 0;
    mine_code = PKV_V_BOUNDS;
  }
  for (int r = threadIdx.x; r < a.batch; r += kValThreads) {
    int blk = -1;
    const int code = a.cu_seqlens ? check_prefill_doc(a, r, &blk) : check_decode_row(a, r, &blk);
    if (code) {
      ++n_bad;
      if (mine < 0) {
        mine = r;
        mine_code = code;
        mine_blk = blk;
      }
    }
  }
  if (n_bad) {
    atomicAdd(&count, n_bad);
    atomicMin(&first, mine);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.report[0] = count;
    if (count == 0) {
      a.report[1] = -1;
      a.report[2] = 0;
      a.report[3] = -1;
    }
  }
  if (count != 0 && mine == first) {  // exactly one thread owns the first index
    a.report[1] = mine;
    a.report[2] = mine_code;
    a.report[3] = mine_blk;
  }
}

hipError_t launch_validate(const ValidateArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kValThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
