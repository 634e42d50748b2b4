// Reachable-rate probes that the benchmark reports beside the attention
// kernels' figures (libpkvceil.so, loaded by bench.py only; not part of the
// attention library's ABI).  They compute nothing useful: each one moves
// bytes or issues matrix instructions at the fastest rate a plain kernel of
// its shape reaches on this GPU, and keeps its results alive with a
// data-dependent store that never fires for the inputs the benchmark uses.
//
//   ceil_stream_read   one grid-strided front of non-temporal 16-byte loads
//                      over a buffer (the plain HBM read ceiling)
//   ceil_stream_units  the decode launch shape with the arithmetic taken
//                      out: one workgroup of 4 waves per (row, KV head) unit,
//                      each reading its unit's K and V rows (contiguous runs
//                      given by the caller) in 32-key tiles dealt to waves in
//                      turn, one tile in flight per wave
//   ceil_paged_units   the same launch shape and tiles, with the keys found
//                      the way paged decode finds them: the row's slot and
//                      length from batch_idx / kv_len, then one load of the
//                      page ids of its first 64 blocks, then each 16-key
//                      block's rows through its page id (no arithmetic on
//                      the data either)
//   ceil_prefill_shape the packed prefill's launch shape and memory traffic
//                      with the arithmetic taken out: one workgroup per
//                      (query tile of 128 (head, row) pairs, KV head) in the
//                      same document-major order, finding its tile from
//                      cu_seqlens, reading its Q rows once, streaming its
//                      document's K/V rows in 32-key stages (one stage in
//                      flight), and writing its output rows and LSEs, at
//                      the prefill's occupancy (three workgroups per CU)
//   ceil_mfma          back-to-back 16x16x32 bf16 matrix instructions,
//                      16 independent accumulators per wave, two waves per
//                      SIMD (the dense bf16 rate of the instruction the
//                      attention kernels use)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, uint64_t n,
                                                          uint32_t key, uint32_t *sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = ld_nt(p + i), b = ld_nt(p + i + stride), c = ld_nt(p + i + 2 * stride),
                d = ld_nt(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= ld_nt(p + i);
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == key) sink[blockIdx.x & 1023u] = x;
}

// units[2*u] = first pool row of unit u's keys in its KV head plane (K and V
// use the same rows), units[2*u+1] = its number of keys (0: padding, the
// workgroup exits).  Unit u belongs to KV head u % H_kv.
__global__ __launch_bounds__(256) void stream_units_kernel(const char *__restrict__ kpool,
                                                           const char *__restrict__ vpool,
                                                           uint64_t plane_bytes, int H_kv,
                                                           const int32_t *__restrict__ units,
                                                           uint32_t key, uint32_t *sink) {
  const int u = blockIdx.x;
  const int row0 = units[2 * u], n = units[2 * u + 1];
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t head = (uint64_t)(u % H_kv) * plane_bytes;
  const char *kb = kpool + head + (uint64_t)row0 * 256u;
  const char *vb = vpool + head + (uint64_t)row0 * 256u;
  // A 32-key tile of one tensor is 8 KB: 8 loads of 16 bytes per lane; lane l
  // reads key row 4*i + l/16, column l%16 in load i.
  const int ntiles = (n + 31) / 32;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 kr[8], vr[8];
  auto issue = [&](int t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int key_row = 32 * t + 4 * i + (lane >> 4);
      key_row = key_row < n ? key_row : n - 1;
      const uint32_t off = (uint32_t)key_row * 256u + (uint32_t)(lane & 15) * 16u;
      kr[i] = ld_nt(reinterpret_cast<const u32x4 *>(kb + off));
      vr[i] = ld_nt(reinterpret_cast<const u32x4 *>(vb + off));
    }
  };
  int t = wave;
  if (t < ntiles) issue(t);
  while (t < ntiles) {
    u32x4 k2[8], v2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k2[i] = kr[i];
      v2[i] = vr[i];
    }
    const int tn = t + 4;
    if (tn < ntiles) issue(tn);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= k2[i] ^ v2[i];
    t = tn;
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == key) sink[u & 1023] = x;
}

// Unit u = (row u / H_kv, KV head u % H_kv).  Rows in slot 0, beyond the
// table or without keys exit; keys past 64 blocks are not read (the window
// of one page-id load).  Rows are row_bytes apart in a head plane.
__global__ __launch_bounds__(256) void paged_units_kernel(
    const char *__restrict__ kpool, const char *__restrict__ vpool, uint64_t plane_bytes,
    uint32_t row_bytes, int H_kv, const int32_t *__restrict__ page_table, int max_blocks,
    int page_shift, int num_pages, int num_slots, const int32_t *__restrict__ batch_idx,
    const int32_t *__restrict__ kv_len, uint32_t key, uint32_t *sink) {
  const int u = blockIdx.x;
  const int r = u / H_kv, g = u % H_kv;
  const int s = batch_idx[r];
  const int n = min(kv_len[r], min(max_blocks, 64) << page_shift);
  if (s <= 0 || s >= num_slots || n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int pwin = lane < max_blocks ? page_table[(int64_t)s * max_blocks + lane] : 0;
  pwin = min(max(pwin, 0), num_pages - 1);
  const uint64_t head = (uint64_t)g * plane_bytes;
  const char *kb = kpool + head;
  const char *vb = vpool + head;
  const int ntiles = (n + 31) / 32;
  const uint32_t in_page = (1u << page_shift) - 1u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 kr[8], vr[8];
  // Load i of tile t covers keys 32t + 4i .. +3 (clamped to n-1): one
  // 16-key block, hence one page id, for all 64 lanes.
  auto issue = [&](int t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int first = min(32 * t + 4 * i, n - 1);
      const int page = __builtin_amdgcn_readlane(pwin, first >> page_shift);
      const int k = min(32 * t + 4 * i + (lane >> 4), n - 1);
      const uint32_t row = ((uint32_t)page << page_shift) + ((uint32_t)k & in_page);
      const uint32_t off = row * row_bytes + (uint32_t)(lane & 15) * 16u;
      kr[i] = ld_nt(reinterpret_cast<const u32x4 *>(kb + off));
      vr[i] = ld_nt(reinterpret_cast<const u32x4 *>(vb + off));
    }
  };
  int t = wave;
  if (t < ntiles) issue(t);
  while (t < ntiles) {
    u32x4 k2[8], v2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      k2[i] = kr[i];
      v2[i] = vr[i];
    }
    const int tn = t + 4;
    if (tn < ntiles) issue(tn);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= k2[i] ^ v2[i];
    t = tn;
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == key) sink[u & 1023] = x;
}

// Inclusive prefix sum over the wave in registers (DPP row shifts, then the
// row-15 and lane-31 broadcasts).
__device__ __forceinline__ int scan64(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

// Head dim 128, 128 (head, row) pairs per tile: QT = 128 / G rows.  Tiles
// are numbered document by document, a document's last query tile first;
// blockIdx = tile * H_kv + KV head.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_shape_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                          const uint16_t *__restrict__ v, const int32_t *__restrict__ cu,
                          int num_docs, int L, int H_q, int H_kv, uint16_t *__restrict__ out,
                          float *__restrict__ lse) {
  constexpr int D = 128;
  // LDS reserved so that the probe runs at the attention kernel's occupancy,
  // three workgroups per CU (its registers allow three): 48 KB admits three
  // and not four.
  __shared__ uint32_t occ[49152 / 4];
  occ[threadIdx.x] = blockIdx.x;
  __syncthreads();
  if (occ[(threadIdx.x + 1) & 255] == 0xdeadbeefu) lse[0] = 1.f;  // never true; keeps the array
  const int G = H_q / H_kv, QT = 128 / G;
  const int g = blockIdx.x % H_kv, tile = blockIdx.x / H_kv;
  const int lane = threadIdx.x & 63;
  // tile -> (document, query tile)
  int base = 0, doc = -1, qt = 0;
  for (int d0 = 0; d0 < num_docs && doc < 0; d0 += 64) {
    const int d = d0 + lane;
    int t = 0;
    if (d < num_docs) {
      const int lo = min(max(cu[d], 0), L), hi = min(max(cu[d + 1], lo), L);
      t = (hi - lo + QT - 1) / QT;
    }
    const int incl = scan64(t);
    const uint64_t hit = __ballot(base + incl > tile);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      doc = d0 + j;
      qt = base + __builtin_amdgcn_readlane(incl, j) - 1 - tile;
    } else {
      base += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (doc < 0) return;  // uniform
  const int doc_start = min(max(cu[doc], 0), L), doc_end = min(max(cu[doc + 1], doc_start), L);
  const int q_lo = doc_start + qt * QT, q_hi = min(doc_end, q_lo + QT);
  const int k_end = q_hi - doc_start;  // keys of the tile's longest row
  if (k_end <= 0) return;  // uniform; a found tile always has keys
  const int col = threadIdx.x & 15, row0 = threadIdx.x >> 4;  // 16 lanes per 256-byte row
  u32x4 acc = {0u, 0u, 0u, 0u};
  // Q: 128 rows of 256 bytes, row R = row0 + 16 i -> head R / QT, query q_lo + R % QT;
  // in flight together with the first K/V stage, as in the prefill
  int orow[8];
  u32x4 qv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int R = row0 + 16 * i, hh = R / QT, qq = q_lo + R % QT;
    orow[i] = (hh < G && qq < q_hi) ? qq * H_q + g * G + hh : -1;
    qv[i] = u32x4{0u, 0u, 0u, 0u};
    if (orow[i] >= 0) qv[i] = *reinterpret_cast<const u32x4 *>(q + (int64_t)orow[i] * D + col * 8);
  }
  // K/V: 32-key stages of the document's rows, one stage in flight
  const int64_t rs = (int64_t)H_kv * D;  // elements between consecutive tokens
  const uint16_t *kg = k + (int64_t)doc_start * rs + g * D + col * 8;
  const uint16_t *vg = v + (int64_t)doc_start * rs + g * D + col * 8;
  u32x4 ks[2], vs[2];
  auto load = [&](int s0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(s0 + row0 + 16 * i, k_end - 1);
      ks[i] = *reinterpret_cast<const u32x4 *>(kg + key * rs);
      vs[i] = *reinterpret_cast<const u32x4 *>(vg + key * rs);
    }
  };
  load(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc ^= qv[i];
  for (int s0 = 0; s0 < k_end; s0 += 32) {
    u32x4 k2[2], v2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      k2[i] = ks[i];
      v2[i] = vs[i];
    }
    if (s0 + 32 < k_end) load(s0 + 32);
#pragma unroll
    for (int i = 0; i < 2; ++i) acc ^= k2[i] ^ v2[i];
  }
  // output rows and LSEs (values derived from everything read)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (orow[i] < 0) continue;
    *reinterpret_cast<u32x4 *>(out + (int64_t)orow[i] * D + col * 8) = acc;
    if (col == 0) lse[orow[i]] = __uint_as_float(acc.x);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_kernel(int iters, float key, float *sink) {
  const float s = (float)(threadIdx.x & 7) * 0.001f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(s + 0.01f * i);
    b[i] = (__bf16)(0.5f - s);
  }
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (t == key) sink[blockIdx.x & 1023] = t;
}

}  // namespace

extern "C" {

// Grids are the caller's; every kernel is bounded by its arguments.
int ceil_stream_read(const void *buf, uint64_t bytes, int grid, uint32_t *sink, void *stream) {
  if (!buf || !sink || grid <= 0 || (bytes & 15u)) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)buf, bytes / 16u, 0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int ceil_stream_units(const void *kpool, const void *vpool, uint64_t plane_bytes, int H_kv,
                      const int32_t *units, int num_units, uint32_t *sink, void *stream) {
  if (!kpool || !vpool || !units || !sink || H_kv <= 0 || num_units <= 0) return -1;
  hipLaunchKernelGGL(stream_units_kernel, dim3(num_units), dim3(256), 0, (hipStream_t)stream,
                     (const char *)kpool, (const char *)vpool, plane_bytes, H_kv, units,
                     0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// row_bytes: head_dim * 2 (16 lanes of 16 bytes read a row, so at most 256).
int ceil_paged_units(const void *kpool, const void *vpool, uint64_t plane_bytes, uint32_t row_bytes,
                     int H_kv, const int32_t *page_table, int max_blocks, int page_shift,
                     int num_pages, int num_slots, const int32_t *batch_idx,
                     const int32_t *kv_len, int batch, uint32_t *sink, void *stream) {
  if (!kpool || !vpool || !page_table || !batch_idx || !kv_len || !sink || H_kv <= 0 ||
      batch <= 0 || max_blocks <= 0 || num_pages <= 0 || page_shift < 4 || row_bytes != 256u ||
      plane_bytes > 0xffffffffull || (uint64_t)num_pages << page_shift > plane_bytes / row_bytes)
    return -1;
  hipLaunchKernelGGL(paged_units_kernel, dim3((unsigned)batch * (unsigned)H_kv), dim3(256), 0,
                     (hipStream_t)stream, (const char *)kpool, (const char *)vpool, plane_bytes,
                     row_bytes, H_kv, page_table, max_blocks, page_shift, num_pages, num_slots,
                     batch_idx, kv_len, 0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Packed bf16 q [L][H_q][128], k/v [L][H_kv][128], cu_seqlens [num_docs+1];
// writes out [L][H_q][128] and lse [L][H_q] (values meaningless).
int ceil_prefill_shape(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                       int num_docs, int L, int H_q, int H_kv, void *out, float *lse,
                       void *stream) {
  if (!q || !k || !v || !cu_seqlens || !out || !lse || num_docs <= 0 || L <= 0 || H_kv <= 0 ||
      H_q % H_kv != 0 || H_q / H_kv > 16 || 128 % (H_q / H_kv) != 0)
    return -1;
  const int64_t QT = 128 / (H_q / H_kv);
  const int64_t grid = ((L + QT - 1) / QT + num_docs) * H_kv;
  if (grid > 0x7fffffff) return -1;
  hipLaunchKernelGGL(prefill_shape_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, cu_seqlens,
                     num_docs, L, H_q, H_kv, (uint16_t *)out, lse);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int ceil_mfma(int grid, int iters, float *sink, void *stream) {
  if (!sink || grid <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, -1.0f,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
