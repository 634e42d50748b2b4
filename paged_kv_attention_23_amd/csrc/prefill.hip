// Packed document-causal prefill attention on the bf16 matrix cores.
//
// What is computed is the prefill of the qwen3_flex_inference.py page:
// prompts packed into one sequence, each token attending to the tokens of
// its own document up to itself, with GQA and scale.  Documents are the row
// ranges [cu_seqlens[d], cu_seqlens[d+1]).
//
// Decomposition (MI355X-specific):
//  * A workgroup owns one query tile of one document and one KV head: 128
//    (query head, query row) pairs, i.e. QT = 128 / G query rows for all G
//    query heads that share the KV head, so each K/V tile staged in LDS serves
//    G heads.  Tiles never straddle documents.
//  * blockIdx enumerates (tile, KV head) with the KV head fastest; workgroups
//    are dealt round-robin to the 8 XCDs, so with 8 KV heads each XCD serves
//    one head.  Tiles are in document order (a document's tiles back to
//    back, its longest key range first), so the query tiles of a document
//    re-read its K/V from that XCD's L2 rather than from HBM.
//  * Each of the 4 waves owns 32 of the 128 rows (two 16-column blocks).
//    Scores are computed transposed, S^T[key][row] = K Q^T, so the score
//    layout is directly the B operand P^T of O^T = V^T P^T (the same scheme
//    as the decode kernel); V^T operands come from gfx950's transposing LDS
//    reads, which hand each lane one head_dim value at four keys.
//  * K/V stages of 64 keys are double buffered in LDS (row stride padded by
//    16 bytes against bank conflicts); the next stage's global loads are in
//    flight while the current one is used.
//  * Online softmax in base 2 in fp32; causal masking only on stages that
//    reach the diagonal.  The weights are computed against the running
//    reference max straight away; the column max is reduced across lanes
//    only on the rare step that moves the reference, which then recomputes
//    them, so the common step has no cross-lane step before its exponentials.
#include <math.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

#ifndef PKV_PF_QB
#define PKV_PF_QB 2
#endif
#ifndef PKV_PF_BN
#define PKV_PF_BN 64
#endif
#ifndef PKV_PF_WPE
#define PKV_PF_WPE 2
#endif
constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kQB = PKV_PF_QB;                       // 16-column blocks per wave
constexpr int kPfRows = 16 * kQB * kPfWaves;         // (head, query) rows per workgroup
constexpr int kPfBN = PKV_PF_BN;                     // keys per LDS stage (multiple of 32)
constexpr int kHalves = kPfBN / 32;                  // 32-key steps per stage
constexpr int kLazyLog2 = 8;                         // lazy-rescale threshold, log2 units
constexpr float kLazyWeight = float(1 << kLazyLog2); // the largest weight a step keeps

// Layout of one head_dim (64 or 128).  A K/V row of D bf16 values is D/8
// 16-byte pieces; one pass of the workgroup's threads over a stage covers
// kRowsPerPass consecutive key rows (16 at D = 128, 32 at D = 64).  LDS rows
// are padded (K by 16 bytes, V by 64) so that the 16 addresses of an operand
// read group fall in distinct banks at either head_dim.
template <int D>
struct PfGeom {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kRowStride = 2 * D + 16;               // bytes per K row in LDS
  static constexpr int kVRowStride = 2 * D + 64;              // bytes per V row in LDS
  static constexpr int kKTileBytes = kPfBN * kRowStride;      // one K stage
  static constexpr int kStageBytes = kKTileBytes + kPfBN * kVRowStride;  // K, then V
  static constexpr int kSmem = 2 * kStageBytes;               // 2 stages
  static constexpr int kPieces = D / 8;                       // 16-byte pieces per row
  static constexpr int kRowsPerPass = kPfThreads / kPieces;   // rows per pass of the workgroup
  static constexpr int kLoads = kPfBN / kRowsPerPass;         // passes per stage
  static_assert(kRowsPerPass % 16 == 0 && kPfBN % kRowsPerPass == 0, "passes are 16-key aligned");
};

struct PfTile {
  int doc, doc_start, doc_end, q_lo, q_hi;
};

// Tile number -> (document, query tile), document-major: the tiles of
// document 0, then of document 1, ...; within a document the last query tile
// (the longest key range) first.  Consecutive tiles of one KV head therefore
// share their document's K/V, which stays in the XCD's L2 while its tiles
// run.  Every wave computes this redundantly: one load of 64 document
// lengths, a prefix sum and a ballot per 64 documents.
__device__ __forceinline__ int ceil_div_qt(int x, int QT, int qt_shift) {
  return qt_shift >= 0 ? (x + QT - 1) >> qt_shift : (x + QT - 1) / QT;
}

// Document bounds are clamped to [0, L] (and the end to no less than the
// start), so out-of-contract cu_seqlens can never place a row outside the
// packed arrays; for valid bounds the clamps change nothing.
__device__ __forceinline__ int doc_lo(const int32_t *cu, int d, int L) { return min(max(cu[d], 0), L); }
__device__ __forceinline__ int doc_hi(const int32_t *cu, int d, int lo, int L) {
  return min(max(cu[d + 1], lo), L);
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: four
// row shifts give the sums within each 16-lane row, then the last lane of
// row 0 is added to row 1 and of row 2 to row 3, and lane 31 to rows 2 and
// 3.  Lanes whose source lies outside the row take 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ bool find_tile(const int32_t *cu, int num_docs, int L, int QT, int qt_shift, int tile,
                          int lane, PfTile &out) {
  int base = 0;  // tiles of the documents before this chunk
  for (int d0 = 0; d0 < num_docs; d0 += kWave) {
    const int d = d0 + lane;
    int t = 0;
    if (d < num_docs) {
      const int lo = doc_lo(cu, d, L);
      t = ceil_div_qt(doc_hi(cu, d, lo, L) - lo, QT, qt_shift);
    }
    const int incl = wave_incl_scan(t);  // inclusive prefix sum of tile counts over the chunk
    const uint64_t hit = __ballot(base + incl > tile);
    if (hit) {
      const int j = __builtin_ctzll(hit);  // uniform
      const int dd = d0 + j;
      const int end = base + __builtin_amdgcn_readlane(incl, j);
      const int qt = end - 1 - tile;  // query tile inside the document, last first
      out.doc = dd;
      out.doc_start = doc_lo(cu, dd, L);
      out.doc_end = doc_hi(cu, dd, out.doc_start, L);
      out.q_lo = out.doc_start + qt * QT;
      out.q_hi = min(out.doc_end, out.q_lo + QT);
      return true;
    }
    base += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  return false;
}

// Waves per SIMD the register budget is sized for: at head_dim 64 the
// kernel fits three (three workgroups per CU, 43 KB of LDS each).
template <int D>
constexpr int kPfWavesPerEu = D == 64 ? 3 : PKV_PF_WPE;

template <int D, bool kFused, bool kPrefix>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(kPfWavesPerEu<D>)))
void prefill_kernel(PrefillArgs a) {
  static_assert(kFused || !kPrefix, "a paged prefix comes with the chunk's scatter");
  using Gm = PfGeom<D>;
  constexpr int kPfRowStride = Gm::kRowStride, kPfVRowStride = Gm::kVRowStride;
  constexpr int kPfKTileBytes = Gm::kKTileBytes, kPfStageBytes = Gm::kStageBytes;
  constexpr int kPieces = Gm::kPieces, kRowsPerPass = Gm::kRowsPerPass, kPfLoads = Gm::kLoads;
  __shared__ __attribute__((aligned(16))) char smem[Gm::kSmem];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hl = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % a.H_kv;
  const int tile = blockIdx.x / a.H_kv;
  const int G = a.G;
  const int QT = kPfRows / G;  // query rows per tile
  const int qt_shift = (QT & (QT - 1)) == 0 ? __builtin_ctz(QT) : -1;

  PfTile tl;
  if (!find_tile(a.cu_seqlens, a.num_docs, a.L, QT, qt_shift, tile, lane, tl)) return;  // uniform
  tl.doc = __builtin_amdgcn_readfirstlane(tl.doc);  // uniform values: keep them in SGPRs
  tl.doc_start = __builtin_amdgcn_readfirstlane(tl.doc_start);
  tl.doc_end = __builtin_amdgcn_readfirstlane(tl.doc_end);
  tl.q_lo = __builtin_amdgcn_readfirstlane(tl.q_lo);
  tl.q_hi = __builtin_amdgcn_readfirstlane(tl.q_hi);
  // Keys are numbered by their position in the sequence: [0, prefix) are
  // cached in the pages (paged prefix, chunked prefill), [prefix, k_end) are
  // this document's packed rows, position prefix + j at packed row
  // doc_start + j.  Without a paged prefix, prefix = 0.
  // Fused scatter: the document's last query tile reads every packed key of
  // the document (its key range ends at the document end), so it alone
  // writes them into their pages, from the stage registers.  Skip rules as
  // in paged_kv_append.
  int slot = 0, prefix = 0;
  bool scatter = false;
  if constexpr (kFused) {
    slot = a.doc_slots[tl.doc];
    const bool slot_ok = slot > 0 && slot < a.num_slots;
    if constexpr (kPrefix) {
      if (!slot_ok) {  // padding document: every row sees no key (+0, -inf)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          const int R = 16 * kQB * wave + 16 * qb + hl;
          const int hh = qt_shift >= 0 ? R >> qt_shift : R / QT;
          const int qq = tl.q_lo + (qt_shift >= 0 ? R & (QT - 1) : R % QT);
          if (hh >= G || qq >= tl.q_hi) continue;
          const int64_t rh = (int64_t)qq * a.H_q + g * G + hh;
#pragma unroll
          for (int i = 0; i < D / 32; ++i)  // lane lg: the D/4 values from (D/4)*lg
            *reinterpret_cast<u32x4 *>(a.out + rh * D + (D / 4) * lg + 8 * i) = u32x4{0u, 0u, 0u, 0u};
          if (lg == 0) a.lse[rh] = -INFINITY;
        }
        return;
      }
      prefix = min(max(a.prefix_lens[tl.doc], 0), a.max_blocks << a.page_shift);
    }
    scatter = tl.q_hi == tl.doc_end && slot_ok;
  }
  const int k_end = prefix + (tl.q_hi - tl.doc_start);

  // Rows of this wave: column block qb, column hl -> tile row R.
  int col_head[kQB], col_q[kQB], col_pos[kQB];
  bool col_ok[kQB];
  bf16x8 qop[kQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int R = 16 * kQB * wave + 16 * qb + hl;
    const int hh = qt_shift >= 0 ? R >> qt_shift : R / QT;
    const int qq = tl.q_lo + (qt_shift >= 0 ? R & (QT - 1) : R % QT);
    col_ok[qb] = (hh < G) && (qq < tl.q_hi);
    col_head[qb] = g * G + min(hh, G - 1);
    col_q[qb] = col_ok[qb] ? qq : tl.q_lo;
    col_pos[qb] = col_ok[qb] ? prefix + (qq - tl.doc_start) : -1;  // -1: masks every key
    const uint16_t *qr = a.q + ((int64_t)col_q[qb] * a.H_q + col_head[qb]) * D + 8 * lg;
#pragma unroll
    for (int ch = 0; ch < D / 32; ++ch) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (col_ok[qb]) w = *reinterpret_cast<const u32x4 *>(qr + 32 * ch);
      qop[qb][ch] = as_bf16x8(w);
    }
  }

  // Cooperative stage loads: piece p = threadIdx.x + 256*i -> key row p/(D/8), 16-byte column p%(D/8).
  // Keys past k_end (last stage only) are clamped to the last key: they lie
  // past every row's position, so their scores are masked and their
  // probabilities are exactly 0 against finite values.
  const int64_t row_stride = (int64_t)a.H_kv * D;  // elements between consecutive tokens
  const uint32_t row_bytes = (uint32_t)row_stride * 2u;  // < 2^24, checked on the host
  const uint32_t col_bytes = (threadIdx.x % kPieces) * 16u;
  const int row0 = threadIdx.x / kPieces;               // stage row of piece 0
  const uint16_t *kg = a.k + (int64_t)g * D;
  const uint16_t *vg = a.v + (int64_t)g * D;
  const int32_t *pt_row = kFused ? a.page_table + (int64_t)slot * a.max_blocks : nullptr;
  // Cached prefix: page ids of the document's first 64 blocks, one per lane,
  // loaded once.  In a stage inside the prefix, pass i covers the keys
  // key0 + kRowsPerPass*i ..; each 16-key group of them lies in one page
  // (pages hold >= 16 keys and the groups are 16-aligned), so each group
  // needs one page id (a lane read) and one uniform base.
  int pwin = 0;
  if constexpr (kPrefix) {
    const int nblk = (prefix + (1 << a.page_shift) - 1) >> a.page_shift;
    if (lane < nblk && lane < a.max_blocks) pwin = pt_row[lane];
  }
  u32x4 stk[kPfLoads], stv[kPfLoads];
  int spage[kPfLoads];  // fused scatter: page of each piece's key (0 = skip)
  auto load_stage = [&](int s) {
    const int key0 = s * kPfBN;  // position of the stage's first key
    if (kPrefix && key0 + kPfBN <= prefix) {
      // Whole stage in the cached prefix: one page per 16-key piece.
      const int grow = kRowsPerPass == 16 ? row0 : (row0 & 15);  // the lane's row in its 16-key group
      const uint32_t off = (uint32_t)grow * (uint32_t)(D * 2) + col_bytes;
#pragma unroll
      for (int i = 0; i < kPfLoads; ++i) {
        int key = key0 + kRowsPerPass * i;  // first key of the lane's 16-key group
        int page;
        if constexpr (kRowsPerPass == 16) {
          const int blk = key >> a.page_shift;
          page = blk < kWave ? __builtin_amdgcn_readlane(pwin, blk) : pt_row[blk];
        } else {
          page = 0;
#pragma unroll
          for (int j = 0; j < kRowsPerPass / 16; ++j) {  // one uniform page id per group
            const int blk = (key + 16 * j) >> a.page_shift;
            const int pj = blk < kWave ? __builtin_amdgcn_readlane(pwin, blk) : pt_row[blk];
            if ((row0 >> 4) == j) page = pj;
          }
          key += 16 * (row0 >> 4);
        }
        page = min(max(page, 0), a.num_pages - 1);
        const int64_t first = ((int64_t)g * a.plane_rows + ((int64_t)page << a.page_shift) +
                               (key & ((1 << a.page_shift) - 1))) * D;
        stk[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.k_pool + first) + off);
        stv[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.v_pool + first) + off);
      }
    } else if (!kPrefix || key0 >= prefix) {
      // This document's packed rows only: one uniform base per stage and
      // 32-bit lane offsets.
      const int64_t first = (int64_t)(tl.doc_start + key0 - prefix) * row_stride;
      const char *kbs = reinterpret_cast<const char *>(kg + first);
      const char *vbs = reinterpret_cast<const char *>(vg + first);
      const int last = k_end - 1 - key0;  // last live row of the stage
#pragma unroll
      for (int i = 0; i < kPfLoads; ++i) {
        const int r = min(row0 + kRowsPerPass * i, last);
        const uint32_t off = __umul24((uint32_t)r, row_bytes) + col_bytes;
        stk[i] = *reinterpret_cast<const u32x4 *>(kbs + off);
        stv[i] = *reinterpret_cast<const u32x4 *>(vbs + off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPfLoads; ++i) {
        const int p = threadIdx.x + kPfThreads * i;
        const int key = min(key0 + p / kPieces, k_end - 1);
        if (key < prefix) {                 // cached prefix: through the page table
          int page = pt_row[key >> a.page_shift];
          page = min(max(page, 0), a.num_pages - 1);
          const int64_t row = (int64_t)g * a.plane_rows + ((int64_t)page << a.page_shift) +
                              (key & ((1 << a.page_shift) - 1));
          stk[i] = *reinterpret_cast<const u32x4 *>(a.k_pool + row * D + (p % kPieces) * 8);
          stv[i] = *reinterpret_cast<const u32x4 *>(a.v_pool + row * D + (p % kPieces) * 8);
        } else {                            // this document's packed rows
          const int64_t off = (int64_t)(tl.doc_start + key - prefix) * row_stride + (p % kPieces) * 8;
          stk[i] = *reinterpret_cast<const u32x4 *>(kg + off);
          stv[i] = *reinterpret_cast<const u32x4 *>(vg + off);
        }
      }
    }
    if constexpr (kFused) {
      if (scatter) {
#pragma unroll
        for (int i = 0; i < kPfLoads; ++i) {
          const int pos = key0 + row0 + kRowsPerPass * i;
          const int blk = pos >> a.page_shift;
          spage[i] = (pos >= prefix && pos < k_end && blk < a.max_blocks) ? pt_row[blk] : 0;
        }
      }
    }
  };
  auto scatter_stage = [&](int s) {
#pragma unroll
    for (int i = 0; i < kPfLoads; ++i) {
      const int p = threadIdx.x + kPfThreads * i;
      if (spage[i] > 0 && spage[i] < a.num_pages) {
        const int pos = s * kPfBN + p / kPieces;
        const int64_t row = (int64_t)g * a.plane_rows + ((int64_t)spage[i] << a.page_shift) +
                            (pos & ((1 << a.page_shift) - 1));
        // whole 256-byte rows, not read again here: past the caches
        __builtin_nontemporal_store(stk[i], reinterpret_cast<u32x4 *>(a.k_pool + row * D + (p % kPieces) * 8));
        __builtin_nontemporal_store(stv[i], reinterpret_cast<u32x4 *>(a.v_pool + row * D + (p % kPieces) * 8));
      }
    }
  };
  auto store_stage = [&](int buf) {
    char *kb = smem + buf * kPfStageBytes;
    char *vb = kb + kPfKTileBytes;
#pragma unroll
    for (int i = 0; i < kPfLoads; ++i) {
      const int p = threadIdx.x + kPfThreads * i;
      *reinterpret_cast<u32x4 *>(kb + (p / kPieces) * kPfRowStride + (p % kPieces) * 16) = stk[i];
      *reinterpret_cast<u32x4 *>(vb + (p / kPieces) * kPfVRowStride + (p % kPieces) * 16) = stv[i];
    }
  };

  float m_run[kQB], l_run[kQB], neg_m[kQB];  // neg_m: -m_run, or 0 while m_run is -inf
  f32x4 o[kQB][D / 16];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    neg_m[qb] = 0.f;
  }
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int t = 0; t < D / 16; ++t) o[qb][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (k_end + kPfBN - 1) / kPfBN;
  const int q_first = prefix + (tl.q_lo - tl.doc_start);  // position of the tile's first row
  load_stage(0);
  store_stage(0);
  if constexpr (kFused) {
    if (scatter) scatter_stage(0);
  }
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_stage(s + 1);
    const char *kb = smem + buf * kPfStageBytes;
    const char *vb = kb + kPfKTileBytes;
    // Transposing V reads: within each 16-lane group, lane hl addresses key
    // row 4*lg + hl/4 (plus the block's first key) at head_dim
    // 32*(t/2) + 8*(hl%4) + 4*(t%2); the hardware hands lane hl the four
    // keys' values at one head_dim.  (V rows are 320 bytes apart, so the 16
    // addresses of a group fall in distinct banks.)
    const char *v_tr = vb + (4 * lg + (hl >> 2)) * kPfVRowStride + 16 * (hl & 3);
    // S^T blocks of a 32-key half: keys key0 + 16*kb2 + (4*lg + i), columns qb.
    auto qk = [&](int h2, f32x4 (&sc)[2][kQB]) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        bf16x8 kop[D / 32];
        const char *kr = kb + (32 * h2 + 16 * kb2 + hl) * kPfRowStride + 16 * lg;
#pragma unroll
        for (int ch = 0; ch < D / 32; ++ch) kop[ch] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kr + 64 * ch));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ch = 0; ch < D / 32; ++ch) acc = mfma16x16x32(kop[ch], qop[qb][ch], acc);
          sc[kb2][qb] = acc;
        }
      }
    };
    auto softmax_pv = [&](int h2, const f32x4 (&sc)[2][kQB]) {
      const int key0 = s * kPfBN + 32 * h2;  // position of the half's first key
      const bool diag = key0 + 31 >= q_first;  // some key may lie past some query row
      const bool first = key0 == 0;  // the tile's first step: m_run is still -inf, no speculation
      // V^T operands from transposing LDS reads: lane (hl, lg) of step t
      // gets head_dim d = 32*(t/2) + 8*(hl/4) + 4*(t%2) + hl%4 at keys
      // kappa(lg, 0..3) and kappa(lg, 4..7), the key order of P^T.  All eight are read first, so
      // that a column block's PV products can be issued as soon as its
      // softmax is done and run on the matrix cores during the next block's.
      bf16x8 vop[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const int col = 64 * (t >> 1) + 8 * (t & 1);  // bytes: head_dim 32*(t/2) + 4*(t%2)
        const u32x2 lo = lds_read_tr16(v_tr + (32 * h2) * kPfVRowStride + col);
        const u32x2 hi = lds_read_tr16(v_tr + (32 * h2 + 16) * kPfVRowStride + col);
        vop[t] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        // raw scores; scale (> 0) is applied to the max and inside the exponent
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = sc[0][qb][i];
          x[4 + i] = sc[1][qb][i];
        }
        if (diag) {
          const int lim = col_pos[qb] - key0 - 4 * lg;  // key offset i is live iff i <= lim
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int off = i < 4 ? i : 16 + (i - 4);
            if (off > lim) x[i] = -INFINITY;
          }
        }
        // Speculative weights against the current reference point m_run.  The
        // reference must move only when some weight exceeds 2^kLazyLog2; every
        // weight is at most its lane's sum, so the sum the step needs anyway
        // is the test (it may fire on a step that could have stayed, never
        // miss one).  The rare step that moves it takes the column max (max
        // commutes with the positive scale) and recomputes.
        float p[8], ps = 0.f;
        if (!first) {
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(x[i], a.scale_log2, neg_m[qb]));
          ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        }
        if (first || __any(!(ps <= kLazyWeight))) {
          float lm = x[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) lm = fmaxf(lm, x[i]);
          float mt = max_xor16(lm);
          mt = max_xor32(mt);
          mt *= a.scale_log2;
          const float m_new = fmaxf(m_run[qb], mt);
          if (__any(m_run[qb] != -INFINITY)) {  // otherwise o and l are still zero
            const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[qb] - m_new);
            l_run[qb] *= alpha;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) o[qb][t] *= alpha;
          }
          m_run[qb] = m_new;
          neg_m[qb] = (m_new == -INFINITY) ? 0.f : -m_new;
#pragma unroll
          for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(x[i], a.scale_log2, neg_m[qb]));
          ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        }
        l_run[qb] += ps;
        const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        const bf16x8 pop = as_bf16x8(pw);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) o[qb][t] = mfma16x16x32(vop[t], pop, o[qb][t]);
      }
    };
#pragma unroll
    for (int h2 = 0; h2 < kHalves; ++h2) {  // 32-key steps of the stage
      if (s * kPfBN + 32 * h2 >= k_end) break;  // uniform
      f32x4 sc[2][kQB];
      qk(h2, sc);
      softmax_pv(h2, sc);
    }
    if (s + 1 < nsteps) {  // uniform
      store_stage(buf ^ 1);
      if constexpr (kFused) {
        if (scatter) scatter_stage(s + 1);
      }
      __syncthreads();  // stage s+1 is in LDS and every wave is done with stage s
    }
    // After the last stage no wave touches the LDS again and each writes only
    // its own rows, so the waves go on to the epilogue without a barrier.
  }

  // Normalise and write: lane holds O[row][d = 32*(t/2) + 8*lg + 4*(t%2) + i]
  // in o[qb][t][i], so steps 2c and 2c+1 are 8 contiguous values and the four
  // lanes of a row write 64 contiguous bytes per store (D/32 stores).
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float l = l_run[qb];
    l = sum_xor16(l);
    l = sum_xor32(l);
    if (!col_ok[qb]) continue;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const int64_t rh = (int64_t)col_q[qb] * a.H_q + col_head[qb];
    uint16_t *orow = a.out + rh * D + 8 * lg;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {  // 16-byte piece c: d = 32*c + 8*lg + 0..7 = steps 2c, 2c+1
      const f32x4 a0 = o[qb][2 * c], a1 = o[qb][2 * c + 1];
      const u32x4 w = {pack_bf16x2(a0[0] * inv, a0[1] * inv), pack_bf16x2(a0[2] * inv, a0[3] * inv),
                       pack_bf16x2(a1[0] * inv, a1[1] * inv), pack_bf16x2(a1[2] * inv, a1[3] * inv)};
      *reinterpret_cast<u32x4 *>(orow + 32 * c) = w;
    }
    if (lg == 0) a.lse[rh] = (l > 0.f) ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  if (a.L == 0) return hipSuccess;
  const int QT = kPfRows / a.G;
  // Sum over documents of ceil(n_d / QT) is at most ceil(L / QT) + num_docs.
  const int64_t tiles = ((int64_t)a.L + QT - 1) / QT + a.num_docs;
  if (tiles * a.H_kv > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;  // grid would wrap
  const dim3 grid((unsigned)(tiles * a.H_kv));
  if (a.D == 64) {
    if (a.prefix_lens)
      hipLaunchKernelGGL((prefill_kernel<64, true, true>), grid, dim3(kPfThreads), 0, stream, a);
    else if (a.k_pool)
      hipLaunchKernelGGL((prefill_kernel<64, true, false>), grid, dim3(kPfThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<64, false, false>), grid, dim3(kPfThreads), 0, stream, a);
  } else if (a.D == 128) {
    if (a.prefix_lens)
      hipLaunchKernelGGL((prefill_kernel<128, true, true>), grid, dim3(kPfThreads), 0, stream, a);
    else if (a.k_pool)
      hipLaunchKernelGGL((prefill_kernel<128, true, false>), grid, dim3(kPfThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<128, false, false>), grid, dim3(kPfThreads), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
