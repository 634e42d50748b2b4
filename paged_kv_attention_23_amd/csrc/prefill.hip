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
//  * K/V stages (32 keys at head_dim 128, 64 at 64) are double buffered in
//    LDS and written by gfx950's global-to-LDS loads, so no registers stage
//    them; rows are unpadded with their 16-byte chunks XOR-swizzled against
//    bank conflicts.  The next stage's loads are in flight while the current
//    one is used.  The registers this frees let three workgroups share a CU
//    (four at head_dim 64), which hides more of each tile's start-up and
//    epilogue behind the other tiles' work.
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
constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kQB = PKV_PF_QB;                       // 16-column blocks per wave
constexpr int kPfRows = 16 * kQB * kPfWaves;         // (head, query) rows per workgroup
constexpr int kLazyLog2 = 8;                         // lazy-rescale threshold, log2 units
constexpr float kLazyWeight = float(1 << kLazyLog2); // the largest weight a step keeps

// LDS layout of one head_dim (64 or 128).  A K or V row of D bf16 values is
// 2*D bytes, unpadded, in kChunks chunks of 16 bytes; chunk c of row r is
// stored at position c ^ swz(r).  The swizzle depends on r mod 16 only and
// makes both operand reads conflict-free: the K reads of one instruction
// take one chunk from each of 16 consecutive rows, which land on 16 distinct
// positions (D = 128: swz is a bijection of r mod 16; D = 64: two rows share
// 256 bytes of banks, and swz is a bijection over the 8 rows of each
// parity), and the transposing V reads of 16 lanes take chunks 4q..4q+3 of 4
// consecutive rows, which swz sends to disjoint groups of 4 positions (or to
// the other half of the banks).
template <int D, int BN>
struct PfGeom {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kRowBytes = 2 * D;                        // one K or V row
  static constexpr int kChunks = kRowBytes / 16;                 // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;          // rows one global-to-LDS load fills
  static constexpr int kTileBytes = BN * kRowBytes;              // K (or V) of one stage
  static constexpr int kStageBytes = 2 * kTileBytes;             // K, then V
  static constexpr int kLoadsPerWave = BN / kRowsPerLoad / kPfWaves;  // per tensor and stage
  static_assert(kLoadsPerWave * kRowsPerLoad * kPfWaves == BN, "a stage is whole loads per wave");
  static_assert(16 % kRowsPerLoad == 0, "a load's rows lie in one 16-key group");
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
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

// Per head_dim: keys per LDS stage, waves per SIMD the registers are sized
// for, and whether V^T operands are read right before their products
// (fewer live registers) or all at once ahead of the softmax.  At head_dim
// 128 every kernel runs 32-key stages at three waves per SIMD, three
// workgroups per CU (32 KB of LDS each); at head_dim 64, 64-key stages fit
// four waves with all V^T operands read first.
template <int D>
struct PfTune {
  static constexpr int kBN = D == 64 ? 64 : 32;
  static constexpr int kWaves = D == 64 ? 4 : 3;
  static constexpr bool kJitV = kBN == 32;
};

template <int D, bool kFused, bool kPrefix>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(PfTune<D>::kWaves)))
void prefill_kernel(PrefillArgs a) {
  static_assert(kFused || !kPrefix, "a paged prefix comes with the chunk's scatter");
  using Tn = PfTune<D>;
  constexpr int BN = Tn::kBN;  // keys per stage
  using Gm = PfGeom<D, BN>;
  __shared__ __attribute__((aligned(1024))) char sA[Gm::kStageBytes];  // stage buffers
  __shared__ __attribute__((aligned(1024))) char sB[Gm::kStageBytes];
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
  // Fused scatter: each query tile writes its own rows' K/V into their pages,
  // after its outputs.
  int slot = 0, prefix = 0;
  bool slot_ok = false;
  if constexpr (kFused) {
    slot = a.doc_slots[tl.doc];
    slot_ok = slot > 0 && slot < a.num_slots;
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

  // K/V stages: BN keys of K, then of V, in one of two LDS buffers (sA
  // and sB are distinct arrays, so the compiler's wait counting can tell that
  // loads into one buffer never alias reads of the other).  Stages are
  // written by gfx950's global-to-LDS loads, so no register holds stage data:
  // load j of a stage fills 1 KB, rows kRowsPerLoad*j .., lane l the row
  // kRowsPerLoad*j + l/kChunks at position l%kChunks, which holds the row's
  // global chunk (l%kChunks) ^ swz(row).  Keys past k_end (last stage only)
  // are clamped to the last key: they lie past every row's position, so
  // their scores are masked and their probabilities are exactly 0 against
  // finite values.
  const int64_t row_stride = (int64_t)a.H_kv * D;  // elements between consecutive tokens
  const uint32_t row_bytes = (uint32_t)row_stride * 2u;  // < 2^24, checked on the host
  const char *kg = reinterpret_cast<const char *>(a.k + (int64_t)g * D);
  const char *vg = reinterpret_cast<const char *>(a.v + (int64_t)g * D);
  const int32_t *pt_row = kFused ? a.page_table + (int64_t)slot * a.max_blocks : nullptr;
  const int page_mask = (1 << a.page_shift) - 1;
  // Cached prefix: page ids of the document's first 64 blocks, one per lane,
  // loaded once.  A load instruction's rows lie in one 16-key group, so in a
  // stage wholly inside the prefix each instruction needs one page id (a lane
  // read) and every lane adds its row's offset in the page.
  int pwin = 0;
  if constexpr (kPrefix) {
    const int nblk = (prefix + page_mask) >> a.page_shift;
    if (lane < nblk && lane < a.max_blocks) pwin = pt_row[lane];
  }
  // this KV head's planes of the pools, and a key's row in them (32-bit
  // byte offsets: a plane is below 4 GiB, checked on the host)
  const int64_t plane = (int64_t)g * a.plane_rows * D;
  const char *kpool = reinterpret_cast<const char *>(kFused ? a.k_pool + plane : nullptr);
  const char *vpool = reinterpret_cast<const char *>(kFused ? a.v_pool + plane : nullptr);
  auto pool_off = [&](int page, int key) {
    page = min(max(page, 0), a.num_pages - 1);
    return (((uint32_t)page << a.page_shift) + (uint32_t)(key & page_mask)) * (2u * D);
  };
  const int lrow = lane / Gm::kChunks, lpos = lane % Gm::kChunks;
  auto dma_stage = [&](int st, char *dst) {
    const int key0 = st * BN;
    // sources first (a prefix stage may look its pages up), then the loads,
    // so that no wait for a page id holds back loads already issued
    const char *ks[Gm::kLoadsPerWave], *vs[Gm::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < Gm::kLoadsPerWave; ++i) {
      const int j = wave + kPfWaves * i;                  // load instruction of the stage
      const int r = Gm::kRowsPerLoad * j + lrow;          // this lane's stage row
      const uint32_t cb = (uint32_t)(lpos ^ Gm::swz(r)) << 4;  // its global chunk, in bytes
      if (kPrefix && key0 + BN <= prefix) {
        // whole stage in the cached prefix: one page per load instruction
        const int blk = (key0 + Gm::kRowsPerLoad * j) >> a.page_shift;  // uniform
        const int page = blk < kWave ? __builtin_amdgcn_readlane(pwin, blk) : pt_row[blk];
        const uint32_t off = pool_off(page, key0 + r) + cb;
        ks[i] = kpool + off;
        vs[i] = vpool + off;
      } else if (!kPrefix || key0 >= prefix) {
        // this document's packed rows only
        const int64_t first = (int64_t)(tl.doc_start + key0 - prefix) * row_bytes;
        const uint32_t off = __umul24((uint32_t)min(r, k_end - 1 - key0), row_bytes) + cb;
        ks[i] = kg + first + off;
        vs[i] = vg + first + off;
      } else {
        const int key = min(key0 + r, k_end - 1);
        if (key < prefix) {  // cached prefix: through the page table
          const uint32_t off = pool_off(pt_row[key >> a.page_shift], key) + cb;
          ks[i] = kpool + off;
          vs[i] = vpool + off;
        } else {             // this document's packed rows
          const int64_t off = (int64_t)(tl.doc_start + key - prefix) * row_bytes + cb;
          ks[i] = kg + off;
          vs[i] = vg + off;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < Gm::kLoadsPerWave; ++i) {
      char *kd = dst + 1024 * (wave + kPfWaves * i), *vd = kd + Gm::kTileBytes;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(ks[i]),
                                       (__attribute__((address_space(3))) void *)kd, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(vs[i]),
                                       (__attribute__((address_space(3))) void *)vd, 16, 0, 0);
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

  const int nsteps = (k_end + BN - 1) / BN;
  const int q_first = prefix + (tl.q_lo - tl.doc_start);  // position of the tile's first row
  // Operand reads.  K: lane (hl, lg) reads row 16*kb2 + hl (plus the half's
  // first key), chunk lg + 4*ch.  V^T (transposing reads): within each
  // 16-lane group, lane hl addresses key row 4*lg + hl/4 (plus the block's
  // first key) at head_dim 32*(t/2) + 8*(hl%4) + 4*(t%2), i.e. chunk
  // hl%4 + 4*(t/2), byte 8*(t%2) in it; the hardware hands lane hl the four
  // keys' values at one head_dim.  A row's position swizzle depends on the
  // row mod 16 alone, which is fixed per lane for both.
  const int fk = Gm::swz(hl), fv = Gm::swz(4 * lg + (hl >> 2));
  auto run_stage = [&](int s, const char *kb, char *nxt) {
    if (s + 1 < nsteps) dma_stage(s + 1, nxt);
    const char *vb = kb + Gm::kTileBytes;
    // S^T blocks of a 32-key half: keys key0 + 16*kb2 + (4*lg + i), columns qb.
    auto qk = [&](int h2, f32x4 (&sc)[2][kQB]) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        bf16x8 kop[D / 32];
        const char *kr = kb + (32 * h2 + 16 * kb2 + hl) * Gm::kRowBytes;
#pragma unroll
        for (int ch = 0; ch < D / 32; ++ch)
          kop[ch] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kr + (((lg + 4 * ch) ^ fk) << 4)));
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
      const int key0 = s * BN + 32 * h2;  // position of the half's first key
      const bool diag = key0 + 31 >= q_first;  // some key may lie past some query row
      const bool first = key0 == 0;  // the tile's first step: m_run is still -inf, no speculation
      // V^T operands: lane (hl, lg) of step t gets head_dim
      // d = 32*(t/2) + 8*(hl/4) + 4*(t%2) + hl%4 at keys kappa(lg, 0..3) and
      // kappa(lg, 4..7), the key order of P^T.  Read either all first, so
      // that a column block's PV products can be issued as soon as its
      // softmax is done and run on the matrix cores during the next block's,
      // or each right before its products, after every block's softmax.
      const char *v_tr = vb + (32 * h2 + 4 * lg + (hl >> 2)) * Gm::kRowBytes;
      auto read_v = [&](int t) {
        const int col = ((((hl & 3) + 4 * (t >> 1)) ^ fv) << 4) + 8 * (t & 1);
        const u32x2 lo = lds_read_tr16(v_tr + col);
        const u32x2 hi = lds_read_tr16(v_tr + 16 * Gm::kRowBytes + col);
        return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
      };
      bf16x8 vop[Tn::kJitV ? 1 : D / 16], popq[kQB];
      if constexpr (!Tn::kJitV) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) vop[t] = read_v(t);
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
        popq[qb] = as_bf16x8(pw);
        if constexpr (!Tn::kJitV) {
#pragma unroll
          for (int t = 0; t < D / 16; ++t) o[qb][t] = mfma16x16x32(vop[t], popq[qb], o[qb][t]);
        }
      }
      if constexpr (Tn::kJitV) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const bf16x8 v = read_v(t);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) o[qb][t] = mfma16x16x32(v, popq[qb], o[qb][t]);
        }
      }
    };
#pragma unroll
    for (int h2 = 0; h2 < BN / 32; ++h2) {  // 32-key steps of the stage
      if (s * BN + 32 * h2 >= k_end) break;  // uniform
      f32x4 sc[2][kQB];
      qk(h2, sc);
      softmax_pv(h2, sc);
    }
    // Stage s+1 has landed (the barrier's wait covers this wave's loads) and
    // every wave is done with stage s.  After the last stage no wave touches
    // the LDS again and each writes only its own rows, so the waves go on to
    // the epilogue without a barrier.
    if (s + 1 < nsteps) __syncthreads();
  };
  dma_stage(0, sA);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {  // two stages per pass: buffers fixed at each call
    run_stage(s, sA, sB);
    if (s + 1 < nsteps) run_stage(s + 1, sB, sA);
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

  // Fused scatter of this tile's own rows (positions prefix + q - doc_start),
  // with paged_kv_append's skip rules.  The tile has just streamed these rows
  // (its last keys), so they are read from L2; whole rows, not read again
  // here, are stored past the caches.
  if constexpr (kFused) {
    if (slot_ok) {
      const int n = (tl.q_hi - tl.q_lo) * Gm::kChunks;
      for (int p = threadIdx.x; p < n; p += kPfThreads) {
        const int q = tl.q_lo + p / Gm::kChunks, c = p % Gm::kChunks;
        const int pos = prefix + (q - tl.doc_start);
        const int blk = pos >> a.page_shift;
        if (blk >= a.max_blocks) continue;
        const int page = pt_row[blk];
        if (page <= 0 || page >= a.num_pages) continue;
        const int64_t src = ((int64_t)q * a.H_kv + g) * D + c * 8;
        const u32x4 kw = *reinterpret_cast<const u32x4 *>(a.k + src);
        const u32x4 vw = *reinterpret_cast<const u32x4 *>(a.v + src);
        const int64_t row = (int64_t)g * a.plane_rows + ((int64_t)page << a.page_shift) + (pos & page_mask);
        __builtin_nontemporal_store(kw, reinterpret_cast<u32x4 *>(a.k_pool + row * D + c * 8));
        __builtin_nontemporal_store(vw, reinterpret_cast<u32x4 *>(a.v_pool + row * D + c * 8));
      }
    }
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
