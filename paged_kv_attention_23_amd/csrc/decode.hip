// Paged decode attention (one query token per row) and the split-K merge.
//
// What is computed is the decode attention of the qwen3_flex_inference.py
// page: row r attends to logical keys 0..kv_len-1 of its slot, routed through
// the page table, with GQA (H_q / H_kv query heads per KV head) and scale.
// How it is computed is MI355X-specific:
//
//  * One workgroup of 4 waves owns a (row, KV head, split) unit and reads each
//    K/V row of its key range exactly once, serving all G query heads of that
//    KV head.  Waves interleave over 32-key tiles of the range.
//  * Scores: S^T[key][head] = K Q^T on the 16x16x32 bf16 matrix core, Q
//    held in B-operand registers for the whole unit (heads past G are zero
//    columns).  K and V rows are loaded whole (each load instruction reads
//    four complete rows) and staged in per-wave LDS tiles: reading K straight
//    into the A-operand layout (16 rows x 64 bytes per instruction) asks the
//    memory system for every cache line twice, which costs more than the
//    LDS round trip.
//  * Online softmax in base 2 in fp32 registers: each lane owns one head and
//    eight keys of the tile.  Weights are taken against a lazily moved
//    reference max; only a tile that exceeds it by the lazy threshold pays
//    for the two cross-row shuffles of the tile max and the rescale.
//  * O^T[d][head] += V^T P^T on the matrix core.  The score layout already is
//    the B operand P^T (key order permuted consistently); V^T comes from the
//    per-wave V tile through gfx950's transposing LDS reads.  Key rows in
//    both tiles are padded by 16 bytes, so the row writes, the K operand
//    reads and the transposing V reads all hit distinct banks.
//  * The contiguous fast path (flex_vs_vllm.md page, option table: blocks
//    are contiguous) replaces per-block page-table lookups with one linear
//    row base when a unit's pages are consecutive ids.
//  * Split-K (flash-decoding) writes normalised fp32 partials and their
//    log-sum-exp; a separate kernel merges them.
#include <math.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kTileKeys = 32;
constexpr float kDecLazy = 8.f;  // lazy-rescale threshold, log2 units

template <int D>
struct DecGeom {
  static constexpr int kRowStride = 2 * D + 16;  // bytes per key row in a wave's K or V tile
  static constexpr int kVBytes = kTileKeys * kRowStride;  // one wave's K (or V) tile
  static constexpr int kDChunks = D / 32;    // QK steps over head_dim
  static constexpr int kDBlocks = D / 16;    // PV output blocks over head_dim
  static constexpr int kVLoads = D / 16;     // 16-byte V loads per lane per tile
  static constexpr int kLanesPerRow = D / 8; // lanes covering one key row in a V load
  static constexpr int kKeysPerLoad = kWave / kLanesPerRow;
  static constexpr int kMergeFloats = kDecWaves * 16 * D + kDecWaves * 16 * 2;
  static constexpr int kSmemBytes = (2 * kDecWaves * kVBytes > kMergeFloats * 4)
                                        ? 2 * kDecWaves * kVBytes
                                        : kMergeFloats * 4;
};

// Where the keys of one (row, KV head) unit live.  Page ids of 64
// consecutive logical blocks starting at wbase sit one per lane in pwin, so
// a lookup is a single v_readlane with a wave-uniform index.  The window is
// loaded once per segment of at most 64 blocks (outside the tile loop, with
// an explicit wait), so the loop never waits on it.
struct RowCtx {
  const int32_t *pt_row;  // page-table row of the slot
  int contig_base;        // pool row of logical key 0 when contig
  int page_shift, num_pages, max_blocks, hi;
  int wbase;              // first logical block held in pwin
  int pwin;               // per lane: page id of block wbase + lane
  bool contig;
};

__device__ __forceinline__ void load_window(RowCtx &c, int wbase, int lane) {
  c.wbase = wbase;
  const int b = wbase + lane;
  c.pwin = (b < c.max_blocks) ? c.pt_row[b] : 0;
  __builtin_amdgcn_s_waitcnt(0);  // the window is ready before any tile uses it
}

// Pool row of the first key of a 16-key block (key0 is a multiple of 16 and
// page_size >= 16, so the block sits in one page).  Blocks wholly past the
// valid keys map to row 0, which always exists: tiles past the end are still
// loaded (so every pipeline step issues the same number of loads) but they
// all hit the same cached rows and are never used.
__device__ __forceinline__ uint32_t block_row(const RowCtx &c, int key0) {
  if (key0 >= c.hi) return 0u;
  if (c.contig) return (uint32_t)(c.contig_base + key0);
  int page = __builtin_amdgcn_readlane(c.pwin, (key0 >> c.page_shift) - c.wbase);
  page = min(max(page, 0), c.num_pages - 1);
  return ((uint32_t)page << c.page_shift) + (uint32_t)(key0 & ((1 << c.page_shift) - 1));
}

template <bool kNT>
__device__ __forceinline__ u32x4 kv_load(const char *p) {
  if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return *reinterpret_cast<const u32x4 *>(p);
}

// The 32 K (or V) rows of a tile, whole rows: load i covers keys
// i * kKeysPerLoad .. +kKeysPerLoad-1 of the tile, kLanesPerRow lanes of 16
// bytes per row.  kbase/vbase is the KV head's plane; offsets are 32-bit (a
// head plane is below 4 GiB).  K and V are streamed once per call; with kNT
// the loads are non-temporal, which pays when the call keeps the whole chip
// streaming and costs latency when it does not.
template <int D, bool kNT>
__device__ __forceinline__ void load_rows(u32x4 (&v)[D / 16], const RowCtx &c, const char *vbase,
                                          int kt, int lane) {
  using Gm = DecGeom<D>;
  const uint32_t row0 = block_row(c, kt), row1 = block_row(c, kt + 16);
  const uint32_t lane_off = (uint32_t)(lane / Gm::kLanesPerRow) * (2u * D) +
                            (uint32_t)(lane % Gm::kLanesPerRow) * 16u;
#pragma unroll
  for (int i = 0; i < Gm::kVLoads; ++i) {
    const int first = i * Gm::kKeysPerLoad;                 // first key of this load in the tile
    const uint32_t rb = (first < 16) ? row0 : row1;         // a load never straddles blocks
    v[i] = kv_load<kNT>(vbase + (rb + (first & 15)) * (2u * D) + lane_off);
  }
}

// Stage a tile's rows in one of this wave's LDS tiles.  With kZeroTail,
// keys past the range become zeros (for V: 0 * NaN would otherwise poison
// the accumulation; K rows past the range only give scores that are masked).
template <int D, bool kZeroTail>
__device__ __forceinline__ void store_rows(const u32x4 (&v)[D / 16], char *vlds, int kt, int hi,
                                           int lane) {
  using Gm = DecGeom<D>;
  const bool tail = kZeroTail && kt + kTileKeys > hi;
#pragma unroll
  for (int i = 0; i < Gm::kVLoads; ++i) {
    const int key = i * Gm::kKeysPerLoad + lane / Gm::kLanesPerRow;
    u32x4 val = v[i];
    if (tail && kt + key >= hi) val = u32x4{0u, 0u, 0u, 0u};
    const int off = key * Gm::kRowStride + (lane % Gm::kLanesPerRow) * 16;
    *reinterpret_cast<u32x4 *>(vlds + off) = val;
  }
}

template <int D>
__device__ __forceinline__ void compute_tile(const char *klds, int kt, int hi, const char *vlds,
                                             const bf16x8 *qop, float &m_run, float &l_run,
                                             f32x4 *o, float scale_log2, int lane) {
  using Gm = DecGeom<D>;
  const int hl = lane & 15, lg = lane >> 4;
  const bool tail = kt + kTileKeys > hi;

  // 1) scores for two 16-key blocks: S^T = K Q^T.  A-operand lane (hl, lg)
  //    of step ch holds key hl (+16) at head_dim 32*ch + 8*lg .. +7.
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  const char *k_op = klds + hl * Gm::kRowStride + 16 * lg;
#pragma unroll
  for (int ch = 0; ch < Gm::kDChunks; ++ch) {
    const u32x4 k0 = *reinterpret_cast<const u32x4 *>(k_op + 64 * ch);
    const u32x4 k1 = *reinterpret_cast<const u32x4 *>(k_op + 16 * Gm::kRowStride + 64 * ch);
    s0 = mfma16x16x32(as_bf16x8(k0), qop[ch], s0);
    s1 = mfma16x16x32(as_bf16x8(k1), qop[ch], s1);
  }

  // 2) online softmax, base 2.  Lane holds keys 4*lg+i (block 0) and
  //    16+4*lg+i (block 1) of head hl.
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i] * scale_log2;
    x[4 + i] = s1[i] * scale_log2;
  }
  if (tail) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = kt + (i < 4 ? 4 * lg + i : 16 + 4 * lg + (i - 4));
      if (key >= hi) x[i] = -INFINITY;
    }
  }
  // Weights against the running reference m_run, computed straight away;
  // the reference moves (cross-lane max, rescale, recompute) only when some
  // lane's scores exceed it by more than kDecLazy (log2 units), so the
  // common tile has no cross-lane step and no accumulator rescale.
  float lm = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) lm = fmaxf(lm, x[i]);
  float p[8];
  {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(x[i] - m_use);
  }
  if (__any(lm > m_run + kDecLazy)) {
    float mt = max_xor16(lm);
    mt = max_xor32(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while m_run = -inf
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < Gm::kDBlocks; ++t) o[t] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(x[i] - m_use);
  }
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) psum += p[i];
  l_run += psum;

  // 3) P^T is already in B-operand form: element e of k-group lg is key
  //    kappa(lg, e) = e < 4 ? 4*lg + e : 16 + 4*lg + (e - 4).
  const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                    pack_bf16x2(p[6], p[7])};
  const bf16x8 pop = as_bf16x8(pw);

  // 4) O^T += V^T P^T with V^T operands from transposing LDS reads.  In
  //    each 16-lane group, lane hl addresses key row 4*lg + hl/4 (plus 16
  //    for the second read) at head_dim 4*NT*(hl%4) + 4*t, and receives one
  //    head_dim value at four consecutive keys: step t's A-operand row hl is
  //    d = 4*NT*(hl/4) + 4*t + hl%4, keys kappa(lg, 0..7) in P^T's order.
  //    Accumulator (t, i) of lane (hl, lg) is therefore
  //    O[head hl][4*NT*lg + 4*t + i].
  constexpr int NT = Gm::kDBlocks;
  const char *v_tr = vlds + (4 * lg + (hl >> 2)) * Gm::kRowStride + 8 * NT * (hl & 3);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const u32x2 lo = lds_read_tr16(v_tr + 8 * t);
    const u32x2 hi = lds_read_tr16(v_tr + 16 * Gm::kRowStride + 8 * t);
    o[t] = mfma16x16x32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pop, o[t]);
  }
}

// Where one piece's result goes: G rows of D values (row stride D) and G
// log-sum-exps (natural log).  Final results are bf16 rows of the output;
// partial results are normalised fp32 rows in the workspace.
struct PieceOut {
  void *o;
  float *lse;
  bool final_;
};

__device__ __forceinline__ PieceOut final_out(const DecodeArgs &a, int r, int g) {
  const int64_t rh = (int64_t)r * a.H_q + (int64_t)g * a.G;
  return PieceOut{a.out + rh * a.D, a.lse + rh, true};
}

// A piece with no valid key: O = +0, LSE = -inf (a partial with LSE = -inf
// gets weight zero in the merge).
__device__ void write_empty(const PieceOut &dst, int G, int D) {
  const int pairs = G * (D >> 1);
  for (int idx = threadIdx.x; idx < pairs; idx += kDecThreads) {
    const int hh = idx / (D >> 1);
    const int d = 2 * (idx % (D >> 1));
    if (dst.final_)
      *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(dst.o) + hh * D + d) = 0u;
    else
      *reinterpret_cast<f32x2 *>(reinterpret_cast<float *>(dst.o) + hh * D + d) = f32x2{0.f, 0.f};
    if (d == 0) dst.lse[hh] = -INFINITY;
  }
}

// Attention of the G query heads of KV head g in row r over the row's keys
// [lo, hi) (0 <= lo < hi <= n), all four waves of the workgroup together.
// s is the row's slot (valid).  With with_new (fused append, hi == n), key
// n-1 is the caller's new token: it is attended from k_new/v_new rather than
// the pool, and written into its page.  Ends with a workgroup barrier, so the
// caller may start another piece right away.
template <int D, bool kFused, bool kEarlyNew, bool kNT>
__device__ void decode_piece(const DecodeArgs &a, char *smem, int r, int g, int s, int lo, int hi,
                             bool with_new, const PieceOut &dst, int lane, int wave) {
  if constexpr (!kFused) with_new = false;
  using Gm = DecGeom<D>;
  constexpr int NT = Gm::kDBlocks;
  const int hl = lane & 15, lg = lane >> 4;
  const int G = a.G;

  // Q^T as B operands: column hl = query head g*G + hl (zero past G).
  bf16x8 qop[Gm::kDChunks];
  {
    const uint16_t *qr = a.q + ((int64_t)r * a.H_q + g * G + hl) * D + 8 * lg;
#pragma unroll
    for (int ch = 0; ch < Gm::kDChunks; ++ch) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (hl < G) w = *reinterpret_cast<const u32x4 *>(qr + 32 * ch);
      qop[ch] = as_bf16x8(w);
    }
  }

  // New token: K in the Q operand layout (dims 8*lg + 32*ch), V in the
  // accumulator layout (dims NT*4*lg .. NT*4*lg + D/4 - 1).  With kEarlyNew
  // they are loaded before the key loop (their latency hides behind it, at
  // the cost of registers held through it); otherwise after it.
  u32x4 kq[D / 32], vq[D / 32];
  int new_page = 0;
  auto load_new = [&]() {
    const int64_t nrow = ((int64_t)r * a.H_kv + g) * D;
#pragma unroll
    for (int ch = 0; ch < D / 32; ++ch) {
      kq[ch] = *reinterpret_cast<const u32x4 *>(a.k_new + nrow + 8 * lg + 32 * ch);
      vq[ch] = *reinterpret_cast<const u32x4 *>(a.v_new + nrow + NT * 4 * lg + 8 * ch);
    }
    new_page = a.page_table[(int64_t)s * a.max_blocks + (hi >> a.page_shift)];
  };
  // Wave 0's lanes of column 0 write the new K and V rows into their page
  // where paged_kv_append would (a mapped page of this pool).
  auto write_new = [&]() {
    if (hl == 0 && new_page > 0 && new_page < a.num_pages) {
      const int64_t prow = (int64_t)g * a.plane_rows + ((int64_t)new_page << a.page_shift) +
                           (hi & ((1 << a.page_shift) - 1));  // hi = n - 1 by then
#pragma unroll
      for (int ch = 0; ch < D / 32; ++ch) {
        *reinterpret_cast<u32x4 *>(a.k_pool_w + prow * D + 8 * lg + 32 * ch) = kq[ch];
        *reinterpret_cast<u32x4 *>(a.v_pool_w + prow * D + NT * 4 * lg + 8 * ch) = vq[ch];
      }
    }
  };
  // Score of the new token for head hl, base 2: q . k_new from the Q operand
  // registers (fp32 products of bf16 values), summed over the lg lanes.
  auto new_score = [&]() {
    float dot = 0.f;
#pragma unroll
    for (int ch = 0; ch < D / 32; ++ch) {
      const u32x4 qw = __builtin_bit_cast(u32x4, qop[ch]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dot = fmaf(bf16_lo(qw[j]), bf16_lo(kq[ch][j]), dot);
        dot = fmaf(bf16_hi(qw[j]), bf16_hi(kq[ch][j]), dot);
      }
    }
    dot = sum_xor16(dot);
    dot = sum_xor32(dot);
    return dot * a.scale_log2;
  };
  if (with_new) {
    hi -= 1;  // the pool supplies keys [lo, n-1); key n-1 is the new token
    if constexpr (kEarlyNew) {
      if (wave == 0) load_new();
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[Gm::kDBlocks];
#pragma unroll
  for (int t = 0; t < Gm::kDBlocks; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (lo < hi) {
  // Where this piece's keys live; detect consecutive page ids (one wave vote).
  RowCtx c;
  c.pt_row = a.page_table + (int64_t)s * a.max_blocks;
  c.page_shift = a.page_shift;
  c.num_pages = a.num_pages;
  c.max_blocks = a.max_blocks;
  c.hi = hi;
  c.contig = false;
  c.contig_base = 0;
  const int blk_lo = lo >> a.page_shift;
  load_window(c, blk_lo, lane);
  if (a.contig_mode != 2) {
    const int nb = ((hi - 1) >> a.page_shift) - blk_lo + 1;
    const int first = __builtin_amdgcn_readfirstlane(c.pwin);
    bool ok = first >= 0 && first + nb <= a.num_pages;
    if (a.contig_mode == 0 && ok) {
      ok = __all(lane >= nb || c.pwin == first + lane);
      for (int b0 = kWave; b0 < nb && ok; b0 += kWave) {
        const int b = b0 + lane;
        ok = __all(b >= nb || c.pt_row[blk_lo + b] == first + b);
      }
    }
    c.contig = ok;
    c.contig_base = (first - blk_lo) << a.page_shift;
  }

  const char *kbase = reinterpret_cast<const char *>(a.k_pool + (int64_t)g * a.plane_rows * D);
  const char *vbase = reinterpret_cast<const char *>(a.v_pool + (int64_t)g * a.plane_rows * D);

  char *klds = smem + (2 * wave) * Gm::kVBytes;
  char *vlds = smem + (2 * wave + 1) * Gm::kVBytes;

  // The key range is walked in segments of at most 64 blocks (one page-id
  // window each; a single segment when the pages are contiguous).  Within a
  // segment, a software pipeline keeps the next tile's K and V (staging
  // registers) in flight while the current tile, already in LDS, is computed.
  u32x4 kr[D / 16], vr[D / 16];
  for (int seg_lo = lo; seg_lo < hi;) {
    const int seg_blk = seg_lo >> a.page_shift;
    const int seg_hi = c.contig ? hi
                                : (int)min((int64_t)hi, ((int64_t)seg_blk + kWave) << a.page_shift);
    if (!c.contig && seg_blk != c.wbase) load_window(c, seg_blk, lane);
    c.hi = seg_hi;
    const int ntiles = (seg_hi - seg_lo + kTileKeys - 1) / kTileKeys;
    int t = wave;
    load_rows<D, kNT>(vr, c, vbase, seg_lo + t * kTileKeys, lane);
    load_rows<D, kNT>(kr, c, kbase, seg_lo + t * kTileKeys, lane);
    while (t < ntiles) {
      store_rows<D, true>(vr, vlds, seg_lo + t * kTileKeys, seg_hi, lane);
      store_rows<D, false>(kr, klds, seg_lo + t * kTileKeys, seg_hi, lane);
      const int tn = t + kDecWaves;
      load_rows<D, kNT>(vr, c, vbase, seg_lo + tn * kTileKeys, lane);
      load_rows<D, kNT>(kr, c, kbase, seg_lo + tn * kTileKeys, lane);
      compute_tile<D>(klds, seg_lo + t * kTileKeys, seg_hi, vlds, qop, m_run, l_run, o,
                      a.scale_log2, lane);
      t = tn;
    }
    seg_lo = seg_hi;
  }
  }  // lo < hi

  // The new token joins wave 0's running state: score from the Q operand
  // registers (fp32 products of bf16 values), weight p in fp32; then its
  // rows are written.
  if (with_new && wave == 0) {
    if constexpr (!kEarlyNew) load_new();
    const float x = new_score();
    const float m_new = fmaxf(m_run, x);
    const float alpha = fast_exp2(m_run - m_new);  // 0 while m_run = -inf
    const float pn = fast_exp2(x - m_new);
    l_run = l_run * alpha + (lg == 0 ? pn : 0.f);  // l is summed over lg below
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int k = 4 * t + i;  // element of this lane's D/4 new-V values
        const uint32_t w = vq[k >> 3][(k >> 1) & 3];
        o[t][i] = o[t][i] * alpha + pn * ((k & 1) ? bf16_hi(w) : bf16_lo(w));
      }
    m_run = m_new;
    write_new();
  }

  // Combine the 4 waves through LDS (the merge area reuses the V tiles).
  l_run = sum_xor16(l_run);
  l_run = sum_xor32(l_run);
  __syncthreads();
  float *mo = reinterpret_cast<float *>(smem);        // [wave][16 heads][D]
  float *mm = mo + kDecWaves * 16 * D;                // [wave][16]
  float *ml = mm + kDecWaves * 16;                    // [wave][16]
  if (hl < G) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<f32x4 *>(mo + (wave * 16 + hl) * D + 4 * NT * lg + 4 * tt) = o[tt];
    if (lg == 0) {
      mm[wave * 16 + hl] = m_run;
      ml[wave * 16 + hl] = l_run;
    }
  }
  __syncthreads();

  const int pairs = G * (D / 2);
  for (int idx = threadIdx.x; idx < pairs; idx += kDecThreads) {
    const int hh = idx / (D / 2);
    const int d = 2 * (idx % (D / 2));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mm[w * 16 + hh]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = mm[w * 16 + hh];
      const float wt = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      L += wt * ml[w * 16 + hh];
      const f32x2 ov = *reinterpret_cast<const f32x2 *>(mo + (w * 16 + hh) * D + d);
      o0 += wt * ov[0];
      o1 += wt * ov[1];
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    const float lse_nat = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
    if (dst.final_)
      *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(dst.o) + hh * D + d) =
          pack_bf16x2(o0 * inv, o1 * inv);
    else
      *reinterpret_cast<f32x2 *>(reinterpret_cast<float *>(dst.o) + hh * D + d) =
          f32x2{o0 * inv, o1 * inv};
    if (d == 0) dst.lse[hh] = lse_nat;
  }
  __syncthreads();  // the LDS is free for the next piece
}

// Valid keys of row r (0 for padding rows: slot 0 / out of range / kv_len <= 0),
// clamped to the page table's capacity.  has_new: with a fused append, the
// row's new token (position kv_len - 1) lies inside that capacity.
__device__ __forceinline__ int row_keys(const DecodeArgs &a, int r, int &slot, bool &has_new) {
  const int s = a.batch_idx[r];
  const int raw = a.kv_len[r];
  const int cap = a.max_blocks << a.page_shift;
  const int n = min(raw, cap);
  slot = s;
  const bool live = !(s <= 0 || s >= a.num_slots || n <= 0);
  has_new = live && a.k_new != nullptr && raw <= cap;
  return live ? n : 0;
}

// Per-row schedule: blockIdx.x enumerates (split, KV head, row), split
// fastest; split sp of a row covers an equal share of its keys in whole
// 32-key tiles.  With one split the result is final, else a partial.
template <int D, bool kFused, bool kNT>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_rows_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DecGeom<D>::kSmemBytes];
  const int S = a.num_splits;
  const int sp = blockIdx.x % S;
  const int g = (blockIdx.x / S) % a.H_kv;
  const int r = blockIdx.x / (S * a.H_kv);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  int s;
  bool has_new;
  const int n = row_keys(a, r, s, has_new);
  const int chunk = ((n + S - 1) / S + kTileKeys - 1) & ~(kTileKeys - 1);
  const int64_t lo64 = (int64_t)sp * chunk;
  const int lo = (int)min(lo64, (int64_t)n);
  const int hi = (sp == S - 1) ? n : (int)min((int64_t)n, lo64 + chunk);
  PieceOut dst = final_out(a, r, g);
  if (S > 1) {
    const int64_t prh = ((int64_t)sp * a.B + r) * a.H_q + (int64_t)g * a.G;
    dst = PieceOut{a.o_part + prh * D, a.lse_part + prh, false};
  }
  if (lo >= hi) {
    write_empty(dst, a.G, D);
    return;
  }
  const bool with_new = has_new && hi == n;
  decode_piece<D, kFused, true, kNT>(a, smem, r, g, s, lo, hi, with_new, dst, lane, wave);
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One step of the wave scan below on a 64-bit value: the DPP move of both
// halves (0 where the source lane is outside the row or the row is masked).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int64_t dpp_move64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, kRowMask, 0xf, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)v >> 32), kCtrl, kRowMask, 0xf, false);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: four row
// shifts give the sums within each 16-lane row, then the last lane of row 0
// is added to row 1 and of row 2 to row 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ int64_t wave_incl_scan64(int64_t v, int) {
  v += dpp_move64<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move64<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move64<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move64<0x118, 0xf>(v);  // row_shr:8
  v += dpp_move64<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3
  v += dpp_move64<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Sum over the wave, returned as a wave-uniform (scalar) value.
__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
  return readlane64(wave_incl_scan64(v, 0), kWave - 1);
}

// Balanced schedule (flash-decoding with split points balanced across rows).
// For KV head g, the 32-key tiles of all rows, row after row, form one list of
// TT tiles; workgroup w takes tiles [TT*w/W', TT*(w+1)/W') with W' = min(W, TT),
// so every workgroup streams the same number of tiles whatever the row
// lengths.  A row wholly inside one range is written as the final result; a
// row cut by range boundaries leaves one normalised partial per workgroup, in
// slot 0 (the row holding the range's first tile) or slot 1 (the row holding
// its last tile), and the workgroup holding the row's first tile records the
// row in its descriptor for the merge kernel.  Padding rows (no tiles) are
// written by the workgroup whose range holds their position in the list (the
// last workgroup for positions at the end).  Every workgroup recomputes the
// row prefix sums itself (batch_idx / kv_len are a few cached lines), so the
// plan needs no extra launch.  Everything but the lanes' prefix ends is kept
// in scalar registers across the pieces.
template <int D, bool kFused>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_balanced_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DecGeom<D>::kSmemBytes];
  const int g = blockIdx.x % a.H_kv;
  const int w = blockIdx.x / a.H_kv;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = a.num_splits;

  // Pass 1: total tiles.  The lanes' rows of the first 64-row chunk stay in
  // registers for pass 2 (a batch of up to 64 rows is read once).
  int64_t TT = 0;
  int s_first = 0, n_first = 0;
  for (int cb = 0; cb < a.B; cb += kWave) {
    int s = 0, n = 0;
    bool hn = false;
    if (cb + lane < a.B) n = row_keys(a, cb + lane, s, hn);
    n |= hn ? 0 : INT32_MIN;  // bit 31: no fused new token for this row
    if (cb == 0) {
      s_first = s;
      n_first = n;
    }
    TT += wave_sum64(((n & INT32_MAX) + kTileKeys - 1) / kTileKeys);
  }
  const int We = (int)min<int64_t>(W, TT);
  const int last_owner = max(We - 1, 0);
  int desc_r = -1, desc_slot = 0, desc_last = 0;
  if (w < We || w == last_owner) {
    const int64_t t0 = We ? TT * w / We : 0;
    const int64_t t1 = We ? TT * (w + 1) / We : 0;
    int64_t carry = 0;
    for (int cb = 0; cb < a.B && carry <= t1; cb += kWave) {
      const int r = cb + lane;
      int s = s_first, n = n_first;
      if (cb != 0) {
        bool hn = false;
        n = 0;
        if (r < a.B) n = row_keys(a, r, s, hn);
        n |= hn ? 0 : INT32_MIN;
      }
      uint64_t mask;
      int64_t pe;  // end of the lane's row in the tile list
      {
        const int tiles = ((n & INT32_MAX) + kTileKeys - 1) / kTileKeys;
        pe = carry + wave_incl_scan64(tiles, lane);
        const int64_t ps = pe - tiles;
        bool mine = false;
        if (r < a.B) {
          if (tiles > 0) mine = pe > t0 && ps < t1;
          else mine = (ps >= t0 && ps < t1) || (ps == TT && w == last_owner);
        }
        mask = __ballot(mine);
      }
      carry = readlane64(pe, kWave - 1);
      while (mask) {
        const int j = __builtin_ctzll(mask);
        mask &= mask - 1;
        const int rr = cb + j;
        const int sj = __builtin_amdgcn_readlane(s, j);
        const int nenc = __builtin_amdgcn_readlane(n, j);
        const int nj = nenc & INT32_MAX;
        const bool hnj = nenc >= 0;
        const int64_t ej = readlane64(pe, j);
        const int64_t pj = ej - (nj + kTileKeys - 1) / kTileKeys;
        if (nj == 0) {
          write_empty(final_out(a, rr, g), a.G, D);
          continue;
        }
        const int64_t klo = max(pj, t0), khi = min(ej, t1);
        const int lo = (int)(klo - pj) * kTileKeys;
        const int hi = (int)min<int64_t>(nj, (khi - pj) * kTileKeys);
        PieceOut dst = final_out(a, rr, g);
        if (pj < t0 || ej > t1) {
          const int slot = (pj <= t0) ? 0 : 1;
          const int64_t pidx = (((int64_t)g * W + w) * 2 + slot) * a.G;
          dst = PieceOut{a.o_part + pidx * D, a.lse_part + pidx, false};
          if (pj >= t0) {  // this range holds the row's first tile: it owns the merge
            desc_r = rr;
            desc_slot = slot;
            desc_last = (int)((ej * We + TT - 1) / TT) - 1;  // range holding tile ej-1
          }
        }
        decode_piece<D, kFused, false, true>(a, smem, rr, g, sj, lo, hi, hnj && hi == nj, dst, lane, wave);
      }
    }
  }
  if (threadIdx.x == 0) a.desc[(int64_t)g * W + w] = int4{desc_r, desc_slot, desc_last, 0};
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Merge of per-row split partials: one wave per (row, query head).
//   M = max_s L_s; LSE = M + ln sum_s exp(L_s - M); O = sum_s exp(L_s - LSE) O_s
// Partials with L_s = -inf carry weight zero and are not read.
template <int D>
__global__ __launch_bounds__(256) void merge_rows_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t rh = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  const int64_t nrh = (int64_t)a.B * a.H_q;
  if (rh >= nrh) return;
  const int S = a.num_splits;
  constexpr int kPer = D / kWave;  // elements of head_dim per lane
  // The first kPre splits' partials are loaded together with the LSEs (they
  // do not depend on the weights), so the merge waits for one memory round
  // trip rather than two.
  constexpr int kPre = 8;
  float pre[kPre][kPer];
#pragma unroll
  for (int s = 0; s < kPre; ++s) {
    const float *op = a.o_part + ((int64_t)s * nrh + rh) * D + lane * kPer;
#pragma unroll
    for (int k = 0; k < kPer; ++k) pre[s][k] = (s < S) ? op[k] : 0.f;
  }
  // Lane s < S holds split s's LSE; the max, the sum and the weights are
  // wave-uniform, read lane by lane (S is at most 64) rather than through
  // cross-lane shuffles.
  const float ls = (lane < S) ? a.lse_part[(int64_t)lane * nrh + rh] : -INFINITY;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, readlane_f(ls, s));
  if (M == -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) a.out[rh * D + lane * kPer + k] = 0;
    if (lane == 0) a.lse[rh] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int s = 0; s < S; ++s) {
    const float Ls = readlane_f(ls, s);
    if (Ls != -INFINITY) sum += expf(Ls - M);
  }
  const float L = M + logf(sum);
  const float w = (ls == -INFINITY) ? 0.f : expf(ls - L);
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;
#pragma unroll
  for (int s = 0; s < kPre; ++s) {
    if (s >= S) break;
    const float ws = readlane_f(w, s);
    if (ws == 0.f) continue;  // uniform
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] += ws * pre[s][k];
  }
  for (int s = kPre; s < S; ++s) {
    const float ws = readlane_f(w, s);
    if (ws == 0.f) continue;  // uniform
    const float *op = a.o_part + ((int64_t)s * nrh + rh) * D + lane * kPer;
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] += ws * op[k];
  }
  if (kPer == 2) {
    *reinterpret_cast<uint32_t *>(a.out + rh * D + lane * 2) = pack_bf16x2(acc[0], acc[kPer - 1]);
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      a.out[rh * D + lane * kPer + k] = (uint16_t)(pack_bf16x2(acc[k], 0.f) & 0xffffu);
  }
  if (lane == 0) a.lse[rh] = L;
}

// Merge of the balanced schedule's cut rows: one workgroup per (KV head,
// range b).  Range b's descriptor names the cut row whose first tile it holds
// (if any) and the last range that row reaches; the partials are those of
// ranges b .. last (slot desc.y for b, slot 0 for the others).  Each thread
// owns two adjacent outputs of one query head and folds the partials in
// range order with a running maximum:
//   M' = max(M, L_w);  S' = S e^(M-M') + e^(L_w-M');  O' = O e^(M-M') + e^(L_w-M') O_w
// which ends at O = sum_w e^(L_w) O_w / sum_w e^(L_w) and LSE = M + ln S.
// The loads of different ranges do not depend on each other, so unrolling
// keeps several in flight.
template <int D>
__global__ __launch_bounds__(256) void merge_balanced_kernel(DecodeArgs a) {
  const int W = a.num_splits;
  const int g = blockIdx.x % a.H_kv;
  const int b = blockIdx.x / a.H_kv;
  const int4 desc = a.desc[(int64_t)g * W + b];
  const int r = desc.x;
  if (r < 0) return;
  const int wl = min(desc.z, W - 1);
  const int G = a.G;
  const int pairs = G * (D / 2);
  for (int idx = threadIdx.x; idx < pairs; idx += 256) {
    const int hh = idx / (D / 2);
    const int d = 2 * (idx % (D / 2));
    float M = -INFINITY, S = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 4
    for (int w = b; w <= wl; ++w) {
      const int slot = (w == b) ? desc.y : 0;
      const int64_t pidx = (((int64_t)g * W + w) * 2 + slot) * G + hh;
      const float L = a.lse_part[pidx];
      const f32x2 ov = *reinterpret_cast<const f32x2 *>(a.o_part + pidx * D + d);
      if (L == -INFINITY) continue;
      const float Mn = fmaxf(M, L);
      const float keep = (M == -INFINITY) ? 0.f : expf(M - Mn);
      const float add = expf(L - Mn);
      S = S * keep + add;
      o0 = o0 * keep + add * ov[0];
      o1 = o1 * keep + add * ov[1];
      M = Mn;
    }
    const float inv = (S > 0.f) ? 1.f / S : 0.f;
    const int64_t rh = (int64_t)r * a.H_q + (int64_t)g * G + hh;
    *reinterpret_cast<uint32_t *>(a.out + rh * D + d) = pack_bf16x2(o0 * inv, o1 * inv);
    if (d == 0) a.lse[rh] = (S > 0.f) ? M + logf(S) : -INFINITY;
  }
}

template <int D, bool kFused>
static void launch_main(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
  // The balanced schedule serves long contexts and always streams; the
  // per-row schedule streams non-temporally when its units fill the chip.
  if (a.balanced)
    hipLaunchKernelGGL((decode_balanced_kernel<D, kFused>), grid, dim3(kDecThreads), 0, stream, a);
  else if (a.stream_nt)
    hipLaunchKernelGGL((decode_rows_kernel<D, kFused, true>), grid, dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_rows_kernel<D, kFused, false>), grid, dim3(kDecThreads), 0, stream, a);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const bool balanced = a.balanced != 0;
  const bool fused = a.k_new != nullptr;
  const dim3 grid((unsigned)((int64_t)a.num_splits * a.H_kv * (balanced ? 1 : a.B)));
  if (a.D == 128)
    fused ? launch_main<128, true>(a, grid, stream) : launch_main<128, false>(a, grid, stream);
  else
    fused ? launch_main<64, true>(a, grid, stream) : launch_main<64, false>(a, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  if (balanced) {
    const unsigned mblocks = (unsigned)((int64_t)a.H_kv * (a.num_splits - 1));  // last range owns no merge
    if (a.D == 128)
      hipLaunchKernelGGL(merge_balanced_kernel<128>, dim3(mblocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(merge_balanced_kernel<64>, dim3(mblocks), dim3(256), 0, stream, a);
  } else {
    const int64_t nrh = (int64_t)a.B * a.H_q;
    const unsigned mblocks = (unsigned)((nrh + 3) / 4);
    if (a.D == 128)
      hipLaunchKernelGGL(merge_rows_kernel<128>, dim3(mblocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(merge_rows_kernel<64>, dim3(mblocks), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv
