/*
 * CPU reference ("oracle") for grouped-query attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code with the HIP kernels.
 *
 * Every result is computed from its plain definition, in float64, without
 * blocking, fusion or reordering: gather the valid keys of a row through the
 * page table, then take an ordinary max-shifted softmax over them.
 *
 * Sources (page titles of the reference pages):
 *  - flex paged-attention commit, "Why this works" 1-3: the cache is one
 *    contiguous [1, H, num_pages*page_size, D] tensor per K and V; a page
 *    table maps (logical batch, logical block) to a physical page; batch
 *    slot 0 and page 0 are reserved padding.
 *  - qwen3_flex_inference.py, attention forward: the cache update
 *    (update(input_pos, k, v, batch_idx)) runs before attention;
 *    attention is flex_attention with scale = self.scaling and GQA enabled.
 *  - qwen3_flex_inference.py, decode block mask: a decode row attends to the
 *    keys at logical positions 0..input_pos (causal offset), so kv_len =
 *    input_pos + 1 keys are valid.
 *  - qwen3_flex_inference.py, prefill: prompts are packed into one sequence
 *    and masked document-causally (each token sees its own document's
 *    tokens up to itself).
 *  - flex_vs_vllm.md results page, "What broke correctness": a padded row has
 *    no valid key at all and must not produce NaN.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - LSE is the natural log of sum_j exp(scale * q.k_j); a row with no valid
 *    key returns O = +0.0 and LSE = -inf.
 *  - Query head h reads KV head h / (H_q / H_kv) (consecutive query heads
 *    share a KV head).
 *  - The scale multiplies the exact dot product of the bf16 inputs.
 *  - An appended token whose slot is 0, whose block has page 0, or whose
 *    slot / block / page lies outside the table or pool is not written.
 *
 * Parity pins live in tests/test_oracle_pins.py.  Build:
 *   gcc -O2 -fopenmp -fPIC -shared -std=c11 oracle.c -o liboracle.so -lm
 * (no -ffast-math: the arithmetic must stay IEEE float64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* A bfloat16 is the upper 16 bits of an IEEE binary32: widen exactly. */
static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * KV append (scatter).  For token t with slot s = batch_idx[t] and logical
 * position p = input_pos[t], the physical row is
 *     page_table[s][p / page_size] * page_size + p % page_size
 * and K/V of every KV head are copied bit for bit into that row of the pool.
 * Pools are [H_kv][num_pages*page_size][D]; k_new/v_new are [N][H_kv][D].
 */
int oracle_append(uint16_t *k_pool, uint16_t *v_pool, int num_pages, int page_size,
                  int H_kv, int D, const int32_t *page_table, int num_slots, int max_blocks,
                  const int32_t *batch_idx, const int32_t *input_pos, int N,
                  const uint16_t *k_new, const uint16_t *v_new)
{
    if (num_pages <= 0 || page_size <= 0 || H_kv <= 0 || D <= 0 || max_blocks <= 0 || N < 0)
        return ORC_EINVAL;
    const int64_t plane = (int64_t)num_pages * page_size;
    for (int t = 0; t < N; ++t) {
        int s = batch_idx[t];
        int p = input_pos[t];
        if (s <= 0 || s >= num_slots || p < 0) continue;          /* padding slot or no such slot */
        int blk = p / page_size;
        if (blk >= max_blocks) continue;
        int page = page_table[(int64_t)s * max_blocks + blk];
        if (page <= 0 || page >= num_pages) continue;            /* reserved page 0 / unmapped */
        int64_t row = (int64_t)page * page_size + p % page_size;
        for (int h = 0; h < H_kv; ++h) {
            memcpy(&k_pool[((int64_t)h * plane + row) * D], &k_new[((int64_t)t * H_kv + h) * D],
                   sizeof(uint16_t) * (size_t)D);
            memcpy(&v_pool[((int64_t)h * plane + row) * D], &v_new[((int64_t)t * H_kv + h) * D],
                   sizeof(uint16_t) * (size_t)D);
        }
    }
    return ORC_OK;
}

/*
 * Softmax attention of one query vector over n gathered keys (float64):
 *   x_j = scale * sum_d q[d] K[j][d]
 *   m = max_j x_j,   l = sum_j exp(x_j - m)
 *   LSE = m + ln l,  O[d] = sum_j exp(x_j - m) V[j][d] / l
 * n == 0 gives O = 0 and LSE = -inf.  x is caller scratch of n doubles.
 */
static void softmax_attend(const double *q, const double *K, const double *V, int n, int D,
                           double scale, double *x, double *out, double *lse)
{
    if (n <= 0) {
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += q[d] * K[(int64_t)j * D + d];
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
        x[j] = exp(x[j] - m);
        l += x[j];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j) acc += x[j] * V[(int64_t)j * D + d];
        out[d] = acc / l;
    }
    *lse = m + log(l);
}

/*
 * Decode attention over keys [key_lo[r], key_hi[r]) of each row (one query
 * token per row).  The full decode uses key_lo = 0 and key_hi = kv_len; a
 * split-K partial uses a sub-range.  Row r is padding when batch_idx[r] == 0
 * or its range is empty: O = +0.0 and LSE = -inf for every head.
 *
 * q: bf16 [B][H_q][D]; pools: bf16 [H_kv][num_pages*page_size][D];
 * page_table: [num_slots][max_blocks]; out: f64 [B][H_q][D]; lse: f64 [B][H_q].
 * Returns ORC_EINVAL (and writes nothing) if any active row would read a
 * block, page or slot outside the table or pool.
 */
int oracle_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                  int num_pages, int page_size, int H_kv, int D, const int32_t *page_table,
                  int num_slots, int max_blocks, const int32_t *batch_idx,
                  const int32_t *key_lo, const int32_t *key_hi, int B, int H_q, double scale,
                  double *out, double *lse)
{
    if (num_pages <= 0 || page_size <= 0 || H_kv <= 0 || D <= 0 || B < 0 || H_q <= 0 ||
        H_q % H_kv != 0)
        return ORC_EINVAL;
    const int G = H_q / H_kv;
    const int64_t plane = (int64_t)num_pages * page_size;
    /* check every address first */
    for (int r = 0; r < B; ++r) {
        int s = batch_idx[r];
        if (s == 0 || key_hi[r] <= key_lo[r]) continue;
        if (s < 0 || s >= num_slots || key_lo[r] < 0) return ORC_EINVAL;
        if ((int64_t)(key_hi[r] - 1) / page_size >= max_blocks) return ORC_EINVAL;
        for (int j = key_lo[r]; j < key_hi[r]; ++j) {
            int page = page_table[(int64_t)s * max_blocks + j / page_size];
            if (page < 0 || page >= num_pages) return ORC_EINVAL;
        }
    }
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int r = 0; r < B; ++r) {
        for (int g = 0; g < H_kv; ++g) {
            int s = batch_idx[r];
            int lo = key_lo[r], hi = key_hi[r];
            int n = (s == 0 || hi <= lo) ? 0 : hi - lo;
            double *K = NULL, *V = NULL, *x = NULL;
            double *qd = (double *)malloc(sizeof(double) * (size_t)D);
            if (n > 0) {
                K = (double *)malloc(sizeof(double) * (size_t)n * D);
                V = (double *)malloc(sizeof(double) * (size_t)n * D);
                x = (double *)malloc(sizeof(double) * (size_t)n);
            }
            if (!qd || (n > 0 && (!K || !V || !x))) {
#pragma omp atomic write
                err = 1;
            } else {
                /* gather: logical key j -> physical row through the page table */
                for (int i = 0; i < n; ++i) {
                    int j = lo + i;
                    int page = page_table[(int64_t)s * max_blocks + j / page_size];
                    int64_t row = (int64_t)page * page_size + j % page_size;
                    const uint16_t *kr = &k_pool[((int64_t)g * plane + row) * D];
                    const uint16_t *vr = &v_pool[((int64_t)g * plane + row) * D];
                    for (int d = 0; d < D; ++d) {
                        K[(int64_t)i * D + d] = bf16_to_f64(kr[d]);
                        V[(int64_t)i * D + d] = bf16_to_f64(vr[d]);
                    }
                }
                for (int hh = 0; hh < G; ++hh) {
                    int h = g * G + hh;
                    const uint16_t *qr = &q[((int64_t)r * H_q + h) * D];
                    for (int d = 0; d < D; ++d) qd[d] = bf16_to_f64(qr[d]);
                    softmax_attend(qd, K, V, n, D, scale, x, &out[((int64_t)r * H_q + h) * D],
                                   &lse[(int64_t)r * H_q + h]);
                }
            }
            free(qd);
            free(K);
            free(V);
            free(x);
        }
    }
    return err ? ORC_EINVAL : ORC_OK;
}

/*
 * Merge of split-K partials.  For each (row, head), over S partials with
 * log-sum-exps L_s and normalised outputs O_s:
 *   M = max_s L_s;  if M = -inf the result is O = 0, LSE = -inf;
 *   otherwise LSE = M + ln sum_s exp(L_s - M),
 *             O   = sum_s exp(L_s - LSE) O_s.
 * A partial with L_s = -inf has weight zero and its O_s is never read.
 * o_part: f64 [S][B][H_q][D]; lse_part: f64 [S][B][H_q].
 */
int oracle_merge(int S, int B, int H_q, int D, const double *o_part, const double *lse_part,
                 double *out, double *lse)
{
    if (S <= 0 || B < 0 || H_q <= 0 || D <= 0) return ORC_EINVAL;
    const int64_t stride = (int64_t)B * H_q;
    for (int64_t rh = 0; rh < stride; ++rh) {
        double M = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (lse_part[s * stride + rh] > M) M = lse_part[s * stride + rh];
        double *o = &out[rh * D];
        if (M == -INFINITY) {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            lse[rh] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int s = 0; s < S; ++s) {
            double ls = lse_part[s * stride + rh];
            if (ls != -INFINITY) sum += exp(ls - M);
        }
        double L = M + log(sum);
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int s = 0; s < S; ++s) {
            double ls = lse_part[s * stride + rh];
            if (ls == -INFINITY) continue;
            double w = exp(ls - L);
            const double *os = &o_part[(s * stride + rh) * D];
            for (int d = 0; d < D; ++d) o[d] += w * os[d];
        }
        lse[rh] = L;
    }
    return ORC_OK;
}

/*
 * Packed document-causal prefill.  Documents occupy rows
 * [cu_seqlens[d], cu_seqlens[d+1]) of the packed q/k/v; row i of document d
 * attends to keys j in [cu_seqlens[d], i] with the GQA head map and scale.
 * q: bf16 [L][H_q][D]; k, v: bf16 [L][H_kv][D]; out: f64 [L][H_q][D];
 * lse: f64 [L][H_q].  Every row has at least itself as a key.
 */
int oracle_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, int n_docs, int L, int H_q, int H_kv, int D,
                   double scale, double *out, double *lse)
{
    if (n_docs < 0 || L < 0 || H_q <= 0 || H_kv <= 0 || D <= 0 || H_q % H_kv != 0)
        return ORC_EINVAL;
    if (cu_seqlens[0] != 0 || cu_seqlens[n_docs] != L) return ORC_EINVAL;
    for (int d = 0; d < n_docs; ++d)
        if (cu_seqlens[d + 1] < cu_seqlens[d]) return ORC_EINVAL;
    const int G = H_q / H_kv;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int d = 0; d < n_docs; ++d) {
        for (int g = 0; g < H_kv; ++g) {
            const int start = cu_seqlens[d];
            const int n = cu_seqlens[d + 1] - start;
            if (n == 0) continue;
            /* gather this document's keys and values of KV head g */
            double *K = (double *)malloc(sizeof(double) * (size_t)n * D);
            double *V = (double *)malloc(sizeof(double) * (size_t)n * D);
            double *x = (double *)malloc(sizeof(double) * (size_t)n);
            double *qd = (double *)malloc(sizeof(double) * (size_t)D);
            if (!K || !V || !x || !qd) {
#pragma omp atomic write
                err = 1;
            } else {
                for (int i = 0; i < n; ++i)
                    for (int dd = 0; dd < D; ++dd) {
                        K[(int64_t)i * D + dd] = bf16_to_f64(k[((int64_t)(start + i) * H_kv + g) * D + dd]);
                        V[(int64_t)i * D + dd] = bf16_to_f64(v[((int64_t)(start + i) * H_kv + g) * D + dd]);
                    }
                for (int i = 0; i < n; ++i) {
                    for (int hh = 0; hh < G; ++hh) {
                        int h = g * G + hh;
                        const uint16_t *qr = &q[((int64_t)(start + i) * H_q + h) * D];
                        for (int dd = 0; dd < D; ++dd) qd[dd] = bf16_to_f64(qr[dd]);
                        /* keys start..start+i: the first i+1 gathered rows */
                        softmax_attend(qd, K, V, i + 1, D, scale, x,
                                       &out[((int64_t)(start + i) * H_q + h) * D],
                                       &lse[(int64_t)(start + i) * H_q + h]);
                    }
                }
            }
            free(K);
            free(V);
            free(x);
            free(qd);
        }
    }
    return err ? ORC_EINVAL : ORC_OK;
}
