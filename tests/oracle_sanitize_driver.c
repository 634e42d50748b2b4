/*
 * Runs every entry point of oracle/oracle.c on small seeded inputs so that
 * the CPU reference can be checked under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py builds and runs
 * it).  The inputs exercise the skip rules of the append (slot 0, unmapped
 * blocks, page 0), padding rows and empty key ranges in decode, partials with
 * LSE = -inf in the merge and empty documents in prefill.  A few exact
 * properties are checked as well; the exit status is non-zero on failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_append(uint16_t *k_pool, uint16_t *v_pool, int num_pages, int page_size, int H_kv,
                  int D, const int32_t *page_table, int num_slots, int max_blocks,
                  const int32_t *batch_idx, const int32_t *input_pos, int N,
                  const uint16_t *k_new, const uint16_t *v_new);
int oracle_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                  int num_pages, int page_size, int H_kv, int D, const int32_t *page_table,
                  int num_slots, int max_blocks, const int32_t *batch_idx,
                  const int32_t *key_lo, const int32_t *key_hi, int B, int H_q, double scale,
                  double *out, double *lse);
int oracle_merge(int S, int B, int H_q, int D, const double *o_part, const double *lse_part,
                 double *out, double *lse);
int oracle_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *cu_seqlens, int n_docs, int L, int H_q, int H_kv, int D,
                   double scale, double *out, double *lse);

static uint32_t rng_state = 2300u;
static uint32_t next_u32(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state;
}
/* a bf16 bit pattern of a value in about [-2, 2) */
static uint16_t rand_bf16(void) {
  const float f = (float)((int32_t)(next_u32() >> 8) - (1 << 23)) / (float)(1 << 22);
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16);
}
static double bf16_value(uint16_t h) {
  const uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

static int failures = 0;
static void check(int ok, const char *what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

int main(void) {
  enum { P = 12, PS = 16, HKV = 2, HQ = 4, D = 8, SLOTS = 4, MB = 3, B = 4 };
  const int64_t plane = (int64_t)P * PS;
  uint16_t *kp = malloc(sizeof(uint16_t) * HKV * plane * D);
  uint16_t *vp = malloc(sizeof(uint16_t) * HKV * plane * D);
  for (int64_t i = 0; i < HKV * plane * D; ++i) {
    kp[i] = rand_bf16();
    vp[i] = rand_bf16();
  }
  /* slot 0 reserved; slot 1 pages 3,7,1; slot 2 pages 5,0 (block 1 unmapped); slot 3 page 9 */
  const int32_t pt[SLOTS * MB] = {0, 0, 0, 3, 7, 1, 5, 0, 0, 9, 0, 0};

  /* append: a valid token, one to slot 0, one to an unmapped block, one past the table */
  {
    const int N = 4;
    const int32_t bi[4] = {1, 0, 2, 3};
    const int32_t pos[4] = {20, 3, 17, 3 * PS};
    uint16_t *kn = malloc(sizeof(uint16_t) * N * HKV * D), *vn = malloc(sizeof(uint16_t) * N * HKV * D);
    for (int i = 0; i < N * HKV * D; ++i) {
      kn[i] = rand_bf16();
      vn[i] = rand_bf16();
    }
    uint16_t *k0 = malloc(sizeof(uint16_t) * HKV * plane * D);
    memcpy(k0, kp, sizeof(uint16_t) * HKV * plane * D);
    check(oracle_append(kp, vp, P, PS, HKV, D, pt, SLOTS, MB, bi, pos, N, kn, vn) == 0, "append rc");
    /* token 0: slot 1, position 20 = block 1 (page 7), offset 4 */
    const int64_t row = 7 * PS + 4;
    check(memcmp(&kp[(1 * plane + row) * D], &kn[(0 * HKV + 1) * D], sizeof(uint16_t) * D) == 0,
          "append writes the mapped row");
    /* page 0 is never written */
    check(memcmp(k0, kp, sizeof(uint16_t) * PS * D) == 0, "append leaves page 0 alone");
    free(kn);
    free(vn);
    free(k0);
  }

  /* decode: a padding row, an empty range, a one-key row and a full row */
  {
    uint16_t q[B * HQ * D];
    for (int i = 0; i < B * HQ * D; ++i) q[i] = rand_bf16();
    const int32_t bi[B] = {0, 3, 1, 1};
    const int32_t lo[B] = {0, 0, 0, 5};
    const int32_t hi[B] = {7, 1, 40, 5}; /* row 1: one key; row 3: empty range */
    double out[B * HQ * D], lse[B * HQ];
    check(oracle_decode(q, kp, vp, P, PS, HKV, D, pt, SLOTS, MB, bi, lo, hi, B, HQ, 0.35, out, lse) == 0,
          "decode rc");
    for (int h = 0; h < HQ; ++h) {
      check(isinf(lse[0 * HQ + h]) && lse[0 * HQ + h] < 0, "padding row LSE is -inf");
      check(out[(0 * HQ + h) * D] == 0.0, "padding row output is 0");
      check(isinf(lse[3 * HQ + h]) && lse[3 * HQ + h] < 0, "empty range LSE is -inf");
      /* one key (slot 3, page 9, row 0): O = v exactly */
      const int g = h / (HQ / HKV);
      for (int d = 0; d < D; ++d)
        check(out[(1 * HQ + h) * D + d] == bf16_value(vp[(g * plane + 9 * PS) * D + d]), "one key gives v");
    }
    /* out-of-range slot is rejected, not read */
    const int32_t bad[B] = {0, 7, 1, 1};
    check(oracle_decode(q, kp, vp, P, PS, HKV, D, pt, SLOTS, MB, bad, lo, hi, B, HQ, 0.35, out, lse) != 0,
          "decode rejects a slot past the table");
  }

  /* merge: S = 3 partials, one with LSE = -inf, one row with all -inf */
  {
    enum { S = 3, BR = 2 };
    double op[S * BR * HQ * D], lp[S * BR * HQ], out[BR * HQ * D], lse[BR * HQ];
    for (int i = 0; i < S * BR * HQ * D; ++i) op[i] = bf16_value(rand_bf16());
    for (int i = 0; i < S * BR * HQ; ++i) lp[i] = bf16_value(rand_bf16());
    for (int h = 0; h < HQ; ++h) {
      lp[(1 * BR + 0) * HQ + h] = -INFINITY;
      for (int s = 0; s < S; ++s) lp[(s * BR + 1) * HQ + h] = -INFINITY;
    }
    check(oracle_merge(S, BR, HQ, D, op, lp, out, lse) == 0, "merge rc");
    for (int h = 0; h < HQ; ++h) check(isinf(lse[1 * HQ + h]) && out[(1 * HQ + h) * D] == 0.0, "all -inf row");
  }

  /* prefill: documents of 0, 1, 5, 0 and 9 rows */
  {
    enum { L = 15, ND = 5 };
    const int32_t cu[ND + 1] = {0, 0, 1, 6, 6, 15};
    uint16_t *q = malloc(sizeof(uint16_t) * L * HQ * D);
    uint16_t *k = malloc(sizeof(uint16_t) * L * HKV * D), *v = malloc(sizeof(uint16_t) * L * HKV * D);
    for (int i = 0; i < L * HQ * D; ++i) q[i] = rand_bf16();
    for (int i = 0; i < L * HKV * D; ++i) {
      k[i] = rand_bf16();
      v[i] = rand_bf16();
    }
    double *out = malloc(sizeof(double) * L * HQ * D), *lse = malloc(sizeof(double) * L * HQ);
    check(oracle_prefill(q, k, v, cu, ND, L, HQ, HKV, D, 0.35, out, lse) == 0, "prefill rc");
    /* the one-row document attends to itself only: O = v */
    for (int h = 0; h < HQ; ++h)
      for (int d = 0; d < D; ++d)
        check(out[(0 * HQ + h) * D + d] == bf16_value(v[(0 * HKV + h / (HQ / HKV)) * D + d]),
              "one-row document gives v");
    free(q);
    free(k);
    free(v);
    free(out);
    free(lse);
  }

  free(kp);
  free(vp);
  if (failures) return 1;
  printf("oracle sanitized run ok\n");
  return 0;
}
