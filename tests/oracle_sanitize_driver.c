/* Drives the CPU oracle through every entry point on small caches so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer checks its
 * memory accesses and arithmetic (tests/test_sanitizers.py builds and runs
 * it).  Prints "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/kvq_oracle.h"

static uint64_t rng_state = 0x1234567ull;
static float rnd(void) { /* xorshift64*, uniform in [-2, 2) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (float)((rng_state * 0x2545F4914F6CDD1Dull) >> 40) / (float)(1u << 24) * 4.0f - 2.0f;
}

static int run(int L, int B, int Hq, int Hkv, int D, int g, const int32_t *cap,
               const int32_t *vb, const int32_t *ve, const uint8_t *kb, const uint8_t *vbits,
               int rotate) {
  orc_config c = {L, B, Hq, Hkv, D, g, cap, vb, ve, kb, vbits, rotate};
  orc_cache_info info;
  int l, s, h, X, t;
  if (orc_validate(&c) || orc_cache_bytes(&c, &info)) return 1;
  uint8_t *cache = (uint8_t *)calloc(info.total_bytes, 1);
  for (l = 0; l < L; l++)
    for (s = 0; s < B; s++)
      for (h = 0; h < Hkv; h++)
        for (X = 0; X < 2; X++) {
          float *src = (float *)malloc(sizeof(float) * (size_t)cap[s] * D);
          for (t = 0; t < cap[s] * D; t++) src[t] = rnd();
          if (orc_store_rows(&c, cache, l, s, h, X, 0, cap[s], src)) return 2;
          free(src);
        }
  double *row = (double *)malloc(sizeof(double) * D);
  for (s = 0; s < B; s++)
    for (t = 0; t < cap[s]; t++) {
      if (orc_load_row(&c, cache, L - 1, s, Hkv - 1, 1, t, row)) return 3;
      if (orc_load_row_stored(&c, cache, 0, s, 0, 0, t, row)) return 3;
    }
  int32_t *lens = (int32_t *)malloc(sizeof(int32_t) * B);
  for (s = 0; s < B; s++) lens[s] = cap[s];
  size_t nq = (size_t)L * B * Hq * D;
  uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * nq);
  double *out = (double *)malloc(sizeof(double) * nq);
  for (size_t i = 0; i < nq; i++) q[i] = orc_bf16_round_nearest_even(rnd());
  if (orc_decode_all(&c, cache, 0, L, lens, q, 0.125f, out)) return 4;
  for (size_t i = 0; i < nq; i++)
    if (!isfinite(out[i])) return 5;
  double *sc = (double *)malloc(sizeof(double) * cap[0]);
  double *sc2 = (double *)malloc(sizeof(double) * cap[0]);
  double o1[128], lse;
  if (orc_decode_one(&c, cache, 0, 0, 0, cap[0], q, 0.125f, o1, &lse, sc)) return 6;
  if (orc_decode_one(&c, cache, 0, 0, Hq - 1, cap[0], q, 0.125f, o1, &lse, sc2)) return 6;
  if (!(orc_kl_logits(sc, sc2, cap[0]) >= -1e-12)) return 7;
  free(sc); free(sc2); free(q); free(out); free(lens); free(row); free(cache);
  return 0;
}

int main(void) {
  int rc;
  {
    const int32_t cap[] = {37, 50, 9, 64}, vb[] = {5, 7, 0, 20}, ve[] = {30, 7, 9, 64};
    const uint8_t kb[] = {4, 2, 8, 16, 2, 4}, vbits[] = {2, 4, 16, 8, 4, 2};
    if ((rc = run(3, 4, 4, 2, 64, 32, cap, vb, ve, kb, vbits, 0))) return printf("fail %d\n", rc), 1;
    if ((rc = run(3, 4, 4, 2, 64, 32, cap, vb, ve, kb, vbits, 1))) return printf("fail %d\n", rc), 1;
  }
  {
    const int32_t cap[] = {300}, vb[] = {14}, ve[] = {290};
    const uint8_t kb[] = {4, 8, 2, 16}, vbits[] = {2, 4, 8, 16};
    if ((rc = run(1, 1, 28, 4, 128, 64, cap, vb, ve, kb, vbits, 1))) return printf("fail %d\n", rc), 1;
    if ((rc = run(1, 1, 28, 4, 128, 128, cap, vb, ve, kb, vbits, 0))) return printf("fail %d\n", rc), 1;
  }
  /* every width on the quantiser directly, including a constant group */
  for (int b = 2; b <= 8; b *= 2) {
    float x[64];
    uint8_t codes[64];
    uint16_t s16, m16;
    for (int i = 0; i < 64; i++) x[i] = rnd();
    orc_quantize_group(x, 64, b, codes, &s16, &m16);
    for (int i = 0; i < 64; i++) x[i] = 1.5f;
    orc_quantize_group(x, 64, b, codes, &s16, &m16);
  }
  printf("ok\n");
  return 0;
}
