/* The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a small decoder built from the
 * seeded generator, decoded through its cache and recomputed without one, the cache accessors, and
 * the argument checks. Any memory error or undefined behaviour aborts with the sanitizer's report; a
 * wrong result exits 1. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/oracle.h"

void si_normal_bf16(uint64_t seed, uint64_t offset, int64_t n, double mean, double std, uint16_t* out);

static int failures = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint16_t* tensor(uint64_t seed, int64_t n, double mean, double std) {
  uint16_t* t = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
  si_normal_bf16(seed, 0, n, mean, std, t);
  return t;
}

int main(void) {
  const orc_config c = {2, 64, 4, 2, 16, 96, 300, 1e-5, 10000.0, 0, 1};
  const int d = c.d, q = c.hq * c.dh, kvd = c.hk * c.dh;
  const uint16_t* t[3 + 12 * 2];
  uint16_t* own[3 + 12 * 2] = {0};
  int n = 0;
  own[n] = tensor(1, (int64_t)c.v * d, 0, 0.08); t[n] = own[n]; ++n;           /* embed */
  own[n] = tensor(2, d, 1, 0.1); t[n] = own[n]; ++n;                          /* final norm */
  own[n] = tensor(3, (int64_t)c.v * d, 0, 0.08); t[n] = own[n]; ++n;          /* lm head */
  for (int l = 0; l < c.n_layers; ++l) {
    const int64_t sizes[12] = {d, (int64_t)q * d, (int64_t)kvd * d, (int64_t)kvd * d, q, kvd, kvd,
                               (int64_t)d * q, d, (int64_t)c.f * d, (int64_t)c.f * d, (int64_t)d * c.f};
    for (int i = 0; i < 12; ++i) {
      const int gain = i == 0 || i == 8;
      own[n] = tensor(100 + 16 * l + i, sizes[i], gain ? 1 : 0, gain ? 0.1 : 0.08);
      t[n] = own[n];
      ++n;
    }
  }
  orc_model* m = orc_create(&c, t, 2, 24);
  EXPECT(m != NULL);
  double* logits = (double*)malloc(sizeof(double) * c.v);
  double* ref = (double*)malloc(sizeof(double) * c.v);
  int toks[12];
  for (int p = 0; p < 12; ++p) {
    toks[p] = (7 + 31 * p) % c.v;
    const int a = orc_step(m, 0, toks[p], p, (double)p, logits);
    const int b = orc_forward_nocache(m, toks, p + 1, 0.0, ref);
    EXPECT(a == b && a >= 0 && a < c.v);
    double num = 0, den = 0;
    for (int i = 0; i < c.v; ++i) {
      num += (logits[i] - ref[i]) * (logits[i] - ref[i]);
      den += ref[i] * ref[i];
    }
    EXPECT(sqrt(num / den) < 1e-12);
  }
  /* the second sequence's cache: write rows, read them back */
  uint16_t* kv = tensor(9, 3 * kvd, 0, 1);
  uint16_t* back = (uint16_t*)malloc(sizeof(uint16_t) * 3 * kvd);
  EXPECT(orc_set_kv(m, 1, 1, 5, 3, kv, kv) == 0);
  EXPECT(orc_get_kv(m, 1, 1, 5, 3, back, back) == 0);
  for (int i = 0; i < 3 * kvd; ++i) EXPECT(back[i] == kv[i]);
  /* arguments out of range are refused */
  EXPECT(orc_step(m, 2, 0, 0, 0.0, logits) < 0);
  EXPECT(orc_step(m, 0, c.v, 0, 0.0, logits) < 0);
  EXPECT(orc_step(m, 0, 0, 24, 24.0, logits) < 0);
  EXPECT(orc_set_kv(m, 0, 0, 22, 3, kv, kv) != 0);
  EXPECT(orc_get_kv(m, 2, 0, 0, 1, back, back) != 0);
  const orc_config bad = {2, 64, 3, 2, 16, 96, 300, 1e-5, 10000.0, 0, 1};
  EXPECT(orc_create(&bad, t, 1, 8) == NULL);
  orc_destroy(m);
  free(logits); free(ref); free(kv); free(back);
  for (int i = 0; i < n; ++i) free(own[i]);
  printf("oracle checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
