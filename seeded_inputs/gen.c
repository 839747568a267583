/*
 * Seeded synthetic inputs shared by the oracle and the HIP path.
 *
 * This file holds no arithmetic of the decode step. It only draws numbers:
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014; constants as published by Vigna), used as a
 *     counter-based generator: output k of stream `seed` is mix(seed + (k+1)*gamma).
 *   - Box-Muller (1958) normals in double: element i of a stream takes the pair
 *     j = i/2, u1 = ((out(2j) >> 11) + 1) * 2^-53 in (0,1], u2 = (out(2j+1) >> 11) * 2^-53,
 *     r = sqrt(-2 ln u1), even i -> r cos(2 pi u2), odd i -> r sin(2 pi u2).
 *   - bf16 values are mean + std*z rounded to float (round to nearest even) and then
 *     to bf16 (round to nearest even on the float bit pattern).
 * Every element depends only on (seed, index), so any slice can be drawn alone and
 * the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
static inline uint64_t sm_out(uint64_t seed, uint64_t k) { return sm_mix(seed + (k + 1) * GAMMA); }

static inline double normal_at(uint64_t seed, uint64_t i) {
  const uint64_t j = i >> 1;
  const uint64_t a = sm_out(seed, 2 * j), b = sm_out(seed, 2 * j + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53;
  const double u2 = (double)(b >> 11) * 0x1.0p-53;
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t si_splitmix_out(uint64_t seed, uint64_t k) { return sm_out(seed, k); }
double si_normal_at(uint64_t seed, uint64_t i) { return normal_at(seed, i); }

/* out[t] = bf16(float(mean + std * normal(seed, offset + t))), t in [0, n) */
void si_normal_bf16(uint64_t seed, uint64_t offset, int64_t n, double mean, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    const double v = mean + std * normal_at(seed, offset + (uint64_t)t);
    out[t] = f32_to_bf16_rne((float)v);
  }
}

/* out[t] = lo + out(seed, t) mod (hi - lo + 1), inclusive range */
void si_uniform_int(uint64_t seed, int64_t n, int64_t lo, int64_t hi, int32_t* out) {
  const uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t t = 0; t < n; ++t) out[t] = (int32_t)(lo + (int64_t)(sm_out(seed, (uint64_t)t) % span));
}

/* Fisher-Yates shuffle of 0..n-1: for i = n-1 .. 1, swap a[i] with a[out(n-1-i) mod (i+1)] */
void si_permutation(uint64_t seed, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i >= 1; --i) {
    const int64_t j = (int64_t)(sm_out(seed, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1));
    const int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
