/*
 * synth.c - seeded synthetic inputs for the matmul sum-check prover.
 *
 * This module draws random numbers and nothing else: it holds none of the
 * prover's arithmetic (no field multiply, no witness, no fold). Both the CPU
 * oracle and the GPU path read the bytes it writes.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). Output i (0-based) of the
 * stream with seed S is mix(S + (i+1)*GAMMA), so any index can be generated
 * independently and the fills below are parallel and deterministic.
 *
 * Distributions (plain readings of the workload descriptions; libm is used
 * for log/cos/sqrt, host only):
 *   uniform127 : (x mod 255) - 127                     -> [-127, 127]
 *   int4       : (x mod 15) - 7                        -> [-7, 7]
 *   gauss32    : Box-Muller, cos branch, element i takes outputs 2i, 2i+1:
 *                u1 = ((x1>>11)+1)*2^-53, u2 = (x2>>11)*2^-53,
 *                g = sqrt(-2 ln u1) cos(2 pi u2); v = round_half_away(32 g),
 *                clamped to [-127, 127]
 *   laplace16  : u = ((x>>11)+0.5)*2^-53; L = 16 ln(2u) for u < 1/2, else
 *                -16 ln(2 - 2u); v = round_half_away(L) clamped to [-127,127]
 *   zipf       : P(e) proportional to (e+1)^-a over e in [0, n); inverse CDF
 *                in double with u = (x>>11)*2^-53
 *   challenge  : x mod p, p = 2^64 - 2^32 + 1 (a uniformly drawn field value)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Output number idx (0-based) of the stream seeded with seed. */
static inline uint64_t sm_at(uint64_t seed, uint64_t idx) {
  return sm_mix(seed + (idx + 1) * SM_GAMMA);
}

void synth_raw(uint64_t seed, uint64_t start, int64_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sm_at(seed, start + (uint64_t)i);
}

void synth_challenges(uint64_t seed, uint64_t start, int64_t n, uint64_t* out) {
  const uint64_t p = 0xFFFFFFFF00000001ULL;
  for (int64_t i = 0; i < n; ++i) out[i] = sm_at(seed, start + (uint64_t)i) % p;
}

void synth_uniform127(uint64_t seed, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)((int)(sm_at(seed, (uint64_t)i) % 255u) - 127);
}

void synth_int4(uint64_t seed, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)((int)(sm_at(seed, (uint64_t)i) % 15u) - 7);
}

static inline int8_t round_clamp127(double v) {
  double a = floor(fabs(v) + 0.5);
  if (a > 127.0) a = 127.0;
  return (int8_t)(v < 0 ? -(int)a : (int)a);
}

void synth_gauss32(uint64_t seed, int64_t n, int8_t* out) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t x1 = sm_at(seed, 2 * (uint64_t)i), x2 = sm_at(seed, 2 * (uint64_t)i + 1);
    double u1 = (double)((x1 >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(x2 >> 11) * 0x1.0p-53;
    double g = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
    out[i] = round_clamp127(32.0 * g);
  }
}

void synth_laplace16(uint64_t seed, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t x = sm_at(seed, (uint64_t)i);
    double u = ((double)(x >> 11) + 0.5) * 0x1.0p-53;
    double l = (u < 0.5) ? 16.0 * log(2.0 * u) : -16.0 * log(2.0 - 2.0 * u);
    out[i] = round_clamp127(l);
  }
}

void synth_zipf(uint64_t seed, int64_t n, int32_t n_items, double a, int32_t* out) {
  double* cdf = (double*)malloc(sizeof(double) * (size_t)n_items);
  double tot = 0.0;
  for (int32_t e = 0; e < n_items; ++e) tot += pow((double)(e + 1), -a);
  double acc = 0.0;
  for (int32_t e = 0; e < n_items; ++e) {
    acc += pow((double)(e + 1), -a) / tot;
    cdf[e] = acc;
  }
  cdf[n_items - 1] = 1.0;
  for (int64_t i = 0; i < n; ++i) {
    double u = (double)(sm_at(seed, (uint64_t)i) >> 11) * 0x1.0p-53;
    int32_t e = 0;
    while (e < n_items - 1 && cdf[e] <= u) ++e;
    out[i] = e;
  }
  free(cdf);
}
