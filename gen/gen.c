/* Seeded synthetic inputs (host C, OpenMP). Same definition as gen/__init__.py:
 *
 *   uniform(seed, k) = top 24 bits of splitmix64(seed + (k + 1) * gamma) / 2^24
 *   (pulsatrix HIPBackend page, dropout_forward note; SplitMix64 of Steele, Lea
 *   and Flood, 2014), then Box-Muller on counter pairs (2p, 2p+1) in double,
 *   times sigma, rounded once to float32, optionally to bfloat16 (nearest, ties
 *   to even).
 *
 * This file holds no attention arithmetic. Build:
 *   gcc -O2 -fopenmp -fPIC -shared gen/gen.c -o gen/libgen.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ULL;

static inline uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline double uniform24(uint64_t seed, uint64_t k) {
  uint64_t z = splitmix64_mix(seed + (k + 1) * GAMMA);
  return (double)(z >> 40) * (1.0 / 16777216.0);
}

/* n normals N(0, sigma^2) as float32, element e from the pair p = e / 2 at
 * counters first_counter + 2p and first_counter + 2p + 1. */
void gen_normal_f32(uint64_t seed, uint64_t first_counter, int64_t n, double sigma, float* out) {
  const double two_pi = 6.283185307179586476925286766559;
  int64_t npairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npairs; ++p) {
    uint64_t base = first_counter + 2 * (uint64_t)p;
    double u1 = uniform24(seed, base);
    double u2 = uniform24(seed, base + 1);
    double r = sqrt(-2.0 * log1p(-u1));
    double th = two_pi * u2;
    int64_t e = 2 * p;
    out[e] = (float)(r * cos(th) * sigma);
    if (e + 1 < n) out[e + 1] = (float)(r * sin(th) * sigma);
  }
}

/* float32 -> bfloat16 bits, nearest with ties to even; NaN -> 0x7FC0. */
void gen_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &in[i], 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) {
      out[i] = 0x7FC0;
    } else {
      uint32_t lsb = (b >> 16) & 1u;
      out[i] = (uint16_t)((b + 0x7FFFu + lsb) >> 16);
    }
  }
}

void gen_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b = (uint32_t)in[i] << 16;
    memcpy(&out[i], &b, 4);
  }
}
