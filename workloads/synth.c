/*
 * synth.c -- seeded synthetic inputs for the spectral-mix workloads.
 *
 * This module only draws numbers; it contains none of the spectral mix's
 * arithmetic.  It is the one piece that both the GPU library's callers and
 * the CPU oracle's callers share: both sides receive the exact same arrays.
 *
 * Generator (counter-based, so the result does not depend on thread count):
 *   element i of stream `seed` takes the SplitMix64 output (Steele, Lea and
 *   Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
 *   constants as in Vigna's public reference code) of the state
 *   seed XOR (i * 0x9E3779B97F4A7C15);
 *   a standard normal uses the Box-Muller transform (Box and Muller, 1958)
 *   on the two 32-bit halves of that output, each mapped to (0, 1];
 *   a uniform on [0, 1) uses the top 53 bits.
 * Values are produced in double and rounded to binary32 (round to nearest).
 * bfloat16 values are binary32 values rounded to nearest-even on bit 16.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t state) {
  uint64_t z = state + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, int64_t i) {
  return splitmix64(seed ^ ((uint64_t)i * 0x9E3779B97F4A7C15ull));
}

static inline double normal_at(uint64_t seed, int64_t i) {
  uint64_t z = draw(seed, i);
  double u1 = ((double)(z >> 32) + 1.0) * (1.0 / 4294967296.0);        /* (0, 1] */
  double u2 = ((double)(z & 0xffffffffull) + 1.0) * (1.0 / 4294967296.0); /* (0, 1] */
  const double two_pi = 6.283185307179586476925286766559;
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline double uniform_at(uint64_t seed, int64_t i) {
  return (double)(draw(seed, i) >> 11) * (1.0 / 9007199254740992.0); /* [0, 1) */
}

void synth_normal_f32(uint64_t seed, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)normal_at(seed, i);
}

void synth_uniform_f32(uint64_t seed, int64_t n, double lo, double hi, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * uniform_at(seed, i));
}

/* out[i] = a * normal(seed_a, i) + b * normal(seed_b, i) summed in double. */
void synth_normal_mix_f32(uint64_t seed_a, double a, uint64_t seed_b, double b, int64_t n,
                          float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(a * normal_at(seed_a, i) + b * normal_at(seed_b, i));
}

/*
 * Smooth ("random walk") component for a [B, L, C] tensor: per column (b, c)
 * the running sum along L of N(0,1) draws (stream `seed`, flat index of the
 * element), then centred and scaled to unit population variance per column.
 * Result: out = a * white + b * walk, with white from stream seed_white.
 */
void synth_walk_mix_f32(uint64_t seed_white, double a, uint64_t seed_walk, double b,
                        int64_t B, int64_t L, int64_t C, float *out) {
  const int64_t ncol = B * C;
#pragma omp parallel
  {
    double *col = (double *)malloc(sizeof(double) * (size_t)L);
#pragma omp for schedule(dynamic, 4)
    for (int64_t j = 0; j < ncol; ++j) {
      if (!col) continue;
      int64_t bb = j / C, c = j % C;
      int64_t base = bb * L * C + c;
      double acc = 0.0, sum = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        acc += normal_at(seed_walk, base + t * C);
        col[t] = acc;
        sum += acc;
      }
      double mean = sum / (double)L, var = 0.0;
      for (int64_t t = 0; t < L; ++t) var += (col[t] - mean) * (col[t] - mean);
      var /= (double)L;
      double inv = var > 0.0 ? 1.0 / sqrt(var) : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t i = base + t * C;
        out[i] = (float)(a * normal_at(seed_white, i) + b * (col[t] - mean) * inv);
      }
    }
    free(col);
  }
}

/* binary32 -> bfloat16 bits, round to nearest even (inputs here are finite). */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
  }
}

void synth_bf16_to_f32(const uint16_t *in, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    memcpy(&out[i], &u, sizeof u);
  }
}
