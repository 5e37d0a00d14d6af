/*
 * Seeded synthetic inputs for the selective scan: a counter-based generator.
 *
 * This module produces input tensors only. It holds none of the scan's
 * arithmetic; both the HIP path's tests and the fp64 oracle read the buffers
 * it writes, so parity never depends on the generator's exact values.
 *
 * Generator (stated here so that anyone can re-implement it):
 *   - SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 *     pseudorandom number generators", OOPSLA 2014) applied to a counter:
 *       key      = mix64(seed * 0x9E3779B97F4A7C15 + stream)
 *       word(i)  = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *     where mix64(z): z ^= z>>30; z *= 0xBF58476D1CE4E5B9;
 *                     z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
 *   - uniform(i) = (word(i) >> 11) * 2^-53, in [0, 1).
 *   - normal(i): Box-Muller on the pair j = i/2 with u1 = uniform(2j),
 *     u2 = uniform(2j+1): r = sqrt(-2 ln(1 - u1)); even i -> r cos(2 pi u2),
 *     odd i -> r sin(2 pi u2). Computed in double, rounded to float.
 *   - log-uniform(i) on [lo, hi]: exp(ln lo + uniform(i) (ln hi - ln lo)),
 *     in double, rounded to float.
 *   - float -> bfloat16 by round-to-nearest-even on the bit pattern.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static const uint64_t GOLDEN = 0x9E3779B97F4A7C15ULL;

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

static inline uint64_t word_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline double uniform_at(uint64_t key, uint64_t i) {
  return (double)(word_at(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

static uint64_t make_key(uint64_t seed, uint64_t stream) { return mix64(seed * GOLDEN + stream); }

enum { K_NORMAL = 0, K_LOGUNIFORM = 1, K_UNIFORM = 2 };

typedef struct {
  int kind;
  uint64_t key;
  float* out;
  size_t begin, end;
  double lo, hi;
} job_t;

static void* run_job(void* p) {
  job_t* j = (job_t*)p;
  const double two_pi = 6.283185307179586476925286766559;
  for (size_t i = j->begin; i < j->end; ++i) {
    double v;
    if (j->kind == K_NORMAL) {
      uint64_t pair = i >> 1;
      double u1 = uniform_at(j->key, 2 * pair);
      double u2 = uniform_at(j->key, 2 * pair + 1);
      double r = sqrt(-2.0 * log(1.0 - u1));
      v = (i & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
    } else if (j->kind == K_LOGUNIFORM) {
      double u = uniform_at(j->key, i);
      v = exp(log(j->lo) + u * (log(j->hi) - log(j->lo)));
    } else {
      double u = uniform_at(j->key, i);
      v = j->lo + u * (j->hi - j->lo);
    }
    j->out[i] = (float)v;
  }
  return NULL;
}

static void fill(int kind, uint64_t seed, uint64_t stream, float* out, size_t n, double lo, double hi,
                 int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < (size_t)1 << 16) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  uint64_t key = make_key(seed, stream);
  size_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    size_t b = per * t, e = b + per;
    if (b > n) b = n;
    if (e > n) e = n;
    jobs[t] = (job_t){kind, key, out, b, e, lo, hi};
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
  run_job(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, float* out, size_t n, int nthreads) {
  fill(K_NORMAL, seed, stream, out, n, 0.0, 0.0, nthreads);
}

void synth_loguniform_f32(uint64_t seed, uint64_t stream, double lo, double hi, float* out, size_t n,
                          int nthreads) {
  fill(K_LOGUNIFORM, seed, stream, out, n, lo, hi, nthreads);
}

void synth_uniform_f32(uint64_t seed, uint64_t stream, double lo, double hi, float* out, size_t n,
                       int nthreads) {
  fill(K_UNIFORM, seed, stream, out, n, lo, hi, nthreads);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t i) { return word_at(make_key(seed, stream), i); }

/* float -> bfloat16, round to nearest even (inputs here are finite). */
void synth_f32_to_bf16(const float* in, uint16_t* out, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

void synth_bf16_to_f32(const uint16_t* in, float* out, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)in[i] << 16;
    memcpy(&out[i], &u, 4);
  }
}
