/*
 * synth_core.c -- counter-based N(0,1) samples for the synthetic inputs of
 * the windowed-GQA tests and benchmark.
 *
 * Row r of the request has the key (seed, tensor, b[r], head[r], pos[r],
 * version[r]); its elements are drawn from that key alone, so any subset of
 * rows can be regenerated independently.  SplitMix64 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) hashes the
 * key; each 64-bit output yields two 24-bit uniforms, and the Box-Muller
 * transform turns them into two normal samples (computed in double, stored
 * as float).  No attention or cache arithmetic lives here.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t row_hash(uint64_t seed, uint64_t tensor, int64_t b, int64_t head,
                         int64_t pos, int64_t version) {
  uint64_t h = mix64(seed * GAMMA + tensor + GAMMA);
  h = mix64(h + ((uint64_t)b + 1u) * GAMMA);
  h = mix64(h + ((uint64_t)head + 1u) * GAMMA);
  h = mix64(h + ((uint64_t)pos + 1u) * GAMMA);
  h = mix64(h + ((uint64_t)version + 1u) * GAMMA);
  return h;
}

/* out[r * n + d] for r < nrows, d < n. */
void synth_normal_rows(uint64_t seed, uint32_t tensor, int64_t nrows,
                       const int64_t* b, const int64_t* head, const int64_t* pos,
                       const int64_t* version, int32_t n, double stddev,
                       float* out) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    const uint64_t h = row_hash(seed, tensor, b[r], head[r], pos[r], version[r]);
    float* o = out + r * (int64_t)n;
    for (int32_t m = 0; 2 * m < n; ++m) {
      const uint64_t x = mix64(h + ((uint64_t)m + 1u) * GAMMA);
      const double u1 = ((double)(x >> 40) + 0.5) / 16777216.0;
      const double u2 = ((double)(x & 0xFFFFFFu) + 0.5) / 16777216.0;
      const double rad = sqrt(-2.0 * log(u1)) * stddev;
      o[2 * m] = (float)(rad * cos(two_pi * u2));
      if (2 * m + 1 < n) o[2 * m + 1] = (float)(rad * sin(two_pi * u2));
    }
  }
}
