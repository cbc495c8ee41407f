/*
 * synth.c -- seeded synthetic tensors for the W8A8 quantized-linear tests and bench.
 *
 * This file holds no quantization arithmetic: only a counter-based random
 * stream, normal deviates, and the rounding of the drawn values to the
 * storage type (bf16 or fp32).  Both the GPU tests and the CPU oracle take
 * their inputs from here; nothing here calls either of them.
 *
 * Random stream: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  Output number i
 * of stream `seed` is mix64(seed + (i + 1) * GOLDEN), so any element can be
 * drawn independently of the others (counter-based).
 *
 * Normals: Box-Muller (G. E. P. Box, M. E. Muller, 1958), cosine branch only,
 * from the uniforms of counters 2i and 2i+1, in fp64.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared synth.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GOLDEN); }

/* uniform in the open interval (0,1): 53 random bits, offset by half a step */
static inline double unif(uint64_t seed, uint64_t i) {
  return ((double)(draw(seed, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal(uint64_t seed, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif(seed, 2 * i), u2 = unif(seed, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite) */
static inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* raw stream: out[k] = draw(seed, first + k) */
void synth_u64(uint64_t seed, uint64_t first, int64_t n, uint64_t* out) {
  for (int64_t k = 0; k < n; ++k) out[k] = draw(seed, first + (uint64_t)k);
}

/* uniforms in (0,1): out[k] = unif(seed, first + k) */
void synth_uniform(uint64_t seed, uint64_t first, int64_t n, double* out) {
  for (int64_t k = 0; k < n; ++k) out[k] = unif(seed, first + (uint64_t)k);
}

/*
 * Fill a row-major [rows, cols] tensor.  Element (r, c), with i = r*cols + c:
 *   v = normal(seed, i) * stddev * row_scale[r] * col_mult[c] * tail(i)
 * where tail(i) = tail_mult if unif(tail_seed, i) < tail_p, else 1.
 * row_scale / col_mult may be NULL (all ones).  v is rounded once to fp32,
 * and for dtype 1 then to bf16 (RNE).  out is float* (dtype 0) or uint16_t*
 * bf16 bits (dtype 1).
 */
void synth_fill(uint64_t seed, int64_t rows, int64_t cols, double stddev, const double* row_scale,
                const double* col_mult, uint64_t tail_seed, double tail_p, double tail_mult, int dtype,
                void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double rs = row_scale ? row_scale[r] : 1.0;
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t i = (uint64_t)(r * cols + c);
      double v = normal(seed, i) * stddev * rs;
      if (col_mult) v *= col_mult[c];
      if (tail_p > 0.0 && unif(tail_seed, i) < tail_p) v *= tail_mult;
      float f = (float)v;
      if (dtype == 0)
        ((float*)out)[i] = f;
      else
        ((uint16_t*)out)[i] = f32_to_bf16(f);
    }
  }
}
