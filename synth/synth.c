/*
 * synth.c - seeded, counter-based synthetic inputs for the tree-verify path.
 *
 * This module draws numbers and stores them; it holds none of the method's
 * arithmetic.  Both the CPU oracle and the GPU path read the exact bits it
 * writes, so a value never differs between the two sides because of how it
 * was produced.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: output c of stream `key` is the SplitMix64 finaliser applied to
 * key + (c + 1) * golden_gamma, i.e. the (c+1)-th output of a SplitMix64
 * sequence whose state starts at `key`.  Any element of any tensor can be
 * regenerated on its own.
 *
 * Normals: Box-Muller (G. Box, M. Muller, 1958) in double precision, using
 * outputs 2j and 2j+1 for the pair (2j, 2j+1): element 2j takes r*cos(t),
 * element 2j+1 takes r*sin(t).
 *
 * Value recipes (per element or per row, in double, then cast to float):
 *   SYN_NORMAL      x ~ N(0,1), times `scale`
 *   SYN_NORMAL_L2   a row of N(0,1) divided by its Euclidean norm
 *   SYN_SIGMOID     1 / (1 + exp(-x)),            x ~ N(0,1)
 *   SYN_EXP_NEG_SP  exp(-softplus(x)) = 1/(1+e^x), x ~ N(0,1)
 * Storage: float32 and/or bfloat16 bits (round to nearest even from the
 * float32 value).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_NORMAL 0
#define SYN_NORMAL_L2 1
#define SYN_SIGMOID 2
#define SYN_EXP_NEG_SP 3

static const uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

static inline uint64_t sm64_finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Output number c (0-based) of the SplitMix64 sequence whose state starts at key. */
uint64_t synth_u64(uint64_t key, uint64_t c) { return sm64_finalise(key + (c + 1) * kGamma); }

/* Uniform on the open interval (0, 1) from the top 53 bits. */
static inline double u01_open(uint64_t x) { return ((double)(x >> 11) + 0.5) * 0x1.0p-53; }

double synth_normal(uint64_t key, uint64_t i) {
  const uint64_t j = i >> 1;
  const double u1 = u01_open(synth_u64(key, 2 * j));
  const double u2 = u01_open(synth_u64(key, 2 * j + 1));
  const double r = sqrt(-2.0 * log(u1));
  const double t = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

/* Stream key for (seed, name): FNV-1a of the name, mixed with the seed. */
uint64_t synth_key(uint64_t seed, const char *name) {
  uint64_t h = 0xcbf29ce484222325ULL;
  for (const unsigned char *p = (const unsigned char *)name; *p; ++p) {
    h ^= *p;
    h *= 0x100000001b3ULL;
  }
  return sm64_finalise(seed ^ sm64_finalise(h));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/*
 * Fill rows [row0, row0 + rows) of a row-major [*, cols] tensor of stream `key`.
 * Element (r, c) is counter index r * cols + c.  out_f32 and/or out_bf16 may be
 * NULL.  Rows are independent, so the work is split over threads by row.
 */
void synth_fill(uint64_t key, int kind, int64_t row0, int64_t rows, int64_t cols, double scale,
                float *out_f32, uint16_t *out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint64_t base = (uint64_t)(row0 + r) * (uint64_t)cols;
    double norm = 1.0;
    if (kind == SYN_NORMAL_L2) {
      double ss = 0.0;
      for (int64_t c = 0; c < cols; ++c) {
        const double x = synth_normal(key, base + (uint64_t)c);
        ss += x * x;
      }
      norm = sqrt(ss);
    }
    for (int64_t c = 0; c < cols; ++c) {
      const double x = synth_normal(key, base + (uint64_t)c);
      double y;
      switch (kind) {
        case SYN_NORMAL_L2: y = x / norm; break;
        case SYN_SIGMOID: y = 1.0 / (1.0 + exp(-x)); break;
        case SYN_EXP_NEG_SP: y = 1.0 / (1.0 + exp(x)); break;
        default: y = x * scale; break;
      }
      const float f = (float)y;
      if (out_f32) out_f32[r * cols + c] = f;
      if (out_bf16) out_bf16[r * cols + c] = f32_to_bf16_rne(f);
    }
  }
}
