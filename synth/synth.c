/* Seeded synthetic input generator shared by the tests, the benchmark and the
 * CPU reference.  It holds none of the layer's arithmetic: it only turns
 * (seed, tag, a, b, element index) into pseudo-random numbers.
 *
 * Generator: a counter-based use of the SplitMix64 output function
 * (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014).  Element stream s has a 64-bit key derived from
 * (seed, tag, a, b); draw i is mix64(key + (i + 1) * GAMMA).  Because every
 * draw depends only on its index, any slab (one expert's weight, one adapter's
 * A or B) can be produced alone and in parallel, and always gives the same
 * bits.
 *
 * Normals come from the Box-Muller transform on pairs of 53-bit uniforms.
 * Normal values are rounded fp64 -> fp32 (C conversion, round-to-nearest) and
 * then fp32 -> bf16 with round-to-nearest-even on the bit pattern.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ (tag + 1) * 0xD1B54A32D192ED03ULL);
  k = mix64(k ^ (a + 1) * 0xAEF17502108EF2D9ULL);
  k = mix64(k ^ (b + 1) * 0xDB4F0B9175AE2165ULL);
  return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform in the open interval (0, 1) with 53 random bits */
static inline double u01(uint64_t r) { return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t u = v.u;
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* normal number n (n-th value of the stream): pair m = n/2 uses draws 2m, 2m+1 */
static inline void normal_pair(uint64_t key, int64_t m, double* z0, double* z1) {
  double u1 = u01(draw(key, (uint64_t)(2 * m)));
  double u2 = u01(draw(key, (uint64_t)(2 * m + 1)));
  double rad = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *z0 = rad * cos(th);
  *z1 = rad * sin(th);
}

void synth_uniform_f64(uint64_t key, int64_t n, double* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = u01(draw(key, (uint64_t)i));
}

void synth_normal_f64(uint64_t key, int64_t n, double mean, double std, double* out) {
  int64_t npair = (n + 1) / 2;
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t m = 0; m < npair; ++m) {
    double z0, z1;
    normal_pair(key, m, &z0, &z1);
    out[2 * m] = mean + std * z0;
    if (2 * m + 1 < n) out[2 * m + 1] = mean + std * z1;
  }
}

void synth_normal_bf16(uint64_t key, int64_t n, double std, uint16_t* out) {
  int64_t npair = (n + 1) / 2;
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t m = 0; m < npair; ++m) {
    double z0, z1;
    normal_pair(key, m, &z0, &z1);
    out[2 * m] = f32_to_bf16_rne((float)(std * z0));
    if (2 * m + 1 < n) out[2 * m + 1] = f32_to_bf16_rne((float)(std * z1));
  }
}

/* Round an fp32 array to bf16 (RNE) bit patterns; used to store hand-built fixtures. */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
