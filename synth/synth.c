/*
 * Seeded synthetic inputs: a stateless counter-based generator.
 *
 * Element i of a stream (seed, tag) is a pure function of (seed, tag, i), so any
 * slice of any tensor can be regenerated without generating what precedes it.
 *
 *   key     = mix64(seed ^ mix64(tag))
 *   bits(i) = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)      (splitmix64 output i)
 *   u1, u2  = ((bits >> 32) + 0.5) / 2^32, ((bits & 0xffffffff) + 0.5) / 2^32
 *   normal  = sqrt(-2 ln u1) * cos(2 pi u2)                    (Box-Muller, cos branch)
 *   value   = f32(sigma * normal), then bf16 round-to-nearest-even for bf16 tensors
 *   id(i)   = ((bits(i) >> 32) * V) >> 32                      (multiply-shift into [0, V))
 *
 * mix64 is the splitmix64 finaliser (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). This file holds no arithmetic of
 * the transformer: it only draws numbers.
 */
#include <math.h>
#include <stdint.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_bits(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double stream_normal(uint64_t key, uint64_t i) {
  const uint64_t b = stream_bits(key, i);
  const double u1 = ((double)(b >> 32) + 0.5) * 0x1p-32;
  const double u2 = ((double)(b & 0xffffffffULL) + 0.5) * 0x1p-32;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  const uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t tag) { return mix64(seed ^ mix64(tag)); }

void synth_bits(uint64_t key, uint64_t offset, int64_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = stream_bits(key, offset + (uint64_t)i);
}

void synth_normal_f32(uint64_t key, uint64_t offset, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * stream_normal(key, offset + (uint64_t)i));
}

void synth_normal_bf16(uint64_t key, uint64_t offset, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)(sigma * stream_normal(key, offset + (uint64_t)i)));
}

void synth_ids(uint64_t key, uint64_t offset, int64_t n, int32_t vocab, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (int32_t)(((stream_bits(key, offset + (uint64_t)i) >> 32) * (uint64_t)vocab) >> 32);
}
