/*
 * Seeded, counter-based synthetic inputs for the MoE layer workloads.
 *
 * This file generates INPUTS only: activations, weights, noise draws and
 * permutations. It holds none of the layer's arithmetic (no router, no top-k,
 * no capacity, no expert FFN, no combine). Both the CPU oracle's tests and the
 * GPU path's tests and benchmark take their inputs from here, so the two sides
 * see bit-identical tensors.
 *
 * Generator definition (all of it is stated here so it can be re-implemented
 * anywhere):
 *   mix64(z)            : the SplitMix64 output function (Steele, Lea, Flood,
 *                         "Fast splittable pseudorandom number generators",
 *                         OOPSLA 2014), with the 0xBF58476D1CE4E5B9 /
 *                         0x94D049BB133111EB multipliers.
 *   key(seed, stream)   = mix64(mix64(seed + G) ^ mix64(stream * G2 + G))
 *   draw(key, i)        = mix64(key + (i + 1) * G)          (i = 0, 1, ...)
 *   uniform(r)          = ((r >> 11) + 0.5) * 2^-53          in (0, 1)
 *   normal element i    = sqrt(-2 ln u1) * cos(2 pi u2),
 *                         u1 = uniform(draw(key, 2i)), u2 = uniform(draw(key, 2i+1))
 *                         (Box and Muller, 1958; one value per pair so that
 *                          element i depends on its own counters only)
 *   G  = 0x9E3779B97F4A7C15, G2 = 0xD1B54A32D192ED03.
 * Element i of a stream never depends on how many elements are drawn, so any
 * slice of a tensor can be regenerated on its own.
 *
 * bf16 storage: a value is first rounded to fp32, then to bf16 with
 * round-to-nearest-even on the fp32 bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_G 0x9E3779B97F4A7C15ULL
#define SYN_G2 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + SYN_G) ^ mix64(stream * SYN_G2 + SYN_G));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * SYN_G); }

static inline double uniform01(uint64_t r) {
  return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = uniform01(draw(key, 2 * i));
  double u2 = uniform01(draw(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t syn_draw_u64(uint64_t seed, uint64_t stream, uint64_t i) {
  return draw(stream_key(seed, stream), i);
}

/* out[j] = fl32(sigma * normal(offset + j)), j < n */
void syn_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                    float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = (float)(sigma * normal_at(key, offset + (uint64_t)j));
}

/* out[j] = bf16_rne(fl32(sigma * normal(offset + j))) as raw bits */
void syn_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                     uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = f32_to_bf16_rne((float)(sigma * normal_at(key, offset + (uint64_t)j)));
}

/* Perturbed copy of a base tensor: out[j] = bf16_rne(fl32(base[j] + sigma * normal(offset + j))) */
void syn_perturb_bf16(const float* base, uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      double sigma, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = f32_to_bf16_rne((float)((double)base[j] + sigma * normal_at(key, offset + (uint64_t)j)));
}

/* fp32 -> bf16 bits, round to nearest even */
void syn_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}

/* bf16 bits -> fp32 (exact) */
void syn_bf16_to_f32(const uint16_t* in, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    uint32_t u = (uint32_t)in[j] << 16;
    memcpy(&out[j], &u, 4);
  }
}

/* Seeded Fisher-Yates shuffle of 0..n-1 (Durstenfeld's form); draw m picks the
 * partner of position n-1-m. */
void syn_permutation(uint64_t seed, uint64_t stream, int64_t n, int64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = i;
  for (int64_t i = n - 1, m = 0; i > 0; --i, ++m) {
    double u = uniform01(draw(key, (uint64_t)m));
    int64_t j = (int64_t)(u * (double)(i + 1));
    if (j > i) j = i;
    int64_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
