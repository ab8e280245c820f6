/* Host implementation of the seeded synthetic-input generator declared in gen.h.
 * Build with -ffp-contract=off so that lo + (hi-lo)*t is two separately rounded operations,
 * exactly as the GPU fill kernels evaluate it. */
#include "gen.h"

#include <math.h>
#include <string.h>

#define BQ_GOLDEN 0x9E3779B97F4A7C15ULL

uint64_t bq_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t bq_draw(uint64_t key, uint64_t i) { return bq_mix64(key + (i + 1) * BQ_GOLDEN); }

static uint64_t derive(uint64_t parent, uint64_t field) { return bq_mix64(parent ^ bq_mix64(field + BQ_GOLDEN)); }

uint64_t bq_tensor_key(uint64_t seed, int64_t family, int64_t layer, int64_t tensor, int64_t expert,
                       int64_t matrix) {
  uint64_t k = bq_mix64(seed + BQ_GOLDEN);
  k = derive(k, (uint64_t)family);
  k = derive(k, (uint64_t)layer);
  k = derive(k, (uint64_t)tensor);
  k = derive(k, (uint64_t)(expert + 1)); /* expert -1 (the shared expert) maps to 0 */
  k = derive(k, (uint64_t)matrix);
  return k;
}

/* Round a finite double to bf16, ties to even, by integer arithmetic on its bits: bf16 keeps 7
 * explicit mantissa bits, so the rounding point is double mantissa bit 45. The rounded double
 * has at most 8 significant bits, so the conversion to float is exact and the bf16 pattern is
 * the float's upper half. */
uint16_t bq_bf16_rne(double v) {
  uint64_t b;
  memcpy(&b, &v, 8);
  uint64_t lsb = (b >> 45) & 1u;
  b += ((1ULL << 44) - 1u) + lsb;
  b &= ~((1ULL << 45) - 1u);
  double r;
  memcpy(&r, &b, 8);
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

void bq_gen_codes(uint64_t key, int bits, int64_t start, int64_t n, uint8_t* out) {
  const int per = 64 / bits;
  const uint64_t mask = (1ULL << bits) - 1u;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t e = start + i;
    const uint64_t w = bq_draw(key, (uint64_t)(e / per));
    out[i] = (uint8_t)((w >> (bits * (int)(e % per))) & mask);
  }
}

void bq_gen_uniform_bf16(uint64_t key, double lo, double hi, int64_t start, int64_t n, uint16_t* out) {
  const double d = hi - lo;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double t = (double)(bq_draw(key, (uint64_t)(start + i)) >> 11) * 0x1p-53;
    const double p = d * t;
    const double v = lo + p;
    out[i] = bq_bf16_rne(v);
  }
}

void bq_gen_ints_u16(uint64_t key, int lo, int hi, int64_t start, int64_t n, uint16_t* out) {
  const uint64_t span = (uint64_t)(hi - lo) + 1u;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)(lo + (int)(bq_draw(key, (uint64_t)(start + i)) % span));
}

static double normal_at(uint64_t key, int64_t m) {
  const double u1 = (double)((bq_draw(key, (uint64_t)(2 * m)) >> 11) + 1) * 0x1p-53;
  const double u2 = (double)(bq_draw(key, (uint64_t)(2 * m + 1)) >> 11) * 0x1p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

void bq_gen_normal_bf16(uint64_t key, double sigma, int64_t start, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = bq_bf16_rne(sigma * normal_at(key, start + i));
}

void bq_gen_normal_f32(uint64_t key, double sigma, int64_t start, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, start + i));
}
