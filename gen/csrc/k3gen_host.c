/* Host side of the seeded input generator; the rules are stated in k3gen.h. */
#include "k3gen.h"

#include <math.h>
#include <string.h>

#define K3GEN_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t k3gen_draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * K3GEN_GAMMA); }

uint64_t k3gen_key(uint64_t seed, uint64_t tensor_id) {
  return mix64(mix64(seed + K3GEN_GAMMA) ^ (tensor_id * 0xD1B54A32D192ED03ULL));
}

void k3gen_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    uint64_t g = start + (uint64_t)j;
    out[j] = (uint8_t)(k3gen_draw(key, g >> 3) >> (8 * (g & 7)));
  }
}

void k3gen_scales(uint64_t key, uint64_t start, uint64_t n, int lo, int hi, uint8_t* out) {
  const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    uint64_t d = k3gen_draw(key, start + (uint64_t)j);
    out[j] = (uint8_t)(127 + lo + (int)(((d >> 32) * span) >> 32));
  }
}

static double box_muller(uint64_t key, uint64_t j) {
  const double two_m53 = 1.0 / 9007199254740992.0;
  uint64_t d1 = k3gen_draw(key, 2 * j), d2 = k3gen_draw(key, 2 * j + 1);
  double u1 = (double)((d1 >> 11) + 1) * two_m53; /* (0, 1] */
  double u2 = (double)(d2 >> 11) * two_m53;       /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

/* fp64 -> bf16 bits, round-to-nearest-even in a single rounding step
 * (normal range only, which is all a scaled standard normal reaches). */
static uint16_t f64_to_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  double m = frexp(v, &e);                 /* v = m 2^e, 0.5 <= |m| < 1 */
  double q = ldexp(nearbyint(ldexp(m, 8)), e - 8); /* 8 significant bits */
  float qf = (float)q;                     /* exact */
  uint32_t b;
  memcpy(&b, &qf, 4);
  return (uint16_t)(b >> 16);
}

void k3gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = f64_to_bf16(sigma * box_muller(key, start + (uint64_t)j));
}

void k3gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = (float)(sigma * box_muller(key, start + (uint64_t)j));
}
