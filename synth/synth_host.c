/* Seeded synthetic inputs, host side in C (the definition is the docstring of
 * synth/__init__.py; this is a faster implementation of the same generator for
 * large host-side inputs). Holds no attention arithmetic. */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t row_key(uint64_t seed, int64_t f0, int64_t f1, int64_t f2, int64_t f3, int64_t f4,
                        int64_t f5) {
  uint64_t h = seed;
  h = mix64(h + GAMMA + (uint64_t)f0);
  h = mix64(h + GAMMA + (uint64_t)f1);
  h = mix64(h + GAMMA + (uint64_t)f2);
  h = mix64(h + GAMMA + (uint64_t)f3);
  h = mix64(h + GAMMA + (uint64_t)f4);
  h = mix64(h + GAMMA + (uint64_t)f5);
  return h;
}

static double store_round(double z, int bf16) {
  float f = (float)z;
  if (!bf16) return (double)f;
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* out[n][heads][d]: rows with identities (layer, kind, a[r], b[r], which, head). */
void synth_rows_c(uint64_t seed, int64_t layer, int64_t kind, const int64_t* a, const int64_t* b,
                  int64_t n, int64_t which, int heads, int d, int bf16, double scale,
                  double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++) {
    for (int h = 0; h < heads; h++) {
      uint64_t key = row_key(seed, layer, kind, a[r], b[r], which, h);
      double* o = out + (r * heads + h) * d;
      for (int e = 0; e < d / 2; e++) {
        uint64_t r1 = mix64(key + (2 * (uint64_t)e + 1) * GAMMA);
        uint64_t r2 = mix64(key + (2 * (uint64_t)e + 2) * GAMMA);
        double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53;
        double u2 = (double)(r2 >> 11) * 0x1.0p-53;
        double rho = sqrt(-2.0 * log(u1));
        double t = 2.0 * 3.141592653589793 * u2;
        o[2 * e] = store_round(scale * (rho * cos(t)), bf16);
        o[2 * e + 1] = store_round(scale * (rho * sin(t)), bf16);
      }
    }
  }
}
