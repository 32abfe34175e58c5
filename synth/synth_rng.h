/* Seeded synthetic inputs, device side.
 *
 * The same generator as synth/__init__.py (its docstring is the definition):
 * splitmix64 (Vigna) counter streams keyed by a hash chain over a row's
 * identity, Box-Muller normals in double, then round-to-nearest-even to the
 * storage type. It holds no attention arithmetic; the library uses it only to
 * bulk-fill large synthetic caches on the device.
 */
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull

__host__ __device__ inline uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Stream state of a row: fields (layer, kind, a, b, which, head). */
__host__ __device__ inline uint64_t synth_row_key(uint64_t seed, int64_t layer, int64_t kind,
                                                  int64_t a, int64_t b, int64_t which,
                                                  int64_t head) {
  uint64_t h = seed;
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)layer);
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)kind);
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)a);
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)b);
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)which);
  h = synth_mix64(h + SYNTH_GAMMA + (uint64_t)head);
  return h;
}

/* Elements 2e and 2e+1 of the row whose stream state is `key`. */
__device__ inline void synth_pair(uint64_t key, uint64_t e, double* z0, double* z1) {
  uint64_t r1 = synth_mix64(key + (2 * e + 1) * SYNTH_GAMMA);
  uint64_t r2 = synth_mix64(key + (2 * e + 2) * SYNTH_GAMMA);
  double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;
  double rho = sqrt(-2.0 * log(u1));
  double s, c;
  sincos(2.0 * 3.14159265358979323846 * u2, &s, &c);
  *z0 = rho * c;
  *z1 = rho * s;
}

/* float -> bf16 bits, round to nearest even (inputs are finite). */
__device__ inline uint16_t synth_f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
