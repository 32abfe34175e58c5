// Device helpers shared by the HIP kernels of the AbridgeKV hot path
// (element conversion, wavefront reductions, row shapes, table access, the
// bf16 dot and MFMA wrappers) and the dispatch macro of their launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace abk {

// ---- element types ------------------------------------------------------------

struct bf16_t {
  uint16_t u;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.u << 16); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t{(uint16_t)((u >> 16) | 0x40)};  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t{(uint16_t)(u >> 16)};
}

// 16 bytes of a row -> floats (8 for bf16, 4 for fp32).
__device__ __forceinline__ void unpack16(const uint4& w, float* f, bf16_t) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(x[i] << 16);
    f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& w, float* f, float) {
  f[0] = __uint_as_float(w.x);
  f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z);
  f[3] = __uint_as_float(w.w);
}

// ---- wavefront reductions -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N = 1..64, a power of two); every lane of
// a group ends with the group's sum. Within 16 lanes the DPP row operations do
// it: swap neighbours, swap pairs, mirror 8, mirror 16.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Reduce across the lane bits above log2(STRIDE) (sum or max).
template <int STRIDE>
__device__ __forceinline__ float across_sum(float x) {
#pragma unroll
  for (int o = STRIDE; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float across_max(float x) {
#pragma unroll
  for (int o = STRIDE; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane bits 3..5 (the 8 row slots of an 8-lanes-per-row
// layout) without the LDS crossbar: DPP row_ror:8 pairs lanes i and i^8 inside
// a 16-lane row, v_permlane16_swap exchanges neighbouring rows and
// v_permlane32_swap the two halves of the wavefront.
__device__ __forceinline__ float slots8_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float slots8_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Rows are read 16 bytes per lane: EPL elements per lane, LPR lanes per row,
// RPL rows per wavefront load, at most MAXCH loads per 64-row page.
template <typename T, int D>
struct RowCfg {
  static constexpr int EPL = 16 / (int)sizeof(T);
  static constexpr int LPR = D / EPL;
  static constexpr int RPL = 64 / LPR;
  static constexpr int MAXCH = (64 + RPL - 1) / RPL;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row shape");
};

__device__ __forceinline__ const int32_t* meta_of(const DevPool& P, int slot, int layer) {
  return P.meta + (slot * P.L + layer) * 4;
}
__device__ __forceinline__ int32_t* ptab_of(const DevPool& P, int slot, int layer) {
  return P.ptab + (size_t)(slot * P.L + layer) * P.tstride;
}

// XOR swizzle of a 16-byte chunk position by bits 0, 1, 3 and 4 of a K row: the
// 16 rows that one quarter of an MFMA A-operand read touches (keys 8a + 4m + b,
// a, b in 0..3, for a fixed m) land on 16 different chunk positions, so the
// 256 bytes they read hit every bank once
__device__ __forceinline__ int kswz(int row) { return (((row >> 3) & 3) << 2) | (row & 3); }

// ---- RoPE in fp64 ---------------------------------------------------------------
// The (cos, sin) table is fp64, computed on the host as cos/sin(pos *
// base^(-2i/d)). Rotations run in fp64 without contraction and are rounded once
// to the storage type, so stored keys and rotated queries are the correctly
// rounded values of the exact rotation of the stored inputs.
// rotate-half pair (a, b) = (x_i, x_{i+d/2}) -> (a cos - b sin, b cos + a sin)
__device__ __forceinline__ double rot_first(double a, double b, double2 cs) {
#pragma clang fp contract(off)
  return a * cs.x - b * cs.y;
}
__device__ __forceinline__ double rot_second(double a, double b, double2 cs) {
#pragma clang fp contract(off)
  return b * cs.x + a * cs.y;
}
// Rotate-half RoPE of element d of a row x (D elements, any layout via lambda).
template <int D, typename F>
__device__ __forceinline__ double rope_elem(F x, int d, const double2* rope_row) {
  constexpr int H = D / 2;
  if (d < H) return rot_first(x(d), x(d + H), rope_row[d]);
  return rot_second(x(d - H), x(d), rope_row[d - H]);
}

// ---- small helpers -----------------------------------------------------------------

__device__ __forceinline__ int sgpr(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Merge the split partials of one (sequence, KV head): weights
// exp2(m_s - M) / L per (split, query head) in LDS, then every output element
// is one weighted sum over the splits.
template <typename T, int D, int G>
__global__ void __launch_bounds__(1024) decode_merge_kernel(DecodeArgs a) {
  __shared__ float sm_pm[kMaxSplits * G], sm_pl[kMaxSplits * G], sm_M[G], sm_L[G];
  const int i = blockIdx.x, h = blockIdx.y;
  const int b0 = a.prefix[i], ns = a.prefix[i + 1] - b0;
  if (ns == 1) return;  // single split: the split kernel wrote out and lse
  const int Hkv = a.P.Hkv, Hq = Hkv * G;
  auto part = [&](int s, int g) { return a.part + (((size_t)(b0 + s) * Hkv + h) * G + g) * (D + 2); };
  for (int t = threadIdx.x; t < ns * G; t += blockDim.x) {
    const float* pp = part(t / G, t % G);
    sm_pm[t] = pp[D];
    sm_pl[t] = pp[D + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
    for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, sm_pm[s2 * G + g]);
    float Ls = 0.f;
    for (int s2 = 0; s2 < ns; ++s2) Ls += sm_pl[s2 * G + g] * fast_exp2(sm_pm[s2 * G + g] - M);
    sm_M[g] = M;
    sm_L[g] = Ls;
    a.lse[(size_t)i * Hq + h * G + g] = (M + __log2f(Ls)) * 0.6931471805599453f;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < ns * G; t += blockDim.x)
    sm_pm[t] = fast_exp2(sm_pm[t] - sm_M[t % G]) / sm_L[t % G];
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int g = t / D, d = t % D;
    float O = 0.f;
    for (int s2 = 0; s2 < ns; ++s2) O += part(s2, g)[d] * sm_pm[s2 * G + g];
    ((T*)a.out)[((size_t)i * Hq + h * G + g) * D + d] = from_f32<T>(O);
  }
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// bf16 bits of a float, rounded to nearest even by the hardware conversion
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // v_cvt_pk_bf16_f32: nearest even
}
// double -> float rounded to odd (the neighbour toward zero, last bit forced
// to 1, when inexact): a later nearest-even rounding to a format at least two
// bits narrower then equals a single nearest-even rounding of the double
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  float f = (float)d;
  if ((double)f != d) {
    uint32_t b = __float_as_uint(f);
    if (fabs((double)f) > fabs(d)) b -= 1;
    f = __uint_as_float(b | 1u);
  }
  return f;
}
// a double rounded once (nearest even) to the storage type T
template <typename T>
__device__ __forceinline__ T from_f64(double d);
template <>
__device__ __forceinline__ float from_f64<float>(double d) { return (float)d; }
template <>
__device__ __forceinline__ bf16_t from_f64<bf16_t>(double d) {
  return bf16_t{(uint16_t)bf16_bits(f64_to_f32_odd(d))};
}
// ... and widened back to float: the rotated query in the pool dtype
template <typename T>
__device__ __forceinline__ float round_to(double d) { return to_f32(from_f64<T>(d)); }
// two doubles -> packed bf16 pair (a in the low half), each rounded once
__device__ __forceinline__ uint32_t pack_bf16x2_f64(double a, double b) {
  return bf16_bits(f64_to_f32_odd(a)) | (bf16_bits(f64_to_f32_odd(b)) << 16);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (a in the low half), nearest even, one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ int bitrev_dev(int k, int nbits) {
  return nbits == 0 ? 0 : (int)(__brev((unsigned)k) >> (32 - nbits));
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));  // ds_read_b64_tr_b16 result

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// max / sum over the four 16-lane rows of a wavefront (lane bits 4 and 5)
__device__ __forceinline__ float rows4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- dispatch over element type and head dim ---------------------------------------

#define ABK_DISPATCH_TD(dtype, D, ...)                                  \
  do {                                                                  \
    if (dtype == 0) {                                                   \
      using T = float;                                                  \
      if (D == 16) { constexpr int DD = 16; __VA_ARGS__; }              \
      else if (D == 64) { constexpr int DD = 64; __VA_ARGS__; }         \
      else if (D == 128) { constexpr int DD = 128; __VA_ARGS__; }       \
      else return hipErrorInvalidValue;                                 \
    } else {                                                            \
      using T = bf16_t;                                                 \
      if (D == 16) { constexpr int DD = 16; __VA_ARGS__; }              \
      else if (D == 64) { constexpr int DD = 64; __VA_ARGS__; }         \
      else if (D == 128) { constexpr int DD = 128; __VA_ARGS__; }       \
      else return hipErrorInvalidValue;                                 \
    }                                                                   \
  } while (0)

static inline int threads_for(int Hkv, int D) {
  int t = Hkv * (D / 2);
  t = t < 64 ? 64 : t;
  return t > 1024 ? 1024 : t;
}

}  // namespace abk
