// HIP kernels of the AbridgeKV attention hot path, written for CDNA4 (gfx950):
// 64-lane wavefronts, DPP row reductions, 16-byte coalesced page loads.
//
// What is computed follows the pages on AbridgeKV (arXiv 2610.20641): the
// abstract and Fig. 1(a) (code rows written by pause tokens, raw block rows
// freed), Fig. 2(a) (the block mask) and Fig. 2(b) (pause token k of block b
// at position P + b*C + bitrev(k)*C/K). RoPE is rotate-half; stored keys are
// rotated once, in fp32, and rounded to the pool dtype.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../synth/synth_rng.h"
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

// Rotate-half RoPE of element d of a row x (D elements, any layout via lambda).
template <int D, typename F>
__device__ __forceinline__ float rope_elem(F x, int d, const float2* rope_row) {
  constexpr int H = D / 2;
  if (d < H) {
    float2 cs = rope_row[d];
    return x(d) * cs.x - x(d + H) * cs.y;
  }
  float2 cs = rope_row[d - H];
  return x(d) * cs.x + x(d - H) * cs.y;
}

// ---- a1: append the current token (RoPE k at its position, write k and v) ----

template <typename T, int D>
__global__ void __launch_bounds__(1024) append_kernel(AppendArgs a) {
  const DevPool P = a.P;
  const int i = blockIdx.x;
  const int slot = a.slot[i];
  const int fresh_page = a.new_page[i];
  int32_t* meta = P.meta + (slot * P.L + a.layer) * 4;
  const int n_pers = meta[0], n_open = meta[1], qpos = meta[2];
  const int r = a.compress ? n_open : n_pers;
  int32_t* tab = ptab_of(P, slot, a.layer) + (a.compress ? P.max_pers : 0);
  const int pidx = r / P.pr, srow = r % P.pr;
  const int page = srow == 0 ? fresh_page : tab[pidx];
  const int pos = qpos + 1;
  const T* k = (const T*)a.k + (size_t)i * P.Hkv * D;
  const T* v = (const T*)a.v + (size_t)i * P.Hkv * D;
  T* kd = (T*)P.kpool + ((size_t)page * P.Hkv * P.pr + srow) * D;
  T* vd = (T*)P.vpool + ((size_t)page * P.Hkv * P.pr + srow) * D;
  const float2* rope = P.rope + (size_t)pos * (D / 2);
  for (int t = threadIdx.x; t < P.Hkv * (D / 2); t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const T* kr = k + hh * D;
    const float x1 = to_f32(kr[j]), x2 = to_f32(kr[j + D / 2]);
    const float2 cs = rope[j];
    T* kdst = kd + (size_t)hh * P.pr * D;
    kdst[j] = from_f32<T>(x1 * cs.x - x2 * cs.y);
    kdst[j + D / 2] = from_f32<T>(x2 * cs.x + x1 * cs.y);
    T* vdst = vd + (size_t)hh * P.pr * D;
    vdst[j] = v[hh * D + j];
    vdst[j + D / 2] = v[hh * D + j + D / 2];
  }
  __syncthreads();  // every thread has read meta and the table
  if (threadIdx.x == 0) {
    P.pos[(size_t)page * P.pr + srow] = pos;
    if (srow == 0) tab[pidx] = page;
    meta[a.compress ? 1 : 0] += 1;
    meta[2] = pos;
  }
}

// ---- a2 + a3: split-KV decode ----------------------------------------------------
//
// Work item (sequence i, split s) x KV head h. A split is a run of pages; a page
// is cut into units of RW rows and wavefront w takes units w, w+4, ... so all
// four wavefronts stream the same pages. A unit is read 16 bytes per lane (LPR
// lanes per row, RPL rows per load): each lane holds its slice of the G
// rotated queries, so one K load feeds G dot products finished by a DPP group
// sum. The next unit's K and V are loaded into registers before the current
// unit is computed. Softmax is online per unit with a wavefront-uniform running
// max (log2 domain); V is accumulated per lane and reduced across row groups
// and wavefronts at the end; a sequence with several splits leaves partials
// (o, m, l) for the merge kernel.

#ifndef ABK_UNIT_ROWS
#define ABK_UNIT_ROWS 16  // rows of a page a wavefront reads per step
#endif
#ifndef ABK_PREFETCH_UNITS
#define ABK_PREFETCH_UNITS 1  // units a wavefront keeps in flight while computing one
#endif
template <typename T, int D>
struct UnitCfg {
  using R = RowCfg<T, D>;
  static constexpr int CW = R::RPL >= ABK_UNIT_ROWS ? 1 : ABK_UNIT_ROWS / R::RPL;  // loads/lane
  static constexpr int RW = CW * R::RPL;                                            // rows/unit
};

__device__ __forceinline__ int sgpr(int x) { return __builtin_amdgcn_readfirstlane(x); }

// a3: merge the split partials of one (sequence, KV head): weights
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

template <typename T, int D, int G>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  using Cfg = RowCfg<T, D>;
  constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPL = Cfg::RPL;
  constexpr int CW = UnitCfg<T, D>::CW, RW = UnitCfg<T, D>::RW;
  const DevPool& P = a.P;
  const int w = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int c = lane % LPR, grp = lane / LPR;

  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.prefix[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo, s = w - a.prefix[i], b0 = a.prefix[i], nsplit = a.prefix[i + 1] - b0;
  const int slot = a.slot[i];
  const int32_t* meta = meta_of(P, slot, a.layer);
  const int n_pers = sgpr(meta[0]), n_open = sgpr(meta[1]), qpos = sgpr(meta[2]);
  const int pr = P.pr;
  const int npp = (n_pers + pr - 1) / pr, nop = (n_open + pr - 1) / pr;
  const int vp0 = s * a.split_pages, vp1 = min(npp + nop, vp0 + a.split_pages);
  const int NQ = (pr + RW - 1) / RW;
  const int nunits = (vp1 - vp0) * NQ;
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int Hq = P.Hkv * G;

  // rotated, pre-scaled query slice: dims c*EPL .. c*EPL+EPL-1 of heads h*G+g.
  // Rotate-half pairs dim d with d +- D/2: the lane loads its own 16 bytes and
  // its partner's, and the (cos, sin) of its dims, all unconditionally.
  float qv[G][EPL];
  {
    constexpr int H = D / 2;
    const int d0 = c * EPL;                 // first dim of this lane
    const int dp = (d0 + H) % D;            // partner dims
    const float sgn = d0 < H ? -1.f : 1.f;  // y = x cos + sgn * x_partner sin
    const float2* rope = P.rope + (size_t)qpos * H + (d0 % H);
    float2 cs[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) cs[e] = rope[e];
    const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const T* qh = (const T*)a.q + ((size_t)i * Hq + h * G + g) * D;
      float x[EPL], xp[EPL];
      unpack16(*(const uint4*)(qh + d0), x, T());
      unpack16(*(const uint4*)(qh + dp), xp, T());
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[g][e] = qs * (x[e] * cs[e].x + sgn * xp[e] * cs[e].y);
    }
  }

  float m_run[G], l_run[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }

  const T* kpool = (const T*)P.kpool;
  const T* vpool = (const T*)P.vpool;
  // unit u -> (element offset of its first row for this lane, valid rows in it)
  auto locate = [&](int u, size_t* off, int* nval) {
    const int vp = vp0 + u / NQ, qq = u % NQ;
    int page, rows;
    if (vp < npp) {
      page = sgpr(tab[vp]);
      rows = (vp == npp - 1) ? n_pers - vp * pr : pr;
    } else {
      const int j = vp - npp;
      page = sgpr(tab[P.max_pers + j]);
      rows = (j == nop - 1) ? n_open - j * pr : pr;
    }
    *off = (((size_t)page * P.Hkv + h) * pr + (size_t)qq * RW) * D + c * EPL;
    *nval = rows - qq * RW;  // rows of this unit that exist (may be <= 0)
  };
  auto load = [&](size_t off, int nval, uint4* kr, uint4* vr) {
#pragma unroll
    for (int ch = 0; ch < CW; ++ch) {
      int r = ch * RPL + grp;
      r = r < nval ? r : (nval > 0 ? nval - 1 : 0);
      kr[ch] = *(const uint4*)(kpool + off + (size_t)r * D);
      vr[ch] = *(const uint4*)(vpool + off + (size_t)r * D);
    }
  };
  auto compute = [&](int nval, const uint4* kr, const uint4* vr) {
    float sc[CW][G];
#pragma unroll
    for (int ch = 0; ch < CW; ++ch) {
      float kf[EPL];
      unpack16(kr[ch], kf, T());
      const bool valid = ch * RPL + grp < nval;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc += qv[g][e] * kf[e];
        acc = group_sum<LPR>(acc);
        sc[ch][g] = valid ? acc : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc[0][g];
#pragma unroll
      for (int ch = 1; ch < CW; ++ch) mx = fmaxf(mx, sc[ch][g]);
      mx = across_max<LPR>(mx);  // finite: the unit has a valid row
      // rescale only when the running max grows (wavefront-uniform branch)
      if (mx > m_run[g]) {
        const float alpha = fast_exp2(m_run[g] - mx);
        m_run[g] = mx;
        l_run[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
      }
    }
#pragma unroll
    for (int ch = 0; ch < CW; ++ch) {
      float vf[EPL];
      unpack16(vr[ch], vf, T());
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(sc[ch][g] - m_run[g]);
        l_run[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] += p * vf[e];
      }
    }
  };

  // ring of NB unit buffers: NB-1 units are in flight while one is computed
  constexpr int NB = ABK_PREFETCH_UNITS + 1;
  uint4 kb[NB][CW], vb[NB][CW];
  size_t offb[NB];
  int nvb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    offb[b] = 0;
    nvb[b] = 0;
  }
#pragma unroll
  for (int b = 0; b < NB - 1; ++b) {
    const int ub = wave + 4 * b;
    if (ub < nunits) {
      locate(ub, &offb[b], &nvb[b]);
      load(offb[b], nvb[b], kb[b], vb[b]);
    }
  }
  int u = wave;
  bool more = u < nunits;
  while (more) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (more) {
        const int un = u + 4 * (NB - 1);
        const int bn = (b + NB - 1) % NB;
        if (un < nunits) {
          locate(un, &offb[bn], &nvb[bn]);
          load(offb[bn], nvb[bn], kb[bn], vb[bn]);
        }
        if (nvb[b] > 0) compute(nvb[b], kb[b], vb[b]);
        u += 4;
        more = u < nunits;
      }
    }
  }

  // reduce across row groups; lanes of group 0 then hold the wavefront's state
  __shared__ float sm_o[4][G][D];
  __shared__ float sm_m[4][G], sm_l[4][G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lw = across_sum<LPR>(l_run[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float oe = across_sum<LPR>(o[g][e]);
      if (grp == 0) sm_o[wave][g][c * EPL + e] = oe;
    }
    if (lane == 0) {
      sm_m[wave][g] = m_run[g];
      sm_l[wave][g] = lw;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += 256) {
    const int g = t / D, d = t % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      // a wavefront that saw no rows has m = -inf, l = 0, o = 0
      const float f = sm_m[ww][g] == -INFINITY ? 0.f : fast_exp2(sm_m[ww][g] - M);
      Ls += sm_l[ww][g] * f;
      O += sm_o[ww][g][d] * f;
    }
    const int hq = h * G + g;
    if (nsplit == 1) {
      ((T*)a.out)[((size_t)i * Hq + hq) * D + d] = from_f32<T>(O / Ls);
      if (d == 0) a.lse[(size_t)i * Hq + hq] = (M + __log2f(Ls)) * 0.6931471805599453f;
    } else {
      float* pp = a.part + (((size_t)w * P.Hkv + h) * G + g) * (D + 2);
      pp[d] = O;
      if (d == 0) {
        pp[D] = M;
        pp[D + 1] = Ls;
      }
    }
  }
}

// ---- a2, bf16 and d = 128: the streaming kernel -------------------------------------
//
// Same work items and output as decode_split_kernel, shaped for CDNA4's VALU:
//  - 8 lanes per row; lane c holds dims [8c, 8c+8) and [64+8c, 64+8c+8), i.e.
//    both halves of its rotate-half pairs, so each wavefront load is 8 rows x
//    128 contiguous bytes;
//  - q.k on v_dot2c_f32_bf16: the rotated, pre-scaled query is split into
//    bf16 hi + lo parts (|q - hi - lo| <= 2^-16 |q|), keys are used as stored;
//  - 3 DPP steps finish a row's dot product; 2 rows x G heads per lane per
//    16-row unit need exp2, not 4 x G;
//  - the unit's base address is wavefront-uniform, lane offsets are fixed, and
//    only partial units clamp rows.

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// nearest-even bf16 bits of a finite float (no NaN handling: queries are finite)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int G>
__global__ void __launch_bounds__(256) decode_bf16_d128_kernel(DecodeArgs a) {
  constexpr int D = 128, UR = 16;  // rows per unit: 2 groups of 8
  const DevPool& P = a.P;
  const int w = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int c8 = lane & 7, r8 = lane >> 3;

  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.prefix[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo, s = w - a.prefix[i], nsplit = a.prefix[i + 1] - a.prefix[i];
  const int slot = a.slot[i];
  const int32_t* meta = meta_of(P, slot, a.layer);
  const int n_pers = sgpr(meta[0]), n_open = sgpr(meta[1]), qpos = sgpr(meta[2]);
  const int pr = P.pr;
  const int npp = (n_pers + pr - 1) / pr, nop = (n_open + pr - 1) / pr;
  const int vp0 = s * a.split_pages, vp1 = min(npp + nop, vp0 + a.split_pages);
  const int NQ = (pr + UR - 1) / UR;
  const int nunits = (vp1 - vp0) * NQ;
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int Hq = P.Hkv * G;

  // query: rotate dims (8c8+e, 64+8c8+e) together, scale, split into hi/lo bf16 pairs
  uint32_t qh[G][8], ql[G][8];
  {
    const float2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
    float cs_c[8], cs_s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = rope[e];
      cs_c[e] = t.x;
      cs_s[e] = t.y;
    }
    const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + g) * D;
      float xa[8], xb[8], y[16];
      unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
      unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = qs * (xa[e] * cs_c[e] - xb[e] * cs_s[e]);
        y[8 + e] = qs * (xb[e] * cs_c[e] + xa[e] * cs_s[e]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t h0 = bf16_bits(y[2 * j]), h1 = bf16_bits(y[2 * j + 1]);
        const float r0 = y[2 * j] - __uint_as_float(h0 << 16);
        const float r1 = y[2 * j + 1] - __uint_as_float(h1 << 16);
        qh[g][j] = h0 | (h1 << 16);
        ql[g][j] = bf16_bits(r0) | (bf16_bits(r1) << 16);
      }
    }
  }

  float m_run[G], l_run[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[g][e] = 0.f;
  }

  const char* kbase = (const char*)P.kpool;
  const char* vbase = (const char*)P.vpool;
  const uint32_t lane_off = (uint32_t)(r8 * D + 8 * c8) * 2;  // bytes, row r8 of a group
  // unit u -> wavefront-uniform byte offset of its first row, rows present
  auto locate = [&](int u, size_t* off, int* nval) {
    const int vp = vp0 + u / NQ, qq = u % NQ;
    int page, rows;
    if (vp < npp) {
      page = sgpr(tab[vp]);
      rows = (vp == npp - 1) ? n_pers - vp * pr : pr;
    } else {
      const int j = vp - npp;
      page = sgpr(tab[P.max_pers + j]);
      rows = (j == nop - 1) ? n_open - j * pr : pr;
    }
    *off = ((((size_t)page * P.Hkv + h) * pr) + (size_t)qq * UR) * D * 2;
    *nval = rows - qq * UR;
  };
  // kr[0..3]: group 0 dims lo/hi half, group 1 dims lo/hi half
  auto load = [&](size_t off, int nval, uint4* kr, uint4* vr) {
    const char* kb = kbase + off;
    const char* vb = vbase + off;
    if (nval >= UR) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const uint32_t o2 = lane_off + rg * 8 * D * 2;
        kr[2 * rg] = *(const uint4*)(kb + o2);
        kr[2 * rg + 1] = *(const uint4*)(kb + o2 + 128);
        vr[2 * rg] = *(const uint4*)(vb + o2);
        vr[2 * rg + 1] = *(const uint4*)(vb + o2 + 128);
      }
    } else {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        int r = rg * 8 + r8;
        r = r < nval ? r : (nval > 0 ? nval - 1 : 0);
        const uint32_t o2 = (uint32_t)(r * D + 8 * c8) * 2;
        kr[2 * rg] = *(const uint4*)(kb + o2);
        kr[2 * rg + 1] = *(const uint4*)(kb + o2 + 128);
        vr[2 * rg] = *(const uint4*)(vb + o2);
        vr[2 * rg + 1] = *(const uint4*)(vb + o2 + 128);
      }
    }
  };
  auto compute = [&](int nval, const uint4* kr, const uint4* vr) {
    float sc[2][G];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const uint32_t k[8] = {kr[2 * rg].x,     kr[2 * rg].y,     kr[2 * rg].z,     kr[2 * rg].w,
                             kr[2 * rg + 1].x, kr[2 * rg + 1].y, kr[2 * rg + 1].z, kr[2 * rg + 1].w};
      const bool valid = rg * 8 + r8 < nval;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc = dot2_bf16(k[j], qh[g][j], acc);
          acc = dot2_bf16(k[j], ql[g][j], acc);
        }
        acc = group_sum<8>(acc);
        sc[rg][g] = valid ? acc : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mx = across_max<8>(fmaxf(sc[0][g], sc[1][g]));
      if (mx > m_run[g]) {  // wavefront-uniform
        const float alpha = fast_exp2(m_run[g] - mx);
        m_run[g] = mx;
        l_run[g] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[g][e] *= alpha;
      }
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float vf[16];
      unpack16(vr[2 * rg], vf, bf16_t());
      unpack16(vr[2 * rg + 1], vf + 8, bf16_t());
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(sc[rg][g] - m_run[g]);
        l_run[g] += p;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[g][e] += p * vf[e];
      }
    }
  };

  constexpr int NB = 2;
  uint4 kb[NB][4], vb[NB][4];
  size_t offb[NB] = {0, 0};
  int nvb[NB] = {0, 0};
  if (wave < nunits) {
    locate(wave, &offb[0], &nvb[0]);
    load(offb[0], nvb[0], kb[0], vb[0]);
  }
  int u = wave;
  bool more = u < nunits;
  while (more) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (more) {
        const int un = u + 4;
        const int bn = (b + 1) % NB;
        if (un < nunits) {
          locate(un, &offb[bn], &nvb[bn]);
          load(offb[bn], nvb[bn], kb[bn], vb[bn]);
        }
        if (nvb[b] > 0) compute(nvb[b], kb[b], vb[b]);
        u += 4;
        more = u < nunits;
      }
    }
  }

  // reduce across the 8 row slots of the wavefront, then across wavefronts
  __shared__ float sm_o[4][G][D];
  __shared__ float sm_m[4][G], sm_l[4][G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lw = across_sum<8>(l_run[g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float oe = across_sum<8>(o[g][e]);
      if (r8 == 0) sm_o[wave][g][(e < 8 ? 0 : 64) + 8 * c8 + (e & 7)] = oe;
    }
    if (lane == 0) {
      sm_m[wave][g] = m_run[g];
      sm_l[wave][g] = lw;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += 256) {
    const int g = t / D, d = t % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = sm_m[ww][g] == -INFINITY ? 0.f : fast_exp2(sm_m[ww][g] - M);
      Ls += sm_l[ww][g] * f;
      O += sm_o[ww][g][d] * f;
    }
    const int hq = h * G + g;
    if (nsplit == 1) {
      ((bf16_t*)a.out)[((size_t)i * Hq + hq) * D + d] = from_f32<bf16_t>(O / Ls);
      if (d == 0) a.lse[(size_t)i * Hq + hq] = (M + __log2f(Ls)) * 0.6931471805599453f;
    } else {
      float* pp = a.part + (((size_t)w * P.Hkv + h) * G + g) * (D + 2);
      pp[d] = O;
      if (d == 0) {
        pp[D] = M;
        pp[D + 1] = Ls;
      }
    }
  }
}

// ---- a2, bf16, d = 128, four query heads per KV head: LDS-staged streaming -------
//
// The workgroup streams a split's pages in units of 32 rows: every thread loads
// its 16-byte pieces of a later unit's K and V into registers (two stages in
// flight), stores the next unit into one of two LDS buffers, and the four
// wavefronts compute the current unit from LDS. Wavefront w takes query heads
// {2(w&1), 2(w&1)+1} of the group over rows [16(w>>1), 16(w>>1)+16) of each
// unit, so each V row is widened to fp32 twice (not once per head) and each
// wavefront holds two heads' query (hi/lo bf16 pairs for v_dot2c_f32_bf16) and
// accumulators. Lane (r, c) covers row r of each 8-row group and dims
// [8c, 8c+8) and [64+8c, 64+8c+8) (rotate-half partners). LDS rows are stored
// with their 16-byte chunks XOR-swizzled by (row & 7) so the 8 rows a
// wavefront reads at once fall in different banks.

template <int NQ>  // 32-row units per page (page_rows / 32)
__global__ void __launch_bounds__(256) decode_bf16_d128_g4_kernel(DecodeArgs a) {
  constexpr int D = 128, G = 4, RB = D * 2, UR = 32;  // 2 pieces of 16 B per thread
  __shared__ uint4 lk[2][UR * RB / 16], lv[2][UR * RB / 16];
  __shared__ float sm_o[2][G][D], sm_m[2][G], sm_l[2][G];
  const DevPool& P = a.P;
  const int w = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int hp = wave & 1, half = wave >> 1;  // head pair, row half
  const int c8 = lane & 7, r8 = lane >> 3;

  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.prefix[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo, s = w - a.prefix[i], nsplit = a.prefix[i + 1] - a.prefix[i];
  const int slot = a.slot[i];
  const int32_t* meta = meta_of(P, slot, a.layer);
  const int n_pers = sgpr(meta[0]), n_open = sgpr(meta[1]), qpos = sgpr(meta[2]);
  const int pr = NQ * UR;
  const int npp = (n_pers + pr - 1) / pr, nop = (n_open + pr - 1) / pr;
  const int vp0 = s * a.split_pages, vp1 = min(npp + nop, vp0 + a.split_pages);
  const int nunits = (vp1 - vp0) * NQ;
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int Hq = P.Hkv * G;

  // this wavefront's two query heads: rotate, scale, split into hi/lo bf16 pairs
  uint32_t qh[2][8], ql[2][8];
  {
    const float2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
    float cs_c[8], cs_s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = rope[e];
      cs_c[e] = t.x;
      cs_s[e] = t.y;
    }
    const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + 2 * hp + j2) * D;
      float xa[8], xb[8], y[16];
      unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
      unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = qs * (xa[e] * cs_c[e] - xb[e] * cs_s[e]);
        y[8 + e] = qs * (xb[e] * cs_c[e] + xa[e] * cs_s[e]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t h0 = bf16_bits(y[2 * j]), h1 = bf16_bits(y[2 * j + 1]);
        qh[j2][j] = h0 | (h1 << 16);
        ql[j2][j] = bf16_bits(y[2 * j] - __uint_as_float(h0 << 16)) |
                    (bf16_bits(y[2 * j + 1] - __uint_as_float(h1 << 16)) << 16);
      }
    }
  }

  // unit u -> wavefront-uniform byte offset of its first row, rows present
  auto locate = [&](int u, size_t* off, int* nval) __attribute__((always_inline)) {
    const int vp = vp0 + (NQ == 1 ? u : u >> 1), qq = NQ == 1 ? 0 : (u & 1);
    int page, rows;
    if (vp < npp) {
      page = sgpr(tab[vp]);
      rows = (vp == npp - 1) ? n_pers - vp * pr : pr;
    } else {
      const int j = vp - npp;
      page = sgpr(tab[P.max_pers + j]);
      rows = (j == nop - 1) ? n_open - j * pr : pr;
    }
    *off = ((((size_t)page * P.Hkv + h) * pr) + (size_t)qq * UR) * RB;
    *nval = rows - qq * UR;
  };
  const char* kbase = (const char*)P.kpool;
  const char* vbase = (const char*)P.vpool;
  // piece ch of this thread: row (t + 256 ch) / 16, chunk (t + 256 ch) % 16
  const int prow0 = threadIdx.x >> 4, pchunk = threadIdx.x & 15;
  const int lds0 = prow0 * 16 + (pchunk ^ (prow0 & 7));  // swizzled LDS slot (rows +16 for ch 1)
  uint4 ak0, av0, ak1, av1, bk0, bv0, bk1, bv1;
  auto gload = [&](int u, uint4* k0, uint4* v0, uint4* k1, uint4* v1) __attribute__((always_inline)) {
    size_t off;
    int nval;
    locate(u, &off, &nval);
    int r0 = prow0, r1 = prow0 + 16;
    if (nval < UR) {
      const int last = nval > 0 ? nval - 1 : 0;
      r0 = r0 < nval ? r0 : last;
      r1 = r1 < nval ? r1 : last;
    }
    const char* kb = kbase + off + pchunk * 16;
    const char* vb = vbase + off + pchunk * 16;
    *k0 = *(const uint4*)(kb + r0 * RB);
    *v0 = *(const uint4*)(vb + r0 * RB);
    *k1 = *(const uint4*)(kb + r1 * RB);
    *v1 = *(const uint4*)(vb + r1 * RB);
  };
  auto swrite = [&](int b, const uint4& k0, const uint4& v0, const uint4& k1, const uint4& v1)
      __attribute__((always_inline)) {
    lk[b][lds0] = k0;
    lv[b][lds0] = v0;
    lk[b][lds0 + 256] = k1;
    lv[b][lds0 + 256] = v1;
  };

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, o[2][16];
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[j2][e] = 0.f;

  auto compute = [&](int b, int nval) __attribute__((always_inline)) {
    float sc[2][2];  // [row group][head]
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int row = half * 16 + rg * 8 + r8;
      const int sw = r8;  // row & 7
      const uint4 ka = lk[b][row * 16 + (c8 ^ sw)];
      const uint4 kb = lk[b][row * 16 + 8 + (c8 ^ sw)];
      const uint32_t k[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
      const bool valid = row < nval;
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc0 = dot2_bf16(k[j], qh[j2][j], acc0);
          acc1 = dot2_bf16(k[j], ql[j2][j], acc1);
        }
        const float acc = group_sum<8>(acc0 + acc1);
        sc[rg][j2] = valid ? acc : -INFINITY;
      }
    }
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const float mx = slots8_max(fmaxf(sc[0][j2], sc[1][j2]));
      if (mx > m_run[j2]) {  // wavefront-uniform; -inf when this half has no rows
        const float alpha = fast_exp2(m_run[j2] - mx);
        m_run[j2] = mx;
        l_run[j2] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j2][e] *= alpha;
      }
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int row = half * 16 + rg * 8 + r8;
      float vf[16];
      unpack16(lv[b][row * 16 + (c8 ^ r8)], vf, bf16_t());
      unpack16(lv[b][row * 16 + 8 + (c8 ^ r8)], vf + 8, bf16_t());
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const float p = m_run[j2] == -INFINITY ? 0.f : fast_exp2(sc[rg][j2] - m_run[j2]);
        l_run[j2] += p;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[j2][e] += p * vf[e];
      }
    }
  };

  // Prologue: unit 0 in LDS buffer 0, units 1 (stage a) and 2 (stage b) in
  // flight. Every step issues the same loads and stores whatever the unit count
  // (indices past the end re-read the last unit, which is still in L2), so the
  // waits before each store can count exactly the newer stage's loads.
  const int ulast = nunits - 1;
  gload(0, &ak0, &av0, &ak1, &av1);
  swrite(0, ak0, av0, ak1, av1);
  gload(min(1, ulast), &ak0, &av0, &ak1, &av1);
  gload(min(2, ulast), &bk0, &bv0, &bk1, &bv1);
  __syncthreads();
  auto step = [&](int u, uint4& k0, uint4& v0, uint4& k1, uint4& v1) __attribute__((always_inline)) {
    const int b = u & 1;
    swrite(b ^ 1, k0, v0, k1, v1);  // its buffer was last read before the previous barrier
    gload(min(u + 3, ulast), &k0, &v0, &k1, &v1);
    if (u < nunits) {
      size_t off;
      int nval;
      locate(u, &off, &nval);
      if (nval > half * 16) compute(b, nval);
    }
    __syncthreads();
  };
  for (int u = 0; u < nunits; u += 2) {
    step(u, ak0, av0, ak1, av1);
    step(u + 1, bk0, bv0, bk1, bv1);
  }

  // reduce over the 8 row slots, then merge the two row halves of each head
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const float lw = slots8_sum(l_run[j2]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float oe = slots8_sum(o[j2][e]);
      if (r8 == 0) sm_o[half][2 * hp + j2][(e < 8 ? 0 : 64) + 8 * c8 + (e & 7)] = oe;
    }
    if (lane == 0) {
      sm_m[half][2 * hp + j2] = m_run[j2];
      sm_l[half][2 * hp + j2] = lw;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += 256) {
    const int g = t / D, d = t % D;
    const float m0 = sm_m[0][g], m1 = sm_m[1][g];
    const float M = fmaxf(m0, m1);
    const float f0 = m0 == -INFINITY ? 0.f : fast_exp2(m0 - M);
    const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
    const float Ls = sm_l[0][g] * f0 + sm_l[1][g] * f1;
    const float O = sm_o[0][g][d] * f0 + sm_o[1][g][d] * f1;
    const int hq = h * G + g;
    if (nsplit == 1) {
      ((bf16_t*)a.out)[((size_t)i * Hq + hq) * D + d] = from_f32<bf16_t>(O / Ls);
      if (d == 0) a.lse[(size_t)i * Hq + hq] = (M + __log2f(Ls)) * 0.6931471805599453f;
    } else {
      float* pp = a.part + (((size_t)w * P.Hkv + h) * G + g) * (D + 2);
      pp[d] = O;
      if (d == 0) {
        pp[D] = M;
        pp[D + 1] = Ls;
      }
    }
  }
}

// ---- a2 + a3, persistent stream-K form of the kernel above ------------------------
//
// One resident wave of workgroups; workgroup w walks flattened units
// [w*T, (w+1)*T), which cover one or a few (sequence, KV head) segments. Per
// segment it runs the same LDS-staged pipeline and math as
// decode_bf16_d128_g4_kernel, then writes the final output (segment inside
// this workgroup) or a partial for decode_stream_merge_kernel. Every workgroup
// does the same amount of streaming, and the per-workgroup set-up (sequence
// lookup, metadata, query rotation, first loads) is paid per segment, not per
// fixed-size split.

template <int NQ>
__global__ void __launch_bounds__(256) decode_stream_kernel(StreamArgs a) {
  constexpr int D = 128, G = 4, RB = D * 2, UR = 32;
  __shared__ uint4 lk[2][UR * RB / 16], lv[2][UR * RB / 16];
  __shared__ float sm_o[2][G][D], sm_m[2][G], sm_l[2][G];
  const DevPool& P = a.P;
  const int w = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int hp = wave & 1, half = wave >> 1;
  const int c8 = lane & 7, r8 = lane >> 3;
  const int pr = NQ * UR;
  const int Hq = P.Hkv * G;
  const char* kbase = (const char*)P.kpool;
  const char* vbase = (const char*)P.vpool;
  const int prow0 = threadIdx.x >> 4, pchunk = threadIdx.x & 15;
  const int lds0 = prow0 * 16 + (pchunk ^ (prow0 & 7));

  int F = w * a.T;
  const int Fend = min(a.U, F + a.T);
  int i = 0;
  while (F < Fend) {
    while (a.useg[i + 1] <= F) ++i;  // sequence of flattened unit F (scalar)
    const int units = (a.useg[i + 1] - a.useg[i]) / P.Hkv;
    const int rel = F - a.useg[i];
    const int h = rel / units, lu0 = rel % units;
    const int segS = a.useg[i] + h * units;
    const int F1 = min(Fend, segS + units);
    const int nunits = F1 - F;
    const int slot = a.slot[i];
    const int32_t* meta = meta_of(P, slot, a.layer);
    const int n_pers = sgpr(meta[0]), n_open = sgpr(meta[1]), qpos = sgpr(meta[2]);
    const int npp = (n_pers + pr - 1) / pr, nop = (n_open + pr - 1) / pr;
    const int32_t* tab = ptab_of(P, slot, a.layer);

    uint32_t qh[2][8], ql[2][8];
    {
      const float2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
      float cs_c[8], cs_s[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 t = rope[e];
        cs_c[e] = t.x;
        cs_s[e] = t.y;
      }
      const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + 2 * hp + j2) * D;
        float xa[8], xb[8], y[16];
        unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
        unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = qs * (xa[e] * cs_c[e] - xb[e] * cs_s[e]);
          y[8 + e] = qs * (xb[e] * cs_c[e] + xa[e] * cs_s[e]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t h0 = bf16_bits(y[2 * j]), h1 = bf16_bits(y[2 * j + 1]);
          qh[j2][j] = h0 | (h1 << 16);
          ql[j2][j] = bf16_bits(y[2 * j] - __uint_as_float(h0 << 16)) |
                      (bf16_bits(y[2 * j + 1] - __uint_as_float(h1 << 16)) << 16);
        }
      }
    }

    // segment-local unit u -> byte offset of its first row, rows present
    auto locate = [&](int u, size_t* off, int* nval) __attribute__((always_inline)) {
      const int lu = lu0 + u;
      const int vp = NQ == 1 ? lu : lu >> 1, qq = NQ == 1 ? 0 : (lu & 1);
      int page, rows;
      if (vp < npp) {
        page = sgpr(tab[vp]);
        rows = (vp == npp - 1) ? n_pers - vp * pr : pr;
      } else {
        const int j = vp - npp;
        page = sgpr(tab[P.max_pers + j]);
        rows = (j == nop - 1) ? n_open - j * pr : pr;
      }
      *off = ((((size_t)page * P.Hkv + h) * pr) + (size_t)qq * UR) * RB;
      *nval = rows - qq * UR;
    };
    uint4 ak0, av0, ak1, av1, bk0, bv0, bk1, bv1;
    auto gload = [&](int u, uint4* k0, uint4* v0, uint4* k1, uint4* v1) __attribute__((always_inline)) {
      size_t off;
      int nval;
      locate(u, &off, &nval);
      int r0 = prow0, r1 = prow0 + 16;
      if (nval < UR) {
        const int last = nval > 0 ? nval - 1 : 0;
        r0 = r0 < nval ? r0 : last;
        r1 = r1 < nval ? r1 : last;
      }
      const char* kb = kbase + off + pchunk * 16;
      const char* vb = vbase + off + pchunk * 16;
      *k0 = *(const uint4*)(kb + r0 * RB);
      *v0 = *(const uint4*)(vb + r0 * RB);
      *k1 = *(const uint4*)(kb + r1 * RB);
      *v1 = *(const uint4*)(vb + r1 * RB);
    };
    auto swrite = [&](int b, const uint4& k0, const uint4& v0, const uint4& k1, const uint4& v1)
        __attribute__((always_inline)) {
      lk[b][lds0] = k0;
      lv[b][lds0] = v0;
      lk[b][lds0 + 256] = k1;
      lv[b][lds0 + 256] = v1;
    };

    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, o[2][16];
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j2][e] = 0.f;

    auto compute = [&](int b, int nval) __attribute__((always_inline)) {
      float sc[2][2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int row = half * 16 + rg * 8 + r8;
        const uint4 ka = lk[b][row * 16 + (c8 ^ r8)];
        const uint4 kb = lk[b][row * 16 + 8 + (c8 ^ r8)];
        const uint32_t k[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
        const bool valid = row < nval;
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            acc0 = dot2_bf16(k[j], qh[j2][j], acc0);
            acc1 = dot2_bf16(k[j], ql[j2][j], acc1);
          }
          const float acc = group_sum<8>(acc0 + acc1);
          sc[rg][j2] = valid ? acc : -INFINITY;
        }
      }
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const float mx = slots8_max(fmaxf(sc[0][j2], sc[1][j2]));
        if (mx > m_run[j2]) {
          const float alpha = fast_exp2(m_run[j2] - mx);
          m_run[j2] = mx;
          l_run[j2] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j2][e] *= alpha;
        }
      }
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int row = half * 16 + rg * 8 + r8;
        float vf[16];
        unpack16(lv[b][row * 16 + (c8 ^ r8)], vf, bf16_t());
        unpack16(lv[b][row * 16 + 8 + (c8 ^ r8)], vf + 8, bf16_t());
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const float p = m_run[j2] == -INFINITY ? 0.f : fast_exp2(sc[rg][j2] - m_run[j2]);
          l_run[j2] += p;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[j2][e] += p * vf[e];
        }
      }
    };

    const int ulast = nunits - 1;
    gload(0, &ak0, &av0, &ak1, &av1);
    swrite(0, ak0, av0, ak1, av1);
    gload(min(1, ulast), &ak0, &av0, &ak1, &av1);
    gload(min(2, ulast), &bk0, &bv0, &bk1, &bv1);
    __syncthreads();
    auto step = [&](int u, uint4& k0, uint4& v0, uint4& k1, uint4& v1) __attribute__((always_inline)) {
      const int b = u & 1;
      swrite(b ^ 1, k0, v0, k1, v1);
      gload(min(u + 3, ulast), &k0, &v0, &k1, &v1);
      if (u < nunits) {
        size_t off;
        int nval;
        locate(u, &off, &nval);
        if (nval > half * 16) compute(b, nval);
      }
      __syncthreads();
    };
    for (int u = 0; u < nunits; u += 2) {
      step(u, ak0, av0, ak1, av1);
      step(u + 1, bk0, bv0, bk1, bv1);
    }

#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const float lw = slots8_sum(l_run[j2]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float oe = slots8_sum(o[j2][e]);
        if (r8 == 0) sm_o[half][2 * hp + j2][(e < 8 ? 0 : 64) + 8 * c8 + (e & 7)] = oe;
      }
      if (lane == 0) {
        sm_m[half][2 * hp + j2] = m_run[j2];
        sm_l[half][2 * hp + j2] = lw;
      }
    }
    __syncthreads();
    const int wa = segS / a.T, wb = (segS + units - 1) / a.T;
    for (int t = threadIdx.x; t < G * D; t += 256) {
      const int g = t / D, d = t % D;
      const float m0 = sm_m[0][g], m1 = sm_m[1][g];
      const float M = fmaxf(m0, m1);
      const float f0 = m0 == -INFINITY ? 0.f : fast_exp2(m0 - M);
      const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
      const float Ls = sm_l[0][g] * f0 + sm_l[1][g] * f1;
      const float O = sm_o[0][g][d] * f0 + sm_o[1][g][d] * f1;
      const int hq = h * G + g;
      if (wa == wb) {
        ((bf16_t*)a.out)[((size_t)i * Hq + hq) * D + d] = from_f32<bf16_t>(O / Ls);
        if (d == 0) a.lse[(size_t)i * Hq + hq] = (M + __log2f(Ls)) * 0.6931471805599453f;
      } else {
        float* pp = a.part + ((((size_t)i * P.Hkv + h) * a.maxp + (w - wa)) * G + g) * (D + 2);
        pp[d] = O;
        if (d == 0) {
          pp[D] = M;
          pp[D + 1] = Ls;
        }
      }
    }
    __syncthreads();  // LDS (buffers and merge area) is reused by the next segment
    F = F1;
  }
}

// Merge the partials of (sequence i, KV head h) written by workgroups wa..wb.
__global__ void __launch_bounds__(512) decode_stream_merge_kernel(StreamArgs a) {
  constexpr int D = 128, G = 4;
  __shared__ float sm_w[kMaxSplits * G], sm_M[G], sm_L[G];
  const int i = blockIdx.x, h = blockIdx.y;
  const int Hkv = a.P.Hkv, Hq = Hkv * G;
  const int units = (a.useg[i + 1] - a.useg[i]) / Hkv;
  const int segS = a.useg[i] + h * units;
  const int wa = segS / a.T, wb = (segS + units - 1) / a.T;
  const int ns = wb - wa + 1;
  if (ns == 1) return;
  auto part = [&](int s, int g) {
    return a.part + ((((size_t)i * Hkv + h) * a.maxp + s) * G + g) * (D + 2);
  };
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY;
    for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, part(s2, g)[D]);
    float Ls = 0.f;
    for (int s2 = 0; s2 < ns; ++s2) {
      const float f = fast_exp2(part(s2, g)[D] - M);
      sm_w[s2 * G + g] = f;
      Ls += part(s2, g)[D + 1] * f;
    }
    sm_M[g] = M;
    sm_L[g] = Ls;
    a.lse[(size_t)i * Hq + h * G + g] = (M + __log2f(Ls)) * 0.6931471805599453f;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int g = t / D, d = t % D;
    float O = 0.f;
    for (int s2 = 0; s2 < ns; ++s2) O += part(s2, g)[d] * sm_w[s2 * G + g];
    ((bf16_t*)a.out)[((size_t)i * Hq + h * G + g) * D + d] = from_f32<bf16_t>(O / sm_L[g]);
  }
}

// ---- a7: the open block's rows leave the device view -----------------------------

__global__ void free_kernel(FreeArgs a) {
  const int i = blockIdx.x;
  for (int l = threadIdx.x; l < a.P.L; l += blockDim.x)
    a.P.meta[(a.slot[i] * a.P.L + l) * 4 + 1] = 0;
}

// ---- prompt rows -----------------------------------------------------------------

template <typename T, int D>
__global__ void __launch_bounds__(1024) prompt_kernel(PromptArgs a) {
  const DevPool& P = a.P;
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x == 0) {
    int32_t* meta = P.meta + (a.slot * P.L + a.layer) * 4;
    meta[0] = a.prompt_len;
    meta[1] = 0;
    meta[2] = a.prompt_len - 1;
  }
  if (r == 0) {
    int32_t* tab = ptab_of(P, a.slot, a.layer);
    for (int t = threadIdx.x; t < (a.prompt_len + P.pr - 1) / P.pr; t += blockDim.x)
      tab[t] = a.pages[t];
  }
  if (r >= a.prompt_len) return;
  const int page = a.pages[r / P.pr], srow = r % P.pr;
  const T* k = (const T*)a.k + (size_t)r * P.Hkv * D;
  const T* v = (const T*)a.v + (size_t)r * P.Hkv * D;
  const float2* rope = P.rope + (size_t)r * (D / 2);
  for (int t = threadIdx.x; t < P.Hkv * (D / 2); t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const float x1 = to_f32(k[hh * D + j]), x2 = to_f32(k[hh * D + j + D / 2]);
    const float2 cs = rope[j];
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.kpool)[o + j] = from_f32<T>(x1 * cs.x - x2 * cs.y);
    ((T*)P.kpool)[o + j + D / 2] = from_f32<T>(x2 * cs.x + x1 * cs.y);
    ((T*)P.vpool)[o + j] = v[hh * D + j];
    ((T*)P.vpool)[o + j + D / 2] = v[hh * D + j + D / 2];
  }
  if (threadIdx.x == 0) P.pos[(size_t)page * P.pr + srow] = r;
}

// ---- a4 + a6: pause RoPE at bit-reversed in-block positions, code-row scatter ----

__device__ __forceinline__ int bitrev_dev(int k, int nbits) {
  return nbits == 0 ? 0 : (int)(__brev((unsigned)k) >> (32 - nbits));
}

template <typename T, int D>
__global__ void __launch_bounds__(1024) pause_rope_scatter_kernel(CompressArgs a) {
  const DevPool& P = a.P;
  const int k = blockIdx.x, i = blockIdx.y;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], pers_before = rec[2], prompt = rec[3];
  const int pages_off = rec[4], npages = rec[5], first_new = rec[6];
  const int pos = prompt + blk * P.C + bitrev_dev(k, a.log2Kp) * (P.C / a.Kp);
  const T* kin = (const T*)a.kp + ((size_t)i * a.Kp + k) * P.Hkv * D;
  const T* vin = (const T*)a.vp + ((size_t)i * a.Kp + k) * P.Hkv * D;
  const float2* rope = P.rope + (size_t)pos * (D / 2);
  const bool keep = k < a.quota;
  int page = 0, srow = 0;
  if (keep) {
    const int row = pers_before + k;
    page = a.desc[pages_off + row / P.pr - pers_before / P.pr];
    srow = row % P.pr;
  }
  for (int t = threadIdx.x; t < P.Hkv * (D / 2); t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const float x1 = to_f32(kin[hh * D + j]), x2 = to_f32(kin[hh * D + j + D / 2]);
    const float2 cs = rope[j];
    const T y1 = from_f32<T>(x1 * cs.x - x2 * cs.y);
    const T y2 = from_f32<T>(x2 * cs.x + x1 * cs.y);
    T* kr = (T*)a.kp_rot + (((size_t)i * P.Hkv + hh) * a.Kp + k) * D;
    kr[j] = y1;
    kr[j + D / 2] = y2;
    if (keep) {
      const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
      ((T*)P.kpool)[o + j] = y1;
      ((T*)P.kpool)[o + j + D / 2] = y2;
      ((T*)P.vpool)[o + j] = vin[hh * D + j];
      ((T*)P.vpool)[o + j + D / 2] = vin[hh * D + j + D / 2];
    }
  }
  if (keep && threadIdx.x == 0) P.pos[(size_t)page * P.pr + srow] = pos;
  if (k == 0 && threadIdx.x == 0) {
    int32_t* tab = ptab_of(P, slot, a.layer);
    const int first_idx = pers_before / P.pr;
    for (int j = first_new; j < npages; ++j) tab[first_idx + j] = a.desc[pages_off + j];
    P.meta[(slot * P.L + a.layer) * 4 + 0] = pers_before + a.quota;
  }
}

// ---- a5: pause-token attention under the block mask (SIMT form) -------------------
//
// One wavefront per (sequence, pause j, query head). Keys: the sequence's
// resident rows at this layer (prompt, earlier code rows, the whole block)
// followed by the rotated pause keys 0..j. 64 keys per step: one lane per key
// scores it, the wavefront takes the step's max, and each lane accumulates
// its D/64 output dims over the step.

template <typename T, int D>
__global__ void __launch_bounds__(64) compress_attn_simt_kernel(CompressArgs a) {
  const DevPool& P = a.P;
  const int j = blockIdx.x, hq = blockIdx.y, i = blockIdx.z;
  const int lane = threadIdx.x;
  const int hk = hq / a.G;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], n_pers = rec[2], prompt = rec[3];
  const int n_ctx = n_pers + P.C;
  const int n_keys = n_ctx + j + 1;
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int pos = prompt + blk * P.C + bitrev_dev(j, a.log2Kp) * (P.C / a.Kp);

  __shared__ float qs[D];
  __shared__ float ps[64];
  {
    const float2* rope = P.rope + (size_t)pos * (D / 2);
    const T* qh = (const T*)a.qp + (((size_t)i * a.Kp + j) * a.Hq + hq) * D;
    const float sc = 1.4426950408889634f / sqrtf((float)D);
    for (int d = lane; d < D; d += 64)
      qs[d] = sc * rope_elem<D>([&](int e) { return to_f32(qh[e]); }, d, rope);
  }
  __syncthreads();

  auto key_row = [&](int r, const T** kr, const T** vr) {
    if (r < n_ctx) {
      int page, srow;
      if (r < n_pers) {
        page = tab[r / P.pr];
        srow = r % P.pr;
      } else {
        const int o = r - n_pers;
        page = tab[P.max_pers + o / P.pr];
        srow = o % P.pr;
      }
      const size_t off = (((size_t)page * P.Hkv + hk) * P.pr + srow) * D;
      *kr = (const T*)P.kpool + off;
      *vr = (const T*)P.vpool + off;
    } else {
      const int kk = r - n_ctx;
      *kr = (const T*)a.kp_rot + (((size_t)i * P.Hkv + hk) * a.Kp + kk) * D;
      *vr = (const T*)a.vp + (((size_t)i * a.Kp + kk) * P.Hkv + hk) * D;
    }
  };

  constexpr int DPL = (D + 63) / 64;
  float m = -INFINITY, l = 0.f, o[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) o[t] = 0.f;
  for (int r0 = 0; r0 < n_keys; r0 += 64) {
    const int r = r0 + lane;
    float s = -INFINITY;
    if (r < n_keys) {
      const T *kr, *vr;
      key_row(r, &kr, &vr);
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += qs[d] * to_f32(kr[d]);
      s = acc;
    }
    float mx = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    const float p = fast_exp2(s - mn);
    float psum = p;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) psum += __shfl_xor(psum, off);
    l = l * alpha + psum;
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[t] *= alpha;
    const int nr = min(64, n_keys - r0);
    for (int rr = 0; rr < nr; ++rr) {
      const T *kr, *vr;
      key_row(r0 + rr, &kr, &vr);
      const float pr_ = ps[rr];
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        const int d = lane + 64 * t;
        if (d < D) o[t] += pr_ * to_f32(vr[d]);
      }
    }
  }
  T* out = (T*)a.out + (((size_t)i * a.Kp + j) * a.Hq + hq) * D;
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    const int d = lane + 64 * t;
    if (d < D) out[d] = from_f32<T>(o[t] / l);
  }
  if (lane == 0) a.lse[((size_t)i * a.Kp + j) * a.Hq + hq] = (m + __log2f(l)) * 0.6931471805599453f;
}

// ---- a5 on bf16 MFMA (d = 128, four query heads per KV head, 64-row pages) -------
//
// Workgroup = (sequence, KV head, tile of 128 query rows); query row r is pause
// r/4, head 4h + r%4. Each of the 4 wavefronts owns 32 query rows (two 16-row
// N-blocks). For every 64-key tile (a context page, then pause-key tiles):
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = the
//                 rotated query (hi + lo bf16 parts, so the product keeps fp32
//                 accuracy), C lane l = keys 4(l/16)+i x query l%16;
//   online softmax per query column, all lane-local plus permlane swaps;
//   O^T += V^T P^T: B = P^T straight from the S^T registers (bf16), A = V^T
//                 from a transposed LDS tile.
// The M-blocks of S^T take keys 32(mb/2) + 8(m/4) + 4(mb%2) + m%4 so that for
// each 32-key step a lane's 8 probabilities are 8 consecutive keys, which is
// one 16-byte read of the transposed V tile. K rows in LDS have their 16-byte
// chunks XOR-swizzled by row so the 16 rows an A-operand read touches use
// different banks. The next tile is loaded into registers while the current
// one is computed; LDS is double-buffered (64 KB).

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

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

__global__ void __launch_bounds__(256) compress_attn_mfma_kernel(CompressArgs a) {
  constexpr int D = 128, G = 4, TK = 64, RB = D * 2;
  __shared__ uint4 lk[2][TK * RB / 16];   // K rows, chunks swizzled by (row & 15)
  __shared__ uint4 lvt[2][D * TK * 2 / 16];  // V^T: [dim][64 keys] bf16, 128 B per dim
  const DevPool& P = a.P;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // workgroup -> (pair = sequence x KV head, query tile); the tiles of one pair
  // share blockIdx.x mod 8, i.e. one XCD and its L2
  const int ntq = (4 * a.Kp + 127) / 128;
  const int npair = a.n * P.Hkv;
  const int b = blockIdx.x, xcd = b & 7, jj = b >> 3;
  const int pair = (jj / ntq) * 8 + xcd, qt = jj % ntq;
  if (pair >= npair) return;
  const int i = pair / P.Hkv, hk = pair % P.Hkv;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], n_pers = rec[2], prompt = rec[3];
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int npp = (n_pers + TK - 1) / TK, nop = P.C / TK;
  const int ntc = npp + nop;  // context tiles
  const int q0 = qt * 128;    // first query row of the workgroup
  const int nq = min(128, 4 * a.Kp - q0);
  const int last_pause = (q0 + nq - 1) >> 2;
  const int ntp = last_pause / TK + 1;  // pause-key tiles
  const int ntiles = ntc + ntp;

  // ---- the wavefront's query rows: rotate at the bitrev position, scale, hi/lo
  uint4 qh[2][4], ql[2][4];  // [N-block][k-step]: dims 32ks + 8 g4 + 0..7
  int qpause[2];
  {
    const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int r = q0 + wave * 32 + nb * 16 + l16;
      const bool rv = r < q0 + nq;
      r = rv ? r : q0;
      const int pz = r >> 2, hh = r & 3;
      qpause[nb] = rv ? pz : -1;
      const int pos = prompt + blk * P.C + bitrev_dev(pz, a.log2Kp) * (P.C / a.Kp);
      const bf16_t* qrow = (const bf16_t*)a.qp + (((size_t)i * a.Kp + pz) * a.Hq + hk * G + hh) * D;
      float x[4][8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) unpack16(*(const uint4*)(qrow + 32 * ks + 8 * g4), x[ks], bf16_t());
      const float2* rope = P.rope + (size_t)pos * (D / 2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float y0[8], y1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float2 cs = rope[32 * ks + 8 * g4 + j];
          y0[j] = qs * (x[ks][j] * cs.x - x[ks + 2][j] * cs.y);
          y1[j] = qs * (x[ks + 2][j] * cs.x + x[ks][j] * cs.y);
        }
        uint32_t h0[4], l0[4], h1[4], l1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t a0 = bf16_bits(y0[2 * j]), a1 = bf16_bits(y0[2 * j + 1]);
          h0[j] = a0 | (a1 << 16);
          l0[j] = bf16_bits(y0[2 * j] - __uint_as_float(a0 << 16)) |
                  (bf16_bits(y0[2 * j + 1] - __uint_as_float(a1 << 16)) << 16);
          a0 = bf16_bits(y1[2 * j]);
          a1 = bf16_bits(y1[2 * j + 1]);
          h1[j] = a0 | (a1 << 16);
          l1[j] = bf16_bits(y1[2 * j] - __uint_as_float(a0 << 16)) |
                  (bf16_bits(y1[2 * j + 1] - __uint_as_float(a1 << 16)) << 16);
        }
        qh[nb][ks] = make_uint4(h0[0], h0[1], h0[2], h0[3]);
        ql[nb][ks] = make_uint4(l0[0], l0[1], l0[2], l0[3]);
        qh[nb][ks + 2] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
        ql[nb][ks + 2] = make_uint4(l1[0], l1[1], l1[2], l1[3]);
      }
    }
  }

  // ---- tile t -> rows: thread t loads rows (tid/16 + 16 c), chunk tid%16
  const int trow = threadIdx.x >> 4, tchunk = threadIdx.x & 15;
  // staged rows of the next tile, named so they stay in registers
  uint4 sk0, sk1, sk2, sk3, sv0, sv1, sv2, sv3;
  auto tile_src = [&](int t, const char** kb, const char** vb, size_t* kstride, size_t* vstride,
                      int* nval) __attribute__((always_inline)) {
    if (t < ntc) {
      int page, rows;
      if (t < npp) {
        page = sgpr(tab[t]);
        rows = (t == npp - 1) ? n_pers - t * TK : TK;
      } else {
        page = sgpr(tab[P.max_pers + (t - npp)]);
        rows = TK;
      }
      const size_t off = (((size_t)page * P.Hkv + hk) * TK) * RB;
      *kb = (const char*)P.kpool + off;
      *vb = (const char*)P.vpool + off;
      *kstride = RB;
      *vstride = RB;
      *nval = rows;
    } else {
      const int k0 = (t - ntc) * TK;
      *kb = (const char*)a.kp_rot + (((size_t)i * P.Hkv + hk) * a.Kp + k0) * RB;
      *vb = (const char*)a.vp + (((size_t)i * a.Kp + k0) * P.Hkv + hk) * RB;
      *kstride = RB;
      *vstride = (size_t)P.Hkv * RB;
      *nval = min(TK, a.Kp - k0);
    }
  };
  auto gload = [&](int t) __attribute__((always_inline)) {
    const char *kb, *vb;
    size_t ks, vs;
    int nval;
    tile_src(t, &kb, &vb, &ks, &vs, &nval);
    auto piece = [&](int c, uint4& kx, uint4& vx) __attribute__((always_inline)) {
      int r = trow + 16 * c;
      r = r < nval ? r : nval - 1;
      kx = *(const uint4*)(kb + r * ks + tchunk * 16);
      vx = *(const uint4*)(vb + r * vs + tchunk * 16);
    };
    piece(0, sk0, sv0);
    piece(1, sk1, sv1);
    piece(2, sk2, sv2);
    piece(3, sk3, sv3);
  };
  auto swrite = [&](int buf) __attribute__((always_inline)) {
    uint16_t* vt = (uint16_t*)lvt[buf];
    auto piece = [&](int c, const uint4& kx, const uint4& vx) __attribute__((always_inline)) {
      const int r = trow + 16 * c;
      lk[buf][r * 16 + (tchunk ^ (r & 15))] = kx;
      // V^T: dims 8 tchunk .. +8 of key r -> [dim][key]
      const int d0 = 8 * tchunk;
      vt[(d0 + 0) * TK + r] = (uint16_t)vx.x;
      vt[(d0 + 1) * TK + r] = (uint16_t)(vx.x >> 16);
      vt[(d0 + 2) * TK + r] = (uint16_t)vx.y;
      vt[(d0 + 3) * TK + r] = (uint16_t)(vx.y >> 16);
      vt[(d0 + 4) * TK + r] = (uint16_t)vx.z;
      vt[(d0 + 5) * TK + r] = (uint16_t)(vx.z >> 16);
      vt[(d0 + 6) * TK + r] = (uint16_t)vx.w;
      vt[(d0 + 7) * TK + r] = (uint16_t)(vx.w >> 16);
    };
    piece(0, sk0, sv0);
    piece(1, sk1, sv1);
    piece(2, sk2, sv2);
    piece(3, sk3, sv3);
  };

  // key of S^T M-block mb, row m (see above)
  auto keyof = [](int mb, int m) { return 32 * (mb >> 1) + 8 * (m >> 2) + 4 * (mb & 1) + (m & 3); };

  f32x4_t acc_o[2][8];  // [N-block][dim block]
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc_o[nb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  auto compute = [&](int t, int buf) __attribute__((always_inline)) {
    const bool ctx = t < ntc;
    int nval;
    {
      const char *kb, *vb;
      size_t ks, vs;
      tile_src(t, &kb, &vb, &ks, &vs, &nval);
    }
    const int kbase = ctx ? 0 : (t - ntc) * TK;  // pause index of key 0 of a pause tile
    f32x4_t s[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int kr = keyof(mb, l16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 ka = lk[buf][kr * 16 + ((4 * ks + g4) ^ (kr & 15))];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          s[mb][nb] = mfma_bf16(ka, qh[nb][ks], s[mb][nb]);
          s[mb][nb] = mfma_bf16(ka, ql[nb][ks], s[mb][nb]);
        }
      }
    }
    // mask, online softmax per query column (lane-local after the row swaps)
    uint4 pb[2][2];  // [N-block][32-key step]: bf16 probabilities, 8 keys
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = keyof(mb, 4 * g4 + e);
          bool ok = key < nval;
          if (!ctx) ok = ok && (kbase + key <= qpause[nb]);
          const float v = ok ? s[mb][nb][e] : -INFINITY;
          s[mb][nb][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = rows4_max(mx);
      const float mn = fmaxf(m_run[nb], mx);
      const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_run[nb] - mn);
      m_run[nb] = mn;
      float ps = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = mn == -INFINITY ? 0.f : fast_exp2(s[mb][nb][e] - mn);
          s[mb][nb][e] = p;  // the score register now holds its probability
          ps += p;
        }
      l_run[nb] = l_run[nb] * alpha + ps;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc_o[nb][db] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // keys 32kk + 8 g4 + j: j < 4 from M-block 2kk, j >= 4 from 2kk+1
        const f32x4_t u0 = s[2 * kk][nb], u1 = s[2 * kk + 1][nb];
        pb[nb][kk] = make_uint4(bf16_bits(u0[0]) | (bf16_bits(u0[1]) << 16),
                                bf16_bits(u0[2]) | (bf16_bits(u0[3]) << 16),
                                bf16_bits(u1[0]) | (bf16_bits(u1[1]) << 16),
                                bf16_bits(u1[2]) | (bf16_bits(u1[3]) << 16));
      }
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + l16;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 va = lvt[buf][(d * TK + 32 * kk + 8 * g4) / 8];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc_o[nb][db] = mfma_bf16(va, pb[nb][kk], acc_o[nb][db]);
      }
    }
  };

  gload(0);
  swrite(0);
  if (ntiles > 1) gload(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      swrite(buf ^ 1);  // last read before the previous barrier
      if (t + 2 < ntiles) gload(t + 2);
    }
    compute(t, buf);
    __syncthreads();
  }

  // ---- output: O^T / l; lane holds dims 16 db + 4 g4 + e of query l16
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float L = rows4_sum(l_run[nb]);
    const int r = q0 + wave * 32 + nb * 16 + l16;
    if (r >= q0 + nq) continue;
    const int pz = r >> 2, hh = r & 3;
    bf16_t* dst = (bf16_t*)a.out + (((size_t)i * a.Kp + pz) * a.Hq + hk * G + hh) * D;
    const float inv = 1.f / L;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t lo = bf16_bits(acc_o[nb][db][0] * inv) | (bf16_bits(acc_o[nb][db][1] * inv) << 16);
      const uint32_t hi = bf16_bits(acc_o[nb][db][2] * inv) | (bf16_bits(acc_o[nb][db][3] * inv) << 16);
      *(uint2*)(dst + 16 * db + 4 * g4) = make_uint2(lo, hi);
    }
    if (g4 == 0)
      a.lse[((size_t)i * a.Kp + pz) * a.Hq + hk * G + hh] = (m_run[nb] + __log2f(L)) * 0.6931471805599453f;
  }
}

// ---- synthetic fill --------------------------------------------------------------

template <typename T, int D>
__global__ void __launch_bounds__(512) fill_kernel(FillArgs a) {
  const DevPool& P = a.P;
  const int r = blockIdx.x, l = blockIdx.y;
  const int32_t* hdr = a.desc + 4 * l;
  const int pers_off = hdr[0], npers = hdr[1], open_off = hdr[2], nopen = hdr[3];
  const int q = a.quota[l], Kp = a.pause[l];
  const int pers_rows = a.compress ? a.prompt_len + a.nb * q : a.prompt_len + a.G;
  const int open_rows = a.compress ? a.G - a.nb * P.C : 0;
  if (r == 0) {
    int32_t* tab = ptab_of(P, a.slot, l);
    for (int t = threadIdx.x; t < npers; t += blockDim.x) tab[t] = a.desc[pers_off + t];
    for (int t = threadIdx.x; t < nopen; t += blockDim.x) tab[P.max_pers + t] = a.desc[open_off + t];
    if (threadIdx.x == 0) {
      int32_t* meta = P.meta + (a.slot * P.L + l) * 4;
      meta[0] = pers_rows;
      meta[1] = open_rows;
      meta[2] = a.prompt_len + a.G - 1;
    }
  }
  if (r >= pers_rows + open_rows) return;
  int kind, ia, ib, pos, page, srow;
  if (r < a.prompt_len) {
    kind = 0; ia = r; ib = 0; pos = r;
  } else if (r < pers_rows) {
    const int c = r - a.prompt_len;
    if (a.compress) {
      kind = 2; ia = c / q; ib = c % q;
      int nbits = 0;
      while ((1 << nbits) < Kp) ++nbits;
      pos = a.prompt_len + ia * P.C + bitrev_dev(ib, nbits) * (P.C / Kp);
    } else {
      kind = 1; ia = c; ib = 0; pos = r;
    }
  } else {
    kind = 1; ia = a.nb * P.C + (r - pers_rows); ib = 0; pos = a.prompt_len + ia;
  }
  if (r < pers_rows) {
    page = a.desc[pers_off + r / P.pr];
    srow = r % P.pr;
  } else {
    page = a.desc[open_off + (r - pers_rows) / P.pr];
    srow = (r - pers_rows) % P.pr;
  }
  // generate the raw row (stored type) into LDS, then rotate the key
  __shared__ float kraw[1024 * 2];  // up to Hkv*D = 1024 elements
  const int n = P.Hkv * D;
  for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
    const int hh = t / (D / 2), e = t % (D / 2);
    double z0, z1;
    synth_pair(synth_row_key(a.seed, l, kind, ia, ib, 0, hh), e, &z0, &z1);
    kraw[hh * D + 2 * e] = to_f32(from_f32<T>((float)z0));
    kraw[hh * D + 2 * e + 1] = to_f32(from_f32<T>((float)z1));
    synth_pair(synth_row_key(a.seed, l, kind, ia, ib, 1, hh), e, &z0, &z1);
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.vpool)[o + 2 * e] = from_f32<T>((float)z0);
    ((T*)P.vpool)[o + 2 * e + 1] = from_f32<T>((float)z1);
  }
  __syncthreads();
  const float2* rope = P.rope + (size_t)pos * (D / 2);
  for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const float x1 = kraw[hh * D + j], x2 = kraw[hh * D + j + D / 2];
    const float2 cs = rope[j];
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.kpool)[o + j] = from_f32<T>(x1 * cs.x - x2 * cs.y);
    ((T*)P.kpool)[o + j + D / 2] = from_f32<T>(x2 * cs.x + x1 * cs.y);
  }
  if (threadIdx.x == 0) P.pos[(size_t)page * P.pr + srow] = pos;
}

// ---- inspection ------------------------------------------------------------------

template <typename T, int D>
__global__ void read_rows_kernel(ReadArgs a) {
  const DevPool& P = a.P;
  const int rr = blockIdx.x, r = a.row0 + rr;
  const int32_t* meta = meta_of(P, a.slot, a.layer);
  const int32_t* tab = ptab_of(P, a.slot, a.layer);
  const int n_pers = meta[0];
  int page, srow;
  if (r < n_pers) {
    page = tab[r / P.pr];
    srow = r % P.pr;
  } else {
    page = tab[P.max_pers + (r - n_pers) / P.pr];
    srow = (r - n_pers) % P.pr;
  }
  for (int t = threadIdx.x; t < P.Hkv * D; t += blockDim.x) {
    const int hh = t / D, d = t % D;
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D + d;
    ((T*)a.k_out)[(size_t)rr * P.Hkv * D + t] = ((const T*)P.kpool)[o];
    ((T*)a.v_out)[(size_t)rr * P.Hkv * D + t] = ((const T*)P.vpool)[o];
  }
}

__global__ void export_kernel(ExportArgs a) {
  const DevPool& P = a.P;
  const int32_t* meta = meta_of(P, a.slot, a.layer);
  const int32_t* tab = ptab_of(P, a.slot, a.layer);
  const int n_pers = meta[0], n_open = meta[1];
  const int npp = (n_pers + P.pr - 1) / P.pr, nop = (n_open + P.pr - 1) / P.pr;
  if (threadIdx.x == 0) {
    a.dst[0] = n_pers;
    a.dst[1] = n_open;
    a.dst[2] = meta[2];
    a.dst[3] = npp + nop;
  }
  for (int t = threadIdx.x; t < npp; t += blockDim.x) a.dst[4 + t] = tab[t];
  for (int t = threadIdx.x; t < nop; t += blockDim.x) a.dst[4 + npp + t] = tab[P.max_pers + t];
  int32_t* posd = a.dst + 4 + npp + nop;
  for (int r = threadIdx.x; r < n_pers + n_open; r += blockDim.x) {
    int page, srow;
    if (r < n_pers) {
      page = tab[r / P.pr];
      srow = r % P.pr;
    } else {
      page = tab[P.max_pers + (r - n_pers) / P.pr];
      srow = (r - n_pers) % P.pr;
    }
    posd[r] = P.pos[(size_t)page * P.pr + srow];
  }
}

// ---- dispatch ----------------------------------------------------------------------

template <template <typename, int> class K>
struct Nop {};

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

static int threads_for(int Hkv, int D) {
  int t = Hkv * (D / 2);
  t = t < 64 ? 64 : t;
  return t > 1024 ? 1024 : t;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int th = threads_for(a.P.Hkv, a.P.D);
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((append_kernel<T, DD>), dim3(a.n), dim3(th), 0, s, a));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t decode_g(const DecodeArgs& a, int32_t total, hipStream_t s) {
  const dim3 grid(total, a.P.Hkv);
  switch (a.G) {
#define ABK_G(GG)                                                                  \
  case GG:                                                                         \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), grid, dim3(256), 0, s, a); \
    if (total > a.n)                                                               \
      hipLaunchKernelGGL((decode_merge_kernel<T, D, GG>), dim3(a.n, a.P.Hkv),      \
                         dim3(GG * D < 1024 ? GG * D : 1024), 0, s, a);            \
    break;
    ABK_G(1) ABK_G(2) ABK_G(4) ABK_G(8)
#undef ABK_G
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int GG>
static void decode_bf16_d128(const DecodeArgs& a, int32_t total, hipStream_t s) {
  hipLaunchKernelGGL((decode_bf16_d128_kernel<GG>), dim3(total, a.P.Hkv), dim3(256), 0, s, a);
  if (total > a.n)
    hipLaunchKernelGGL((decode_merge_kernel<bf16_t, 128, GG>), dim3(a.n, a.P.Hkv),
                       dim3(GG * 128 < 1024 ? GG * 128 : 1024), 0, s, a);
}

hipError_t launch_decode(const DecodeArgs& a, int32_t total_work, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
#ifndef ABK_DECODE_GENERIC_ONLY
  if (a.P.dtype == 1 && a.P.D == 128 && a.G == 4 && (a.P.pr == 32 || a.P.pr == 64)) {
    const dim3 grid(total_work, a.P.Hkv);
    if (a.P.pr == 64)
      hipLaunchKernelGGL((decode_bf16_d128_g4_kernel<2>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_bf16_d128_g4_kernel<1>), grid, dim3(256), 0, s, a);
    if (total_work > a.n)
      hipLaunchKernelGGL((decode_merge_kernel<bf16_t, 128, 4>), dim3(a.n, a.P.Hkv), dim3(512), 0,
                         s, a);
    return hipGetLastError();
  }
  if (a.P.dtype == 1 && a.P.D == 128) {
    switch (a.G) {
      case 1: decode_bf16_d128<1>(a, total_work, s); break;
      case 2: decode_bf16_d128<2>(a, total_work, s); break;
      case 4: decode_bf16_d128<4>(a, total_work, s); break;
      case 8: decode_bf16_d128<8>(a, total_work, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
#endif
  ABK_DISPATCH_TD(a.P.dtype, a.P.D, return decode_g<T, DD>(a, total_work, s));
  return hipSuccess;
}

hipError_t launch_free(const FreeArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(free_kernel, dim3(a.n), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prompt(const PromptArgs& a, hipStream_t s) {
  const int th = threads_for(a.P.Hkv, a.P.D);
  const int rows = a.prompt_len > 0 ? a.prompt_len : 1;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((prompt_kernel<T, DD>), dim3(rows), dim3(th), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int th = threads_for(a.P.Hkv, a.P.D);
  const bool mfma = a.P.dtype == 1 && a.P.D == 128 && a.G == 4 && a.P.pr == 64;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D, {
    hipLaunchKernelGGL((pause_rope_scatter_kernel<T, DD>), dim3(a.Kp, a.n), dim3(th), 0, s, a);
    if (!mfma)
      hipLaunchKernelGGL((compress_attn_simt_kernel<T, DD>), dim3(a.Kp, a.Hq, a.n), dim3(64), 0,
                         s, a);
  });
  if (mfma) {
    // tiles of one (sequence, KV head) pair share blockIdx.x mod 8 (one XCD)
    const int ntq = (4 * a.Kp + 127) / 128;
    const int npair = a.n * a.P.Hkv;
    const int nwg = ((npair + 7) / 8) * 8 * ntq;
    hipLaunchKernelGGL(compress_attn_mfma_kernel, dim3(nwg), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fill(const FillArgs& a, int32_t max_rows, hipStream_t s) {
  const int rows = max_rows > 0 ? max_rows : 1;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((fill_kernel<T, DD>), dim3(rows, a.P.L), dim3(512), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_read(const ReadArgs& a, hipStream_t s) {
  if (a.nrows == 0) return hipSuccess;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((read_rows_kernel<T, DD>), dim3(a.nrows), dim3(256), 0, s, a));
  return hipGetLastError();
}

bool decode_stream_supported(const DevPool& P, int32_t G) {
  return P.dtype == 1 && P.D == 128 && G == 4 && (P.pr == 32 || P.pr == 64);
}

int32_t decode_stream_blocks_per_cu(const DevPool& P) {
  int nb = 0;
  hipError_t e = P.pr == 64
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_stream_kernel<2>, 256, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_stream_kernel<1>, 256, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

hipError_t launch_decode_stream(const StreamArgs& a, int32_t nwg, hipStream_t s) {
  if (a.n == 0 || nwg == 0) return hipSuccess;
  if (a.P.pr == 64)
    hipLaunchKernelGGL((decode_stream_kernel<2>), dim3(nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_stream_kernel<1>), dim3(nwg), dim3(256), 0, s, a);
  if (a.maxp > 1)
    hipLaunchKernelGGL(decode_stream_merge_kernel, dim3(a.n, a.P.Hkv), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_export(const ExportArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(export_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace abk
