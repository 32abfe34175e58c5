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

// ---- a2: split-KV decode partials -----------------------------------------------
//
// Work item (sequence i, split s) x KV head h: 4 wavefronts take the split's
// pages round-robin. A page is read 16 bytes per lane (LPR lanes per row);
// each lane holds its slice of the G rotated queries, so one K load feeds G
// dot products that are finished by a DPP group sum. Softmax is online per
// page with a wavefront-uniform running max (log2 domain), V is accumulated
// per lane and reduced across row groups and wavefronts at the end.

template <typename T, int D, int G>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  using Cfg = RowCfg<T, D>;
  constexpr int EPL = Cfg::EPL, LPR = Cfg::LPR, RPL = Cfg::RPL, MAXCH = Cfg::MAXCH;
  const DevPool& P = a.P;
  const int w = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPR, grp = lane / LPR;

  int lo = 0, hi = a.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.prefix[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo, s = w - a.prefix[i], nsplit = a.prefix[i + 1] - a.prefix[i];
  const int slot = a.slot[i];
  const int32_t* meta = meta_of(P, slot, a.layer);
  const int n_pers = meta[0], n_open = meta[1], qpos = meta[2];
  const int pr = P.pr;
  const int npp = (n_pers + pr - 1) / pr, nop = (n_open + pr - 1) / pr;
  const int vp0 = s * a.split_pages, vp1 = min(npp + nop, vp0 + a.split_pages);
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int Hq = P.Hkv * G;

  // rotated, pre-scaled query slice: dims c*EPL .. c*EPL+EPL-1 of heads h*G+g
  float qv[G][EPL];
  {
    const float2* rope = P.rope + (size_t)qpos * (D / 2);
    const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const T* qh = (const T*)a.q + ((size_t)i * Hq + h * G + g) * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        qv[g][e] = qs * rope_elem<D>([&](int d) { return to_f32(qh[d]); }, c * EPL + e, rope);
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
  for (int vp = vp0 + wave; vp < vp1; vp += 4) {
    int page, rows;
    if (vp < npp) {
      page = tab[vp];
      rows = (vp == npp - 1) ? n_pers - vp * pr : pr;
    } else {
      const int j = vp - npp;
      page = tab[P.max_pers + j];
      rows = (j == nop - 1) ? n_open - j * pr : pr;
    }
    const size_t base = ((size_t)page * P.Hkv + h) * pr * D + c * EPL;
    float sc[MAXCH][G];
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
      if (ch * RPL < rows) {
        const int r = ch * RPL + grp;
        const bool valid = r < rows;
        const int rl = valid ? r : rows - 1;
        const uint4 kw = *(const uint4*)(kpool + base + (size_t)rl * D);
        float kf[EPL];
        unpack16(kw, kf, T());
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc += qv[g][e] * kf[e];
          acc = group_sum<LPR>(acc);
          sc[ch][g] = valid ? acc : -INFINITY;
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) sc[ch][g] = -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = sc[0][g];
#pragma unroll
      for (int ch = 1; ch < MAXCH; ++ch) mx = fmaxf(mx, sc[ch][g]);
      mx = across_max<LPR>(mx);
      const float mn = fmaxf(m_run[g], mx);
      const float alpha = fast_exp2(m_run[g] - mn);
      m_run[g] = mn;
      l_run[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
    }
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
      if (ch * RPL < rows) {
        const int r = ch * RPL + grp;
        const int rl = r < rows ? r : rows - 1;
        const uint4 vw = *(const uint4*)(vpool + base + (size_t)rl * D);
        float vf[EPL];
        unpack16(vw, vf, T());
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = fast_exp2(sc[ch][g] - m_run[g]);
          l_run[g] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[g][e] += p * vf[e];
        }
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
      const float f = fast_exp2(sm_m[ww][g] - M);
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

// ---- a3: merge split partials --------------------------------------------------

template <typename T, int D, int G>
__global__ void __launch_bounds__(1024) decode_combine_kernel(DecodeArgs a) {
  const int i = blockIdx.x, h = blockIdx.y;
  const int b0 = a.prefix[i], ns = a.prefix[i + 1] - b0;
  if (ns == 1) return;
  const int Hkv = a.P.Hkv, Hq = Hkv * G;
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int g = t / D, d = t % D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
      M = fmaxf(M, a.part[(((size_t)(b0 + s) * Hkv + h) * G + g) * (D + 2) + D]);
    float Ls = 0.f, O = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float* pp = a.part + (((size_t)(b0 + s) * Hkv + h) * G + g) * (D + 2);
      const float f = fast_exp2(pp[D] - M);
      Ls += pp[D + 1] * f;
      O += pp[d] * f;
    }
    const int hq = h * G + g;
    ((T*)a.out)[((size_t)i * Hq + hq) * D + d] = from_f32<T>(O / Ls);
    if (d == 0) a.lse[(size_t)i * Hq + hq] = (M + __log2f(Ls)) * 0.6931471805599453f;
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
#define ABK_G(GG)                                                                          \
  case GG:                                                                                 \
    hipLaunchKernelGGL((decode_split_kernel<T, D, GG>), grid, dim3(256), 0, s, a);         \
    if (total > a.n)                                                                       \
      hipLaunchKernelGGL((decode_combine_kernel<T, D, GG>), dim3(a.n, a.P.Hkv),            \
                         dim3(GG * D < 1024 ? GG * D : 1024), 0, s, a);                    \
    break;
    ABK_G(1) ABK_G(2) ABK_G(4) ABK_G(8)
#undef ABK_G
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int32_t total_work, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
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
  ABK_DISPATCH_TD(a.P.dtype, a.P.D, {
    hipLaunchKernelGGL((pause_rope_scatter_kernel<T, DD>), dim3(a.Kp, a.n), dim3(th), 0, s, a);
    hipLaunchKernelGGL((compress_attn_simt_kernel<T, DD>), dim3(a.Kp, a.Hq, a.n), dim3(64), 0, s,
                       a);
  });
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

hipError_t launch_export(const ExportArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(export_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace abk
