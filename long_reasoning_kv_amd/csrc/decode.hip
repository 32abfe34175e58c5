// Decode attention of the AbridgeKV hot path (split-KV partials and their
// combine): the current token of each sequence attends to its resident rows
// (prompt, code rows of finished blocks, the open block) through the
// per-(sequence, layer) page table. See the pages on AbridgeKV (arXiv 2610.20641): the abstract and
// Fig. 1 captions (what stays resident), Fig. 2(a) (text tokens see the
// prompt, earlier code rows and their own block).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "common.h"

namespace abk {

// 16 bytes of a read-once stream (cached K/V rows in a decode step), loaded with
// the nontemporal cache policy: on this chip such streams run about 15% faster
// than under the default policy
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- split-KV decode and merge --------------------------------------------------
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

constexpr int kUnitRows = 16;      // rows of a page a wavefront reads per step
constexpr int kPrefetchUnits = 1;  // units a wavefront keeps in flight while computing one
template <typename T, int D>
struct UnitCfg {
  using R = RowCfg<T, D>;
  static constexpr int CW = R::RPL >= kUnitRows ? 1 : kUnitRows / R::RPL;  // loads/lane
  static constexpr int RW = CW * R::RPL;                                            // rows/unit
};


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
    const double2* rope = P.rope + (size_t)qpos * H + (d0 % H);
    double2 cs[EPL];
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
      for (int e = 0; e < EPL; ++e)
        qv[g][e] = qs * round_to<T>(sgn < 0.f ? rot_first(x[e], xp[e], cs[e]) : rot_second(xp[e], x[e], cs[e]));
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
      kr[ch] = load_stream16(kpool + off + (size_t)r * D);
      vr[ch] = load_stream16(vpool + off + (size_t)r * D);
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
  constexpr int NB = kPrefetchUnits + 1;
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

// ---- bf16 and d = 128: the streaming kernel ------------------------------------------
//
// Same work items and output as decode_split_kernel, shaped for CDNA4's VALU:
//  - 8 lanes per row; lane c holds dims [8c, 8c+8) and [64+8c, 64+8c+8), i.e.
//    both halves of its rotate-half pairs, so each wavefront load is 8 rows x
//    128 contiguous bytes;
//  - q.k on v_dot2c_f32_bf16: the rotated query, rounded once to bf16 and then
//    scaled, is split into bf16 hi + lo parts (|q - hi - lo| <= 2^-16 |q|), so
//    the scale costs no precision; keys are used as stored;
//  - 3 DPP steps finish a row's dot product; 2 rows x G heads per lane per
//    16-row unit need exp2, not 4 x G;
//  - the unit's base address is wavefront-uniform, lane offsets are fixed, and
//    only partial units clamp rows.




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
    const double2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
    double2 cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = rope[e];
    const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + g) * D;
      float xa[8], xb[8], y[16];
      unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
      unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = qs * round_to<bf16_t>(rot_first(xa[e], xb[e], cs[e]));
        y[8 + e] = qs * round_to<bf16_t>(rot_second(xa[e], xb[e], cs[e]));
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
        kr[2 * rg] = load_stream16(kb + o2);
        kr[2 * rg + 1] = load_stream16(kb + o2 + 128);
        vr[2 * rg] = load_stream16(vb + o2);
        vr[2 * rg + 1] = load_stream16(vb + o2 + 128);
      }
    } else {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        int r = rg * 8 + r8;
        r = r < nval ? r : (nval > 0 ? nval - 1 : 0);
        const uint32_t o2 = (uint32_t)(r * D + 8 * c8) * 2;
        kr[2 * rg] = load_stream16(kb + o2);
        kr[2 * rg + 1] = load_stream16(kb + o2 + 128);
        vr[2 * rg] = load_stream16(vb + o2);
        vr[2 * rg + 1] = load_stream16(vb + o2 + 128);
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

// ---- bf16, d = 128, four query heads per KV head: LDS-staged streaming -----------
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
    const double2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
    double2 cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = rope[e];
    const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + 2 * hp + j2) * D;
      float xa[8], xb[8], y[16];
      unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
      unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = qs * round_to<bf16_t>(rot_first(xa[e], xb[e], cs[e]));
        y[8 + e] = qs * round_to<bf16_t>(rot_second(xa[e], xb[e], cs[e]));
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
  auto gload = [&](int u, bool fresh, uint4* k0, uint4* v0, uint4* k1, uint4* v1) __attribute__((always_inline)) {
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
    if (fresh) {
      *k0 = load_stream16(kb + r0 * RB);
      *v0 = load_stream16(vb + r0 * RB);
      *k1 = load_stream16(kb + r1 * RB);
      *v1 = load_stream16(vb + r1 * RB);
    } else {  // a repeat of the last unit: the default policy finds it in L2
      *k0 = *(const uint4*)(kb + r0 * RB);
      *v0 = *(const uint4*)(vb + r0 * RB);
      *k1 = *(const uint4*)(kb + r1 * RB);
      *v1 = *(const uint4*)(vb + r1 * RB);
    }
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
  // (indices past the end re-read the last unit, under the default cache policy
  // so that it comes from L2), so the
  // waits before each store can count exactly the newer stage's loads.
  const int ulast = nunits - 1;
  gload(0, true, &ak0, &av0, &ak1, &av1);
  swrite(0, ak0, av0, ak1, av1);
  gload(min(1, ulast), 1 <= ulast, &ak0, &av0, &ak1, &av1);
  gload(min(2, ulast), 2 <= ulast, &bk0, &bv0, &bk1, &bv1);
  __syncthreads();
  auto step = [&](int u, uint4& k0, uint4& v0, uint4& k1, uint4& v1) __attribute__((always_inline)) {
    const int b = u & 1;
    swrite(b ^ 1, k0, v0, k1, v1);  // its buffer was last read before the previous barrier
    gload(min(u + 3, ulast), u + 3 <= ulast, &k0, &v0, &k1, &v1);
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

// ---- persistent stream-K form of the kernel above ----------------------------------
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
      const double2* rope = P.rope + (size_t)qpos * (D / 2) + 8 * c8;
      double2 cs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = rope[e];
      const float qs = 1.4426950408889634f / sqrtf((float)D);
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + 2 * hp + j2) * D;
        float xa[8], xb[8], y[16];
        unpack16(*(const uint4*)(qrow + 8 * c8), xa, bf16_t());
        unpack16(*(const uint4*)(qrow + 64 + 8 * c8), xb, bf16_t());
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = qs * round_to<bf16_t>(rot_first(xa[e], xb[e], cs[e]));
          y[8 + e] = qs * round_to<bf16_t>(rot_second(xa[e], xb[e], cs[e]));
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
    auto gload = [&](int u, bool fresh, uint4* k0, uint4* v0, uint4* k1, uint4* v1) __attribute__((always_inline)) {
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
      if (fresh) {
        *k0 = load_stream16(kb + r0 * RB);
        *v0 = load_stream16(vb + r0 * RB);
        *k1 = load_stream16(kb + r1 * RB);
        *v1 = load_stream16(vb + r1 * RB);
      } else {  // a repeat of the last unit: the default policy finds it in L2
        *k0 = *(const uint4*)(kb + r0 * RB);
        *v0 = *(const uint4*)(vb + r0 * RB);
        *k1 = *(const uint4*)(kb + r1 * RB);
        *v1 = *(const uint4*)(vb + r1 * RB);
      }
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
    gload(0, true, &ak0, &av0, &ak1, &av1);
    swrite(0, ak0, av0, ak1, av1);
    gload(min(1, ulast), 1 <= ulast, &ak0, &av0, &ak1, &av1);
    gload(min(2, ulast), 2 <= ulast, &bk0, &bv0, &bk1, &bv1);
    __syncthreads();
    auto step = [&](int u, uint4& k0, uint4& v0, uint4& k1, uint4& v1) __attribute__((always_inline)) {
      const int b = u & 1;
      swrite(b ^ 1, k0, v0, k1, v1);
      gload(min(u + 3, ulast), u + 3 <= ulast, &k0, &v0, &k1, &v1);
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

// Merge the partials of (sequence i, KV head h) written by stream-K workers
// wa..wb (workgroups of decode_stream_kernel, wavefronts of decode_mfma_kernel).
// Thread (g, d) fetches, for sixteen partials at a time, their maximum, sum and
// its own output element in one round of independent loads, then combines
// them online; with up to sixteen partials the merge is one memory round trip.
__global__ void __launch_bounds__(512) decode_stream_merge_kernel(StreamArgs a) {
  constexpr int D = 128, G = 4, K = 16;
  const int i = blockIdx.x, h = blockIdx.y;
  const int Hkv = a.P.Hkv, Hq = Hkv * G;
  const int units = (a.useg[i + 1] - a.useg[i]) / Hkv;
  const int segS = a.useg[i] + h * units;
  const int wa = segS / a.T, wb = (segS + units - 1) / a.T;
  // a fused call adds the current token's partial after the tiles' ones
  const int ns = wb - wa + 1 + a.fused;
  if (a.fused && h == 0 && threadIdx.x == 0) {
    // the fused append's row is now in place: advance the counts and position
    int32_t* meta = a.P.meta + (a.slot[i] * a.P.L + a.layer) * 4;
    meta[a.compress ? 1 : 0] += 1;
    meta[2] += 1;
  }
  if (ns == 1) return;
  const float* base = a.part + ((size_t)i * Hkv + h) * (a.maxp + a.fused) * G * (D + 2);
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    // a wavefront's 64 threads share the query head (D = 128), so its partials'
    // maxima and sums are wavefront-uniform: scalar loads, one per wavefront
    const int g = sgpr(t / D), d = t % D;
    float M = -INFINITY, Ls = 0.f, O = 0.f;
    for (int s0 = 0; s0 < ns; s0 += K) {
      float mv[K], lv[K], ov[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int off = (min(s0 + k, ns - 1) * G + g) * (D + 2);
        // (read-only here: written by the decode launch before this one)
        const __attribute__((address_space(4))) float* pc = (const __attribute__((address_space(4))) float*)(base + off);
        mv[k] = pc[D];
        lv[k] = pc[D + 1];
        ov[k] = base[off + d];
      }
      float cm = M;
#pragma unroll
      for (int k = 0; k < K; ++k) cm = s0 + k < ns ? fmaxf(cm, mv[k]) : cm;
      const float r = fast_exp2(M - cm);  // first round: M = -inf, r = 0
      Ls *= r;
      O *= r;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float wgt = s0 + k < ns ? fast_exp2(mv[k] - cm) : 0.f;
        Ls += wgt * lv[k];
        O += wgt * ov[k];
      }
      M = cm;
    }
    ((bf16_t*)a.out)[((size_t)i * Hq + h * G + g) * D + d] = from_f32<bf16_t>(O / Ls);
    if (d == 0) a.lse[(size_t)i * Hq + h * G + g] = (M + __log2f(Ls)) * 0.6931471805599453f;
  }
}

// ---- decode on bf16 MFMA: wavefront-level stream-K over 32-row tiles -------------
//
// Every wavefront is an independent stream over an equal run of the flattened
// (sequence, KV head, 32-row tile) work, so no barrier is needed anywhere. A
// tile's 32 K rows and 32 V rows go straight from HBM into the wavefront's own
// 16 KB of LDS (global_load_lds_dwordx4). The wavefront first reads the whole
// tile into registers (K as MFMA A operands, V through ds_read_b64_tr_b16 as
// V^T operands), then starts loading the next tile into the same LDS and
// computes while it is in flight:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, two M-blocks of 16 keys; B = the
//                 four rotated query heads of the KV head (bf16, rounded once
//                 like stored keys) in columns 0..3; the softmax scale is
//                 applied to the fp32 scores; M-block mb row m is key 8(m/4) + 4mb + m%4,
//                 so lane l ends up with the 8 consecutive keys 8(l/16)+0..7 of
//                 head l%16;
//   online softmax per head column (lane-local, then permlane swaps); the
//                 running maximum only moves when a tile exceeds it by 2^8;
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16; B = P^T straight from the S^T
//                 registers, A = V^T (dims 16db + l%16, keys 8(l/16) + 0..7).
// K rows in LDS have their 16-byte chunks XOR-swizzled by bits 0,1,3,4 of the
// row and V rows by 2*(bits 0,1,3), so both operand reads touch every bank
// evenly. A segment inside one wavefront's run writes out and lse; other pieces
// write partials for decode_stream_merge_kernel (index = wavefront - first).

__device__ __forceinline__ int dm_vswz(int row) { return 2 * ((row & 3) | ((row >> 1) & 4)); }

__global__ void __launch_bounds__(256, 2) decode_mfma_kernel(StreamArgs a) {
  constexpr int D = 128, G = 4, TK = 32, RB = D * 2, PR = 64;
  constexpr int WCH = TK * RB / 16;  // 16-byte chunks of one tile (K or V) = 512
  __shared__ uint4 lk[4 * WCH], lv[4 * WCH];  // one 8 KB K slice and V slice per wavefront
  const DevPool& P = a.P;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int w = blockIdx.x * 4 + wave;  // wavefront id in the stream-K order
  const int Hq = P.Hkv * G;
  const int F0 = w * a.T;
  const int Fend = min(a.U, F0 + a.T);
  const char* kpool = (const char*)P.kpool;
  const char* vpool = (const char*)P.vpool;
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
  typedef const __attribute__((address_space(4))) int32_t* cptr;

  // ---- cursor over (sequence, KV head, tile); all fields wave-uniform
  struct Cur {
    int i, h, lu, units, ptiles, n_pers, n_open, slot;
  };
  auto load_seq = [&](Cur& c) __attribute__((always_inline)) {
    c.units = (a.useg[c.i + 1] - a.useg[c.i]) / P.Hkv;
    c.slot = a.slot[c.i];
    cptr meta = (cptr)meta_of(P, c.slot, a.layer);
    c.n_pers = meta[0];
    c.n_open = meta[1];
    c.ptiles = (c.n_pers + TK - 1) / TK;
  };
  auto cursor_at = [&](int F) __attribute__((always_inline)) {
    Cur c;
    // the sequence whose tiles hold F: useg[i] <= F < useg[i + 1] (binary search)
    int lo = 0, hi = a.n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.useg[mid] <= F) lo = mid;
      else hi = mid - 1;
    }
    c.i = lo;
    load_seq(c);
    const int rel = F - a.useg[c.i];
    c.h = rel / c.units;
    c.lu = rel % c.units;
    return c;
  };
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    if (++c.lu == c.units) {
      c.lu = 0;
      if (++c.h == P.Hkv) {
        c.h = 0;
        ++c.i;
        if (c.i < a.n) load_seq(c);
      }
    }
  };
  // byte offset of the tile's first row in the pools, and its valid rows. The
  // persistent candidate page is read whether or not the tile is persistent:
  // its address does not depend on the row counts, so the two reads overlap.
  auto locate = [&](const Cur& c, size_t* off, int* nval) __attribute__((always_inline)) {
    cptr tab = (cptr)ptab_of(P, c.slot, a.layer);
    const int ppage = tab[min(c.lu >> 1, P.max_pers - 1)];
    int page, r0;
    if (c.lu < c.ptiles) {
      page = ppage;
      r0 = (c.lu & 1) * TK;
      *nval = min(TK, c.n_pers - c.lu * TK);
    } else {
      const int j = c.lu - c.ptiles;
      *nval = min(TK, c.n_open - j * TK);
      // a fused call's only tile of a sequence with no rows yet is empty
      page = *nval > 0 ? tab[P.max_pers + (j >> 1)] : 0;
      r0 = (j & 1) * TK;
    }
    *off = (((size_t)page * P.Hkv + c.h) * PR + r0) * RB;
  };

  // ---- loads: load j of the wavefront fills chunks 64j.. of its slice, i.e.
  // row 4j + lane/16 at swizzled position lane%16; rows past the valid count
  // repeat the last valid row. A step reads each cached row once, so the loads
  // carry the nontemporal policy (nt): on this chip a read-once stream then runs
  // about 15% faster than under the default policy
  constexpr int kNT = 2;
  const int dr = lane >> 4;
  auto issue = [&](const Cur& c) __attribute__((always_inline)) {
    size_t off;
    int nval;
    locate(c, &off, &nval);
    if (nval <= 0) return;  // empty tile: nothing to load
#pragma unroll
    for (int j = 0; j < TK / 4; ++j) {
      const int row = 4 * j + dr;
      const int rc = min(row, nval - 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)(kpool + off + rc * RB + 16 * ((lane & 15) ^ kswz(row))),
          (__attribute__((address_space(3))) void*)(lk + wave * WCH + 64 * j), 16, 0, kNT);
      __builtin_amdgcn_global_load_lds(
          (const void*)(vpool + off + rc * RB + 16 * ((lane & 15) ^ dm_vswz(row))),
          (__attribute__((address_space(3))) void*)(lv + wave * WCH + 64 * j), 16, 0, kNT);
    }
  };

  // ---- per-segment state
  uint4 qh[4];  // B operand of S^T: bf16 rotated query, head l16 (< 4), dims 32ks + 8g4 + 0..7
  f32x4_t acc[8];      // O^T: dims 16db + 4g4 + i of head l16
  float m_run = -1e30f, l_run = 0.f;
  auto start_segment = [&](const Cur& c) __attribute__((always_inline)) {
    cptr meta = (cptr)meta_of(P, c.slot, a.layer);
    const int qpos = meta[2] + (a.fused ? 1 : 0);  // fused: the token appended here
    const int hh = l16 < G ? l16 : 0;
    const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)c.i * Hq + c.h * G + hh) * D;
    const double2* rope = P.rope + (size_t)qpos * (D / 2);
    float x[4][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) unpack16(*(const uint4*)(qrow + 32 * ks + 8 * g4), x[ks], bf16_t());
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      double y0[8], y1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double2 cs = rope[32 * ks + 8 * g4 + j];
        y0[j] = l16 < G ? rot_first(x[ks][j], x[ks + 2][j], cs) : 0.0;
        y1[j] = l16 < G ? rot_second(x[ks][j], x[ks + 2][j], cs) : 0.0;
      }
      qh[ks] = make_uint4(pack_bf16x2_f64(y0[0], y0[1]), pack_bf16x2_f64(y0[2], y0[3]),
                          pack_bf16x2_f64(y0[4], y0[5]), pack_bf16x2_f64(y0[6], y0[7]));
      qh[ks + 2] = make_uint4(pack_bf16x2_f64(y1[0], y1[1]), pack_bf16x2_f64(y1[2], y1[3]),
                              pack_bf16x2_f64(y1[4], y1[5]), pack_bf16x2_f64(y1[6], y1[7]));
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -1e30f;
    l_run = 0.f;
  };
  auto end_segment = [&](const Cur& c) __attribute__((always_inline)) {
    const float L = rows4_sum(l_run);
    const int segS = a.useg[c.i] + c.h * c.units;
    const int wa = segS / a.T, wb = (segS + c.units - 1) / a.T;
    if (l16 < G) {
      const int hq = c.h * G + l16;
      if (wa == wb && !a.fused) {
        const float inv = 1.f / L;
        bf16_t* dst = (bf16_t*)a.out + ((size_t)c.i * Hq + hq) * D;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *(uint2*)(dst + 16 * db + 4 * g4) =
              make_uint2(pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv),
                         pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv));
        if (g4 == 0) a.lse[(size_t)c.i * Hq + hq] = (m_run + __log2f(L)) * 0.6931471805599453f;
      } else {
        float* pp = a.part + ((((size_t)c.i * P.Hkv + c.h) * (a.maxp + a.fused) + (w - wa)) * G + l16) * (D + 2);
#pragma unroll
        for (int db = 0; db < 8; ++db) *(f32x4_t*)(pp + 16 * db + 4 * g4) = acc[db];
        if (g4 == 0) {
          pp[D] = m_run;
          pp[D + 1] = L;
        }
      }
    }
  };

  // ---- fused append: the current token's row of (sequence i, KV head h), one
  // per wavefront spread over the grid, done while the first tile loads. Lane l
  // rotates the dimension pair (l, l + 64) of the key in fp64 (rounded once to
  // bf16, like every stored key), writes the K and V row, and scores the key
  // against the four rotated queries of the head; the result goes to the
  // merge as one more partial of the head (maximum = score, sum = 1, O = v)
  auto fused_row = [&](int x) __attribute__((always_inline)) {
    const int i = x / P.Hkv, h = x % P.Hkv;
    const int slot = a.slot[i];
    cptr meta = (cptr)meta_of(P, slot, a.layer);
    const int n_pers = meta[0], n_open = meta[1], pos = meta[2] + 1;
    const double2 cs = P.rope[(size_t)pos * (D / 2) + lane];
    const size_t kvo = ((size_t)i * P.Hkv + h) * D;
    const bf16_t* kin = (const bf16_t*)a.k + kvo;
    const bf16_t* vin = (const bf16_t*)a.v + kvo;
    const double k1 = to_f32(kin[lane]), k2 = to_f32(kin[lane + 64]);
    const bf16_t kr1 = from_f64<bf16_t>(rot_first(k1, k2, cs));
    const bf16_t kr2 = from_f64<bf16_t>(rot_second(k1, k2, cs));
    const bf16_t v1 = vin[lane], v2 = vin[lane + 64];
    // the row: next row of the open block (persistent list in full-KV mode)
    const int r = a.compress ? n_open : n_pers;
    int32_t* tab = ptab_of(P, slot, a.layer) + (a.compress ? P.max_pers : 0);
    const int pidx = r / PR, srow = r % PR;
    const int page = srow == 0 ? a.new_page[i] : ((cptr)tab)[pidx];
    const size_t o = (((size_t)page * P.Hkv + h) * PR + srow) * D;
    bf16_t* kd = (bf16_t*)P.kpool + o;
    bf16_t* vd = (bf16_t*)P.vpool + o;
    kd[lane] = kr1;
    kd[lane + 64] = kr2;
    vd[lane] = v1;
    vd[lane + 64] = v2;
    if (h == 0 && lane == 0) {
      P.pos[(size_t)page * PR + srow] = pos;
      if (srow == 0) tab[pidx] = page;
    }
    const float kf1 = to_f32(kr1), kf2 = to_f32(kr2);
    const int units = (a.useg[i + 1] - a.useg[i]) / P.Hkv;
    const int segS = a.useg[i] + h * units;
    const int ns = (segS + units - 1) / a.T - segS / a.T + 1;  // the tiles' partials
    float* pp = a.part + (((size_t)i * P.Hkv + h) * (a.maxp + 1) + ns) * G * (D + 2);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bf16_t* qin = (const bf16_t*)a.q + ((size_t)i * Hq + h * G + g) * D;
      const double q1 = to_f32(qin[lane]), q2 = to_f32(qin[lane + 64]);
      const float sc = group_sum<64>(round_to<bf16_t>(rot_first(q1, q2, cs)) * kf1 +
                                     round_to<bf16_t>(rot_second(q1, q2, cs)) * kf2);
      float* pg = pp + g * (D + 2);
      pg[lane] = to_f32(v1);
      pg[lane + 64] = to_f32(v2);
      if (lane == 0) {
        pg[D] = sc * qs;
        pg[D + 1] = 1.f;
      }
    }
  };

  const bool has_tiles = F0 < Fend;
  Cur cc, ci;  // tile being computed, tile being loaded
  if (has_tiles) {
    cc = cursor_at(F0);
    ci = cc;
    issue(ci);
  }
  if (a.fused) {
    // rows x at wavefronts x * (waves / rows) when there are fewer rows than
    // wavefronts, else rows w, w + waves, ...
    const int nit = a.n * P.Hkv, nw = gridDim.x * 4;
    const int st = nit <= nw ? nw / nit : 1;
    for (int x = w % st == 0 ? w / st : nit; x < nit; x += nw) fused_row(x);
  }
  if (!has_tiles) return;
  int last_i = -1, last_h = -1;
  const int vrow0 = 8 * g4 + (l16 >> 2);  // V^T operand rows (+4 for the second half)
  for (int t = F0; t < Fend; ++t) {
    if (cc.i != last_i || cc.h != last_h) {  // query loads join the tile's wait
      start_segment(cc);
      last_i = cc.i;
      last_h = cc.h;
    }
    size_t off;
    int nval;
    locate(cc, &off, &nval);
    // ---- the whole tile from LDS into registers, once its load has landed. The
    // wait is explicit: the load is issued on a conditional path, which the
    // compiler's own tracking of loads into LDS does not follow
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    uint4 ka[2][4], va[8];
    if (nval > 0) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int kr = 8 * (l16 >> 2) + 4 * mb + (l16 & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[mb][ks] = lk[wave * WCH + kr * 16 + ((4 * ks + g4) ^ kswz(kr))];
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint32_t wv[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = vrow0 + 4 * hh;
        const int chunk = (2 * db + ((l16 & 3) >> 1)) ^ dm_vswz(row);
        const int boff = (wave * WCH + row * 16 + chunk) * 16 + 8 * (l16 & 1);
        const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)((const char*)lv + boff));
        const uint2 u = __builtin_bit_cast(uint2, r);
        wv[2 * hh] = u.x;
        wv[2 * hh + 1] = u.y;
      }
      va[db] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    }
    // ---- the next tile into the same LDS (once every read above has landed).
    // The last tile of the run issues nothing: a repeated tile would come from
    // HBM again, since the nontemporal loads do not keep it in L2
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (t + 1 < Fend) {
      advance(ci);
      issue(ci);
    }
    // ---- S^T, softmax, O^T
    if (nval > 0) {
    f32x4_t sc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[mb] = mfma_bf16(ka[mb][ks], qh[ks], sc[mb]);
    }
    if (nval < TK) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[mb][e] = 8 * g4 + 4 * mb + e < nval ? sc[mb][e] : -INFINITY;
    }
    // scores in log2 units: q.k * log2(e)/sqrt(d), folded into the exponent below
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = rows4_max(mx) * qs;
    const bool up = mx > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float mn = up ? mx : m_run;
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] *= alpha;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = fast_exp2(fmaf(sc[0][e], qs, -m_run));
      p[4 + e] = fast_exp2(fmaf(sc[1][e], qs, -m_run));
    }
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    const uint4 pb = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = mfma_bf16(va[db], pb, acc[db]);
    }
    if (cc.lu == cc.units - 1 || t == Fend - 1) end_segment(cc);
    advance(cc);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may land in LDS after the wavefront ends
}

// ---- launchers ---------------------------------------------------------------------

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
  ABK_DISPATCH_TD(a.P.dtype, a.P.D, return decode_g<T, DD>(a, total_work, s));
  return hipSuccess;
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

bool decode_mfma_supported(const DevPool& P, int32_t G) {
  return P.dtype == 1 && P.D == 128 && G == 4 && P.pr == 64;
}

int32_t decode_mfma_waves_per_cu() {
  int nb = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_mfma_kernel, 256, 0);
  return 4 * ((e == hipSuccess && nb > 0) ? nb : 1);
}

hipError_t launch_decode_mfma(const StreamArgs& a, int32_t nwaves, hipStream_t s) {
  if (a.n == 0 || nwaves == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3((nwaves + 3) / 4), dim3(256), 0, s, a);
  if (a.maxp > 1 || a.fused)
    hipLaunchKernelGGL(decode_stream_merge_kernel, dim3(a.n, a.P.Hkv), dim3(512), 0, s, a);
  return hipGetLastError();
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

// ---- the allocation-free decode's workspace ----------------------------------------
// Split partials of abk_decode_attention_noalloc, for callers that cannot
// allocate device memory. Each GPU holds its own copy for the life of the
// process. On the host, the array's name is only a stand-in for it: the
// address that kernels take comes from hipGetSymbolAddress on each device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
}  // namespace abk
