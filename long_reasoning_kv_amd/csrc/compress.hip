// Block compression of the AbridgeKV hot path: pause queries
// and keys are rotated at their in-block bit-reversed positions (Fig. 2(b) of
// arXiv 2610.20641), attend under the block mask (Fig. 2(a)) to the prompt,
// retained code rows, the whole block and earlier pause keys, and the kept
// prefix of the pause rows becomes the layer's code rows (Fig. 1(a)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_mfma.h"
#include "common.h"

namespace abk {

// ---- pause RoPE at bit-reversed in-block positions, code-row scatter -----------


// One thread per (pause token, KV head, 16-byte group of each half row): it
// rotates the group's pairs (d, d + D/2) in fp64 and writes them, rounded once,
// to the workspace and, for a kept token, with its value to the code row.
// kpb pause tokens per workgroup.
template <typename T, int D>
__global__ void __launch_bounds__(256) pause_rope_scatter_kernel(CompressArgs a, int kpb) {
  constexpr int V = 16 / sizeof(T), NJ = D / 2 / V;
  static_assert(NJ * V * 2 == D, "a half row is a whole number of 16-byte groups");
  const DevPool& P = a.P;
  const int i = blockIdx.y;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], pers_before = rec[2], prompt = rec[3];
  const int pages_off = rec[4], npages = rec[5], first_new = rec[6], quota = rec[7];
  // the caller's sequence and first KV head of this entry
  const int ir = i / a.hsplit, H0 = (i % a.hsplit) * P.Hkv, HkvR = P.Hkv * a.hsplit;
  const int per_k = P.Hkv * NJ;
  for (int t = threadIdx.x; t < kpb * per_k; t += blockDim.x) {
    const int k = blockIdx.x * kpb + t / per_k;
    if (k >= a.Kp) break;
    const int hh = (t % per_k) / NJ, j0 = (t % NJ) * V;
    const int pos = prompt + blk * P.C + bitrev_dev(k, a.log2Kp) * (P.C / a.Kp);
    const size_t in_row = (((size_t)ir * a.Kp + k) * HkvR + H0 + hh) * D;
    const T* kin = (const T*)a.kp + in_row;
    const double2* rope = P.rope + (size_t)pos * (D / 2) + j0;
    T x1[V], x2[V], y1[V], y2[V];
    const uint4 w1 = *(const uint4*)(kin + j0), w2 = *(const uint4*)(kin + D / 2 + j0);
    __builtin_memcpy(x1, &w1, 16);
    __builtin_memcpy(x2, &w2, 16);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const double2 cs = rope[e];
      const double a1 = to_f32(x1[e]), a2 = to_f32(x2[e]);
      y1[e] = from_f64<T>(rot_first(a1, a2, cs));
      y2[e] = from_f64<T>(rot_second(a1, a2, cs));
    }
    uint4 o1, o2;
    __builtin_memcpy(&o1, y1, 16);
    __builtin_memcpy(&o2, y2, 16);
    T* kr = (T*)a.kp_rot + (((size_t)i * P.Hkv + hh) * a.Kp + k) * D;
    *(uint4*)(kr + j0) = o1;
    *(uint4*)(kr + D / 2 + j0) = o2;
    if (k < quota) {
      const int row = pers_before + k;
      const int page = a.desc[pages_off + row / P.pr - pers_before / P.pr];
      const int srow = row % P.pr;
      const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
      const T* vin = (const T*)a.vp + in_row;
      *(uint4*)((T*)P.kpool + o + j0) = o1;
      *(uint4*)((T*)P.kpool + o + D / 2 + j0) = o2;
      *(uint4*)((T*)P.vpool + o + j0) = *(const uint4*)(vin + j0);
      *(uint4*)((T*)P.vpool + o + D / 2 + j0) = *(const uint4*)(vin + D / 2 + j0);
      if (hh == 0 && j0 == 0) P.pos[(size_t)page * P.pr + srow] = pos;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int32_t* tab = ptab_of(P, slot, a.layer);
    const int first_idx = pers_before / P.pr;
    for (int j = first_new; j < npages; ++j) tab[first_idx + j] = a.desc[pages_off + j];
    P.meta[(slot * P.L + a.layer) * 4 + 0] = pers_before + quota;
  }
}

// ---- pause-token attention under the block mask (SIMT form) -----------------------
//
// One wavefront per (entry, pause j, query head of the entry). Keys: the sequence's
// resident rows at this layer (prompt, earlier code rows, the whole block)
// followed by the rotated pause keys 0..j. 64 keys per step: one lane per key
// scores it, the wavefront takes the step's max, and each lane accumulates
// its D/64 output dims over the step.

template <typename T, int D>
__global__ void __launch_bounds__(64) compress_attn_simt_kernel(CompressArgs a) {
  const DevPool& P = a.P;
  const int j = blockIdx.x, hq = blockIdx.y, i = blockIdx.z;
  const int lane = threadIdx.x;
  const int hk = hq / a.G;  // the entry's KV head
  // the caller's sequence, and the caller's index of this query head
  const int ir = i / a.hsplit, HQ = (i % a.hsplit) * P.Hkv * a.G + hq, HkvR = P.Hkv * a.hsplit;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], n_pers = rec[2], prompt = rec[3];
  const int n_ctx = n_pers + P.C;
  const int n_keys = n_ctx + j + 1;
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int pos = prompt + blk * P.C + bitrev_dev(j, a.log2Kp) * (P.C / a.Kp);

  __shared__ float qs[D];
  __shared__ float ps[64];
  {
    const double2* rope = P.rope + (size_t)pos * (D / 2);
    const T* qh = (const T*)a.qp + (((size_t)ir * a.Kp + j) * a.Hq + HQ) * D;
    const float sc = 1.4426950408889634f / sqrtf((float)D);
    for (int d = lane; d < D; d += 64)
      qs[d] = sc * round_to<T>(rope_elem<D>([&](int e) { return (double)to_f32(qh[e]); }, d, rope));
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
      *vr = (const T*)a.vp + (((size_t)ir * a.Kp + kk) * HkvR + (i % a.hsplit) * P.Hkv + hk) * D;
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
  T* out = (T*)a.out + (((size_t)ir * a.Kp + j) * a.Hq + HQ) * D;
#pragma unroll
  for (int t = 0; t < DPL; ++t) {
    const int d = lane + 64 * t;
    if (d < D) out[d] = from_f32<T>(o[t] / l);
  }
  if (lane == 0) a.lse[((size_t)ir * a.Kp + j) * a.Hq + HQ] = (m + __log2f(l)) * 0.6931471805599453f;
}

// ---- pause-token attention on bf16 MFMA (d = 128, four query heads per KV head,
// 64-row pages) ------------------------------------------------------------------
//
// Workgroup = (sequence, KV head, tile of 256 query rows); query row r is pause
// r/4, head 4h + r%4. Each of the 8 wavefronts owns 32 query rows and runs the
// per-tile math of attn_mfma.h over the 64-key tiles: the context pages
// (persistent, then open), then the pause-key tiles. Masks are applied only to
// partial and pause tiles.
//
// The tiles run on the ping-pong schedule of pingpong_attention (two groups of
// four wavefronts, one phase apart, through a ring of four LDS buffers).

__global__ void __launch_bounds__(512, 1) compress_attn_mfma_kernel(CompressArgs a) {
  constexpr int D = 128, G = 4, TK = kTileKeys, RB = D * 2, QR = kCompressRows;
  constexpr int TCH = TK * RB / 16;  // 16-byte chunks of a 64-row K (or V) tile
  // the ring: separate arrays so that the compiler can tell them apart
  __shared__ uint4 lk0[TCH], lk1[TCH], lk2[TCH], lk3[TCH];
  __shared__ uint4 lv0[TCH], lv1[TCH], lv2[TCH], lv3[TCH];
  const DevPool& P = a.P;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // workgroup -> (rank of its pair = sequence x KV head in the launch order,
  // query tile, context split); the workgroups of one pair share blockIdx.x
  // mod 8, i.e. one XCD and its L2
  const int ntq = (4 * a.Kp + QR - 1) / QR;
  const int ns = a.nsplit;
  const int npair = a.n * P.Hkv;
  const int b = blockIdx.x, xcd = b & 7, jj = b >> 3;
  const int rank = (jj / (ntq * ns)) * 8 + xcd, qt = (jj % (ntq * ns)) / ns, sp = jj % ns;
  if (rank >= npair) return;
  const int pair = sgpr(a.desc[a.n * kCompRec + rank]);  // pairs in launch order
  const int i = pair / P.Hkv, hk = pair % P.Hkv;
  // the caller's sequence and KV head of this pair
  const int ir = i / a.hsplit, H = (i % a.hsplit) * P.Hkv + hk, HkvR = P.Hkv * a.hsplit;
  const int32_t* rec = a.desc + i * kCompRec;
  const int slot = rec[0], blk = rec[1], n_pers = rec[2], prompt = rec[3];
  const int32_t* tab = ptab_of(P, slot, a.layer);
  const int npp = (n_pers + TK - 1) / TK, nop = P.C / TK;
  const int ntc = npp + nop;  // context tiles
  const int q0 = qt * QR;     // first query row of the workgroup
  const int nq = min(QR, 4 * a.Kp - q0);
  const int last_pause = (q0 + nq - 1) >> 2;
  // this split's tiles: local tile u < nct is context tile tc0 + u (of
  // [tc0, tc1)); in the last split, pause-key tile u - nct follows
  const int cps = (ntc + ns - 1) / ns;
  const int tc0 = min(ntc, sp * cps), tc1 = min(ntc, tc0 + cps);
  const int nct = tc1 - tc0;
  const int ntp = sp == ns - 1 ? last_pause / TK + 1 : 0;  // pause-key tiles
  const int ntiles = nct + ntp;

  // ---- the wavefront's query rows: rotated at the bitrev position, rounded
  // once to bf16 (like stored keys); the softmax scale goes on the fp32 scores.
  // Rows past the workgroup's last are computed on its first row, not stored.
  // Loaded and rotated by the schedule around the first tiles' issue.
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
  WaveAttn wa;
  int qpause[2];
  QueryRaw qraw[2];
  auto qload = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int r = q0 + wave * 32 + nb * 16 + l16;
      const bool rv = r < q0 + nq;
      r = rv ? r : q0;
      const int pz = r >> 2, hh = r & 3;
      qpause[nb] = rv ? pz : -1;
      const int pos = prompt + blk * P.C + bitrev_dev(pz, a.log2Kp) * (P.C / a.Kp);
      const bf16_t* qrow = (const bf16_t*)a.qp + (((size_t)ir * a.Kp + pz) * a.Hq + H * G + hh) * D;
      query_load(qrow, P.rope + (size_t)pos * (D / 2), g4, qraw[nb]);
    }
  };
  auto qfinish = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) query_rotate(qraw[nb], wa.qh[nb]);
    wa.init();
  };

  // ---- tile t: 64 K rows and 64 V rows (a context page, or pause keys). A
  // page id is fetched one tile ahead with a vector load (the template asks
  // for tiles u = 0, 1, 2, ... in order, the last one repeated past the end),
  // so no scalar-load wait sits at the start of a phase; a pending scalar load
  // would also make every LDS wait of the phase a full one.
  // The table holds tstride entries; an index past it reads 0.
  const __amdgpu_buffer_rsrc_t rtab = __builtin_amdgcn_make_buffer_rsrc((void*)tab, 0, P.tstride * 4, 0x00020000);
  // Per-tile address work is kept small and free of branches: it takes issue
  // slots between the products of a matrix phase. Local tile u < nct is
  // context tile tc0 + u, whose page id sits at table index tc0 + u
  // (persistent) or tc0 + u + open_shift (open block); its K and V rows start
  // page * pstride past the head's bases. Pause-key tile u - nct starts at
  // pause key k0 = 64 (u - nct) of the staged rotated keys and of the caller's
  // values.
  const int open_shift = P.max_pers - npp;
  const uint32_t pstride = (uint32_t)P.Hkv * TK * RB;
  const char* kbase_h = (const char*)P.kpool + (size_t)hk * TK * RB;
  const char* vbase_h = (const char*)P.vpool + (size_t)hk * TK * RB;
  const char* kbase_p = (const char*)a.kp_rot + ((size_t)i * P.Hkv + hk) * a.Kp * RB;
  const char* vbase_p = (const char*)a.vp + ((size_t)ir * a.Kp * HkvR + H) * RB;
  const uint32_t vrow_p = HkvR * RB;
  const int nval_last = n_pers - (npp - 1) * TK;
  // page id of local tile u; past the context tiles the value goes unused
  // (the load reads another entry of the table, or 0 past its end)
  auto load_page = [&](int u) __attribute__((always_inline)) {
    const int t = tc0 + u;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rtab, (t < npp ? t : t + open_shift) * 4, 0, 0);
  };
  int next_page = load_page(0);  // page id of the tile asked for next
  // Both kinds of tile start at base + index * stride: the selects pick the
  // operands, so that no branch forms around the products.
  auto tile_src = [&](int u) __attribute__((always_inline)) {
    const int page = __builtin_amdgcn_readfirstlane(next_page);
    next_page = load_page(u + 1);
    // both sides are computed first, so that the compiler picks with selects
    // instead of forming branches around them
    const bool ctx = u < nct;
    const int k0 = max(u - nct, 0) * TK;
    const int nval_c = tc0 + u == npp - 1 ? nval_last : TK;
    const int nval_p = min(TK, a.Kp - k0);
    const uint32_t idx = ctx ? (uint32_t)page : (uint32_t)k0;
    TileSrc ts;
    ts.kb = (ctx ? kbase_h : kbase_p) + (uint64_t)idx * (ctx ? pstride : (uint32_t)RB);
    ts.vb = (ctx ? vbase_h : vbase_p) + (uint64_t)idx * (ctx ? pstride : vrow_p);
    ts.vstride = ctx ? RB : vrow_p;
    ts.nval = ctx ? nval_c : nval_p;
    return ts;
  };
  // softmax of tile u: masks for partial context pages and pause tiles (a
  // uniform test; in a pause tile a query sees pause keys up to its own)
  auto soft = [&](int u, f32x4_t (&s)[4][2], uint4 (&pb)[2][2]) __attribute__((always_inline)) {
    const bool ctx = u < nct;
    const int kbase = ctx ? 0 : (u - nct) * TK;  // pause index of key 0 of a pause tile
    const int nval = ctx ? (tc0 + u == npp - 1 ? nval_last : TK) : min(TK, a.Kp - kbase);
    auto limits = [&](int (&lim)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) lim[nb] = (ctx ? nval : min(nval, qpause[nb] - kbase + 1)) - 8 * g4;
    };
    wa.softmax(s, !ctx || nval < TK, limits, qs, lane, pb);
  };
  pingpong_attention<1>(wa, ntiles, lane, wave, lk0, lk1, lk2, lk3, lv0, lv1, lv2, lv3, tile_src, soft, qload, qfinish);

  // ---- output: O^T / l; lane holds dims 16 db + 4 g4 + e of query l16. With
  // context splits: the unnormalised partial (O, m, l) for compress_merge_kernel
  if (ns > 1) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float L = rows4_sum(wa.l[nb]);
      const int rl = wave * 32 + nb * 16 + l16;
      if (rl >= nq) continue;
      float* pp = a.part + (((((size_t)i * P.Hkv + hk) * ntq + qt) * ns + sp) * QR + rl) * (D + 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) *(f32x4_t*)(pp + 16 * db + 4 * g4) = wa.acc[nb][db];
      if (g4 == 0) {
        pp[D] = wa.m[nb];
        pp[D + 1] = L;
      }
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = q0 + wave * 32 + nb * 16 + l16;
    if (r >= q0 + nq) continue;
    const int pz = r >> 2, hh = r & 3;
    const size_t row = ((size_t)ir * a.Kp + pz) * a.Hq + H * G + hh;
    wa.store(nb, (bf16_t*)a.out + row * D, a.lse + row, lane);
  }
}

// ---- context splits: merge the partials of one (sequence, KV head, query tile) -------
//
// Workgroup = (pair, query tile, group of 8 query rows); 32 threads per row, 4
// dims each. Each thread fetches the maximum, sum and its 4 output elements of
// eight partials in one round of independent loads and combines them online:
// out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s.
__global__ void __launch_bounds__(256) compress_merge_kernel(CompressArgs a) {
  constexpr int D = 128, G = 4, K = 8, QR = kCompressRows, NRG = QR / 8;
  const int ntq = (4 * a.Kp + QR - 1) / QR, ns = a.nsplit;
  const int rg = blockIdx.x % NRG, pq = blockIdx.x / NRG;
  const int pair = pq / ntq, qt = pq % ntq;
  const int i = pair / a.P.Hkv, hk = pair % a.P.Hkv;
  const int ir = i / a.hsplit, H = (i % a.hsplit) * a.P.Hkv + hk;  // the caller's sequence, KV head
  const int q0 = qt * QR, nq = min(QR, 4 * a.Kp - q0);
  const int rl = rg * 8 + (threadIdx.x >> 5);
  if (rl >= nq) return;
  const size_t stride = (size_t)QR * (D + 2);  // one split's partials
  const float* base = a.part + ((((size_t)i * a.P.Hkv + hk) * ntq + qt) * ns * QR + rl) * (D + 2);
  const int d = 4 * (threadIdx.x & 31);
  float M = -INFINITY, Ls = 0.f;
  f32x4_t O = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += K) {
    float mv[K], lv[K];
    f32x4_t ov[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float* pp = base + (size_t)min(s0 + k, ns - 1) * stride;
      mv[k] = pp[D];
      lv[k] = pp[D + 1];
      ov[k] = *(const f32x4_t*)(pp + d);
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
  const int r = q0 + rl, pz = r >> 2, hh = r & 3;
  const float inv = 1.f / Ls;
  bf16_t* dst = (bf16_t*)a.out + (((size_t)ir * a.Kp + pz) * a.Hq + H * G + hh) * D + d;
  *(uint2*)dst = make_uint2(pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv));
  if (d == 0) a.lse[((size_t)ir * a.Kp + pz) * a.Hq + H * G + hh] = (M + __log2f(Ls)) * 0.6931471805599453f;
}

// ---- launcher ----------------------------------------------------------------------

bool compress_mfma_supported(const DevPool& P, int32_t G) {
  return P.dtype == 1 && P.D == 128 && G == 4 && P.pr == 64;
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const bool mfma = a.P.dtype == 1 && a.P.D == 128 && a.G == 4 && a.P.pr == 64;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D, {
    const int per_k = a.P.Hkv * (DD / 2) / (16 / (int)sizeof(T));
    // fewer pause tokens per workgroup when the grid would be small
    int kpb = per_k >= 256 ? 1 : 256 / per_k;
    while (kpb > 1 && (int64_t)((a.Kp + kpb - 1) / kpb) * a.n < 1024) kpb >>= 1;
    hipLaunchKernelGGL((pause_rope_scatter_kernel<T, DD>), dim3((a.Kp + kpb - 1) / kpb, a.n), dim3(256), 0,
                       s, a, kpb);
    if (!mfma)
      hipLaunchKernelGGL((compress_attn_simt_kernel<T, DD>), dim3(a.Kp, a.P.Hkv * a.G, a.n), dim3(64), 0,
                         s, a);
  });
  if (mfma) {
    // tiles of one (sequence, KV head) pair share blockIdx.x mod 8 (one XCD)
    const int ntq = (4 * a.Kp + kCompressRows - 1) / kCompressRows;
    const int npair = a.n * a.P.Hkv;
    const int nwg = ((npair + 7) / 8) * 8 * ntq * a.nsplit;
    hipLaunchKernelGGL(compress_attn_mfma_kernel, dim3(nwg), dim3(512), 0, s, a);
    if (a.nsplit > 1)
      hipLaunchKernelGGL(compress_merge_kernel, dim3(npair * ntq * (kCompressRows / 8)), dim3(256), 0, s,
                         a);
  }
  return hipGetLastError();
}
}  // namespace abk
