// Wavefront-level attention on bf16 MFMA over 64-key tiles staged in LDS (d =
// 128, four query heads per KV head), shared by the block-compression kernel
// and the block-mask prefill kernel.
//
// A wavefront owns 32 query rows as two 16-row N-blocks. For every tile:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = the
//                 rotated query rounded once to bf16 (like stored keys; the
//                 softmax scale goes on the fp32 scores), C lane l = keys
//                 4(l/16)+i x query l%16;
//   online softmax per query column, lane-local plus permlane swaps; the
//                 running maximum is only moved (and O^T rescaled) when a
//                 tile's maximum exceeds it by more than 2^8, which keeps the
//                 result exact and makes rescales rare;
//   O^T += V^T P^T: B = P^T straight from the S^T registers (bf16), A = V^T
//                 read from the row-major V tile with ds_read_b64_tr_b16.
// The M-blocks of S^T take keys 32(mb/2) + 8(m/4) + 4(mb%2) + m%4 so that for
// each 32-key step a lane's 8 probabilities are 8 consecutive keys, which is
// what two transposing reads of V deliver. K and V rows in LDS have their
// 16-byte chunks XOR-swizzled by row (K by kswz: bits 0, 1, 3, 4; V by vt_swz:
// bits 0, 1 and 3) so that an A-operand read of either touches every bank
// evenly.
#pragma once

#include "common.h"

namespace abk {

constexpr int kTileKeys = 64;

// V^T operand of O^T += V^T P^T for dims 16db + l%16 and keys k0 + 8(l/16) + 0..7
// of a row-major, swizzled 64-key V tile: two ds_read_b64_tr_b16. Within each
// 16-lane group, lane s supplies row k0 + 8g + 4hh + s/4 at dims 16db + 4(s%4)
// and receives 4 keys of dim 16db + s.
__device__ __forceinline__ int vt_swz(int row) { return 2 * ((row & 3) | ((row >> 1) & 4)); }
__device__ __forceinline__ uint4 vt_operand(const uint4* __restrict__ tile, int db, int k0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int row = k0 + 8 * g + 4 * hh + (s >> 2);
    const int dim = 16 * db + 4 * (s & 3);
    const int chunk = (dim >> 3) ^ vt_swz(row);
    const char* addr = (const char*)(tile + row * 16 + chunk) + 2 * (dim & 7);
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(addr));
    const uint2 u = __builtin_bit_cast(uint2, r);
    w[2 * hh] = u.x;
    w[2 * hh + 1] = u.y;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Two ds_read_b64_tr_b16 four rows apart (halves hh = 0, 1 of a V^T operand),
// joined as one 128-bit operand without moving registers.
typedef short s16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint4 vt_pair(const char* addr) {
  const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(addr));
  const s16x4_t r1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(addr + 4 * 256));
  return __builtin_bit_cast(uint4, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// key of S^T M-block mb, row m (see above)
__device__ __forceinline__ int tile_key(int mb, int m) {
  return 32 * (mb >> 1) + 8 * (m >> 2) + 4 * (mb & 1) + (m & 3);
}

// B operand of S^T for one 16-row N-block: the query row (bf16, pre-RoPE)
// rotated in fp64 with the position's cos/sin row and rounded once to bf16;
// qh[ks] holds dims 32ks + 8 g4 + 0..7.
__device__ __forceinline__ void query_operand(const bf16_t* qrow, const double2* rope, int g4,
                                              uint4 (&qh)[4]) {
  constexpr int D = 128;
  float x[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) unpack16(*(const uint4*)(qrow + 32 * ks + 8 * g4), x[ks], bf16_t());
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    double y0[8], y1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double2 cs = rope[32 * ks + 8 * g4 + j];
      y0[j] = rot_first(x[ks][j], x[ks + 2][j], cs);
      y1[j] = rot_second(x[ks][j], x[ks + 2][j], cs);
    }
    qh[ks] = make_uint4(pack_bf16x2_f64(y0[0], y0[1]), pack_bf16x2_f64(y0[2], y0[3]),
                        pack_bf16x2_f64(y0[4], y0[5]), pack_bf16x2_f64(y0[6], y0[7]));
    qh[ks + 2] = make_uint4(pack_bf16x2_f64(y1[0], y1[1]), pack_bf16x2_f64(y1[2], y1[3]),
                            pack_bf16x2_f64(y1[4], y1[5]), pack_bf16x2_f64(y1[6], y1[7]));
  }
  (void)D;
}

// Per-lane byte offsets of the operand reads of a 64-key tile. They depend on
// the lane only (both swizzles of a row are functions of its low bits, which
// are the lane's): K operand of M-block mb, k-step ks at k[ks] + kmb_off(mb);
// V^T operand of dim block db, key step kk, half hh at v[db] + vkk_off(kk, hh).
struct TileOffsets {
  uint32_t k[4], v[8];
};
__device__ __forceinline__ TileOffsets tile_offsets(int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  TileOffsets o;
  const int kr0 = tile_key(0, l16);  // key row of M-block 0; kswz(tile_key(mb, l16)) = kswz(kr0)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.k[ks] = kr0 * 256 + 16 * ((4 * ks + g4) ^ kswz(kr0));
  const int g = lane >> 4, sl = lane & 15;
  const int row0 = 8 * g + (sl >> 2);  // vt_swz(row0 + 32 kk + 4 hh) = vt_swz(row0)
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int dim = 16 * db + 4 * (sl & 3);
    o.v[db] = row0 * 256 + 16 * ((dim >> 3) ^ vt_swz(row0)) + 2 * (dim & 7);
  }
  return o;
}
__device__ __forceinline__ constexpr int kmb_off(int mb) { return (32 * (mb >> 1) + 4 * (mb & 1)) * 256; }
__device__ __forceinline__ constexpr int vkk_off(int kk, int hh) { return (32 * kk + 4 * hh) * 256; }

// The running state of a wavefront's 32 query rows.
struct WaveAttn {
  uint4 qh[2][4];       // [N-block][k-step]: B operands of S^T
  f32x4_t acc[2][8];    // [N-block][dim block]: O^T, dims 16 db + 4 g4 + e of query l%16
  float m[2], l[2];     // running maximum (log2 units) and this lane's share of the sum

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[nb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // the finite start keeps exp2(s - m) well defined while a column has
      // seen only masked keys
      m[nb] = -1e30f;
      l[nb] = 0.f;
    }
  }

  // One 64-key tile from its K and V buffers in LDS: qk, softmax, pv.
  template <class Limits>
  __device__ __forceinline__ void tile(const uint4* __restrict__ ck, const uint4* __restrict__ cv,
                                       bool masked, Limits limits, float qs, int lane) {
    f32x4_t s[4][2];
    uint4 pb[2][2];
    const TileOffsets o = tile_offsets(lane);
    qk(ck, o, s);
    softmax(s, masked, limits, qs, lane, pb);
    pv(cv, o, pb);
  }

  // S^T of a tile: s[mb][nb] lane l holds the unscaled scores of keys
  // tile_key(mb, 4 g4 + e) against query column l%16 of N-block nb.
  __device__ __forceinline__ void qk(const uint4* __restrict__ ck, const TileOffsets& o,
                                     f32x4_t (&s)[4][2]) const {
    const char* base = (const char*)ck;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 ka = *(const uint4*)(base + o.k[ks] + kmb_off(mb));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) s[mb][nb] = mfma_bf16(ka, qh[nb][ks], s[mb][nb]);
      }
    }
  }

  // Online softmax of a tile's scores. When `masked`, key tile_key(mb, 4 g4 +
  // e) = 8 g4 + (32(mb/2) + 4(mb%2) + e) of query column nb is kept only if
  // 32(mb/2) + 4(mb%2) + e < lim[nb], the bound in this lane's key
  // coordinates that limits(lim) fills (called only then): one compare per
  // element. qs = log2(e)/sqrt(d). Moves the running maximum (rescaling O^T
  // and the sum) when needed, adds the tile's probabilities to the sum and
  // leaves them, as bf16, in pb[nb][kk] (keys 32 kk + 8 g4 + 0..7).
  template <class Limits>
  __device__ __forceinline__ void softmax(f32x4_t (&s)[4][2], bool masked, Limits limits, float qs, int lane,
                                          uint4 (&pb)[2][2]) {
    (void)lane;
    if (masked) {
      int lim[2];
      limits(lim);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[mb][nb][e] = 32 * (mb >> 1) + 4 * (mb & 1) + e < lim[nb] ? s[mb][nb][e] : -INFINITY;
    }
    // per query column (lane-local after the row swaps)
    float mn[2], alpha[2];
    bool moved = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[mb][nb][e]);
      mx = rows4_max(mx) * qs;  // log2 units
      const bool up = mx > m[nb] + 8.f;
      mn[nb] = up ? mx : m[nb];
      alpha[nb] = fast_exp2(m[nb] - mn[nb]);
      moved = moved || up;
      m[nb] = mn[nb];
    }
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        l[nb] *= alpha[nb];
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[nb][db] *= alpha[nb];
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float ps = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(fmaf(s[mb][nb][e], qs, -mn[nb]));
          s[mb][nb][e] = p;  // the score register now holds its probability
          ps += p;
        }
      l[nb] += ps;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // keys 32kk + 8 g4 + j: j < 4 from M-block 2kk, j >= 4 from 2kk+1
        const f32x4_t u0 = s[2 * kk][nb], u1 = s[2 * kk + 1][nb];
        pb[nb][kk] = make_uint4(pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]),
                                pack_bf16x2(u1[0], u1[1]), pack_bf16x2(u1[2], u1[3]));
      }
    }
  }

  // O^T += V^T P^T for a tile's probabilities pb (V^T through two
  // ds_read_b64_tr_b16 per operand, as in vt_operand).
  __device__ __forceinline__ void pv(const uint4* __restrict__ cv, const TileOffsets& o,
                                     const uint4 (&pb)[2][2]) {
    const char* base = (const char*)cv;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 va = vt_pair(base + o.v[db] + vkk_off(kk, 0));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][db] = mfma_bf16(va, pb[nb][kk], acc[nb][db]);
      }
    }
  }

  // The V^T operands of dim blocks db0..db0+3 of a tile, read into registers:
  // va[db - db0][kk].
  __device__ __forceinline__ static void v_operands(const uint4* __restrict__ cv, const TileOffsets& o, int db0,
                                                    uint4 (&va)[4][2]) {
    const char* base = (const char*)cv;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        va[d][kk] = vt_pair(base + o.v[db0 + d] + vkk_off(kk, 0));
      }
  }
  // O^T += V^T P^T for dim blocks db0..db0+3 from operands in registers.
  __device__ __forceinline__ void pv_regs(const uint4 (&va)[4][2], int db0, const uint4 (&pb)[2][2]) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][db0 + d] = mfma_bf16(va[d][kk], pb[nb][kk], acc[nb][db0 + d]);
  }
  // The K operands of M-blocks mb0, mb0 + 1 of a tile: ka[m][ks].
  __device__ __forceinline__ static void k_operands(const uint4* __restrict__ ck, const TileOffsets& o, int mb0,
                                                    uint4 (&ka)[2][4]) {
    const char* base = (const char*)ck;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ka[m][ks] = *(const uint4*)(base + o.k[ks] + kmb_off(mb0 + m));
  }
  // S^T of M-blocks mb0, mb0 + 1 from their K operands.
  __device__ __forceinline__ void qk_regs(const uint4 (&ka)[2][4], int mb0, f32x4_t (&s)[4][2]) const {
    // four independent accumulation chains, interleaved
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          s[mb0 + m][nb] = mfma_bf16(ka[m][ks], qh[nb][ks], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : s[mb0 + m][nb]);
  }

  // Write query column nb's normalised output (bf16, dims 16 db + 4 g4 + e) to
  // dst and, from the lanes of g4 = 0, its natural-log LSE to *lse_dst.
  __device__ __forceinline__ void store(int nb, bf16_t* dst, float* lse_dst, int lane) const {
    const int g4 = lane >> 4;
    const float L = rows4_sum(l[nb]);
    const float inv = 1.f / L;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *(uint2*)(dst + 16 * db + 4 * g4) =
          make_uint2(pack_bf16x2(acc[nb][db][0] * inv, acc[nb][db][1] * inv),
                     pack_bf16x2(acc[nb][db][2] * inv, acc[nb][db][3] * inv));
    if (g4 == 0) *lse_dst = (m[nb] + __log2f(L)) * 0.6931471805599453f;
  }
};

}  // namespace abk
