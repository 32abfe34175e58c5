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

#include <type_traits>

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
// qh[ks] holds dims 32ks + 8 g4 + 0..7. In two steps, so that the loads can be
// issued ahead of other loads and the rotation done later: query_load fetches
// the lane's query dims and cos/sin pairs, query_rotate rotates and rounds.
struct QueryRaw {
  uint4 q[4];        // dims 32ks + 8 g4 + 0..7 (bf16)
  double2 cs[2][8];  // cos/sin of pairs 32ks + 8 g4 + j, ks < 2
};
__device__ __forceinline__ void query_load(const bf16_t* qrow, const double2* rope, int g4, QueryRaw& r) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) r.q[ks] = *(const uint4*)(qrow + 32 * ks + 8 * g4);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) r.cs[ks][j] = rope[32 * ks + 8 * g4 + j];
}
__device__ __forceinline__ void query_rotate(const QueryRaw& r, uint4 (&qh)[4]) {
  float x[4][8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) unpack16(r.q[ks], x[ks], bf16_t());
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    double y0[8], y1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      y0[j] = rot_first(x[ks][j], x[ks + 2][j], r.cs[ks][j]);
      y1[j] = rot_second(x[ks][j], x[ks + 2][j], r.cs[ks][j]);
    }
    qh[ks] = make_uint4(pack_bf16x2_f64(y0[0], y0[1]), pack_bf16x2_f64(y0[2], y0[3]),
                        pack_bf16x2_f64(y0[4], y0[5]), pack_bf16x2_f64(y0[6], y0[7]));
    qh[ks + 2] = make_uint4(pack_bf16x2_f64(y1[0], y1[1]), pack_bf16x2_f64(y1[2], y1[3]),
                            pack_bf16x2_f64(y1[4], y1[5]), pack_bf16x2_f64(y1[6], y1[7]));
  }
}

// Per-lane byte offsets of the operand reads of a 64-key tile. They depend on
// the lane only (both swizzles of a row are functions of its low bits, which
// are the lane's). K operand of M-block mb, k-step ks at k(ks) + kmb_off(mb);
// V^T operand of dim block db, key step kk, half hh at v(db) + vkk_off(kk, hh).
// The k-step (dim block) moves only bits 6-7 (5-7) of the swizzled offset, so
// one base per operand kind is kept and the step is XORed in.
struct TileOffsets {
  uint32_t kb, vb;  // offsets of k-step 0 and of dim block 0
  __device__ __forceinline__ uint32_t k(int ks) const { return kb ^ (64u * ks); }
  __device__ __forceinline__ uint32_t v(int db) const { return vb ^ (32u * db); }
};
__device__ __forceinline__ TileOffsets tile_offsets(int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  TileOffsets o;
  const int kr0 = tile_key(0, l16);  // key row of M-block 0; kswz(tile_key(mb, l16)) = kswz(kr0)
  o.kb = kr0 * 256 + 16 * (g4 ^ kswz(kr0));
  const int sl = lane & 15;
  const int row0 = 8 * g4 + (sl >> 2);  // vt_swz(row0 + 32 kk + 4 hh) = vt_swz(row0)
  const int dim = 4 * (sl & 3);
  o.vb = row0 * 256 + 16 * ((dim >> 3) ^ vt_swz(row0)) + 2 * (dim & 7);
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

  // Plain v_max_f32 / v_min_f32 / v_max3_f32. fmaxf under IEEE mode must quiet a
  // signalling NaN, so the compiler puts a canonicalising v_max x, x in front
  // of every operand it cannot prove canonical (MFMA and lane-swap results);
  // the scores here are finite or -inf.
  __device__ __forceinline__ static float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  __device__ __forceinline__ static float vmin(float a, float b) {
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  __device__ __forceinline__ static float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
  }
  // Maximum of query column nb's 16 scores in this lane, as a tree.
  __device__ __forceinline__ static float col_max(const f32x4_t (&s)[4][2], int nb) {
    const float a = vmax3(s[0][nb][0], s[0][nb][1], s[0][nb][2]);
    const float b = vmax3(s[0][nb][3], s[1][nb][0], s[1][nb][1]);
    const float c = vmax3(s[1][nb][2], s[1][nb][3], s[2][nb][0]);
    const float d = vmax3(s[2][nb][1], s[2][nb][2], s[2][nb][3]);
    const float e = vmax3(s[3][nb][0], s[3][nb][1], s[3][nb][2]);
    return vmax(vmax3(a, b, c), vmax3(d, e, s[3][nb][3]));
  }
  // The maxima over the four lanes l%16 + 16r (r = 0..3) of both columns at
  // once: the first swap pairs column 0's odd rows with column 1's even rows,
  // so that after it and the 32-lane swap rows 0, 2 hold column 0's maximum
  // and rows 1, 3 column 1's; the last swap hands every lane both.
  __device__ __forceinline__ static void rows4_max2(float& x0, float& x1) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
    const float m = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    const float y = vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    x0 = __uint_as_float(c[0]);
    x1 = __uint_as_float(c[1]);
  }

  // Online softmax of a tile's scores. When `masked`, key tile_key(mb, 4 g4 +
  // e) = 8 g4 + (32(mb/2) + 4(mb%2) + e) of query column nb is kept only if
  // 32(mb/2) + 4(mb%2) + e < lim[nb], the bound in this lane's key
  // coordinates that limits(lim) fills (called only then). qs =
  // log2(e)/sqrt(d). Moves the running maximum (rescaling O^T and the sum)
  // when needed, adds the tile's probabilities to the sum and leaves them, as
  // bf16, in pb[nb][kk] (keys 32 kk + 8 g4 + 0..7).
  template <class Limits>
  __device__ __forceinline__ void softmax(f32x4_t (&s)[4][2], bool masked, Limits limits, float qs, int lane,
                                          uint4 (&pb)[2][2]) {
    (void)lane;
    if (masked) {
      // key position k (0..39) is kept if k < lim, i.e. if (lim - 0.5 - k)
      // 2^120 is positive: that bound is then at least 2^119 and min(s, bound)
      // = s (the scores are far smaller); for a dropped key it is at most
      // -2^119, which the exponential turns into exactly 0. With lim clamped
      // to [-1, 64] no bound overflows. One FMA and one min per score, with
      // no compare-to-mask hazard between them.
      int lim[2];
      limits(lim);
      constexpr float big = 0x1p120f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float fl = ((float)min(max(lim[nb], -1), 64) - 0.5f) * big;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          // four bounds, then their four minima (the empty asm takes all four,
          // so that no min issues right behind the product it reads)
          float bnd[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) bnd[e] = fmaf(-(float)(32 * (mb >> 1) + 4 * (mb & 1) + e), big, fl);
          asm volatile("" : "+v"(bnd[0]), "+v"(bnd[1]), "+v"(bnd[2]), "+v"(bnd[3]));
#pragma unroll
          for (int e = 0; e < 4; ++e) s[mb][nb][e] = vmin(s[mb][nb][e], bnd[e]);
        }
      }
    }
    // The running maximum of a column moves only when the tile's maximum
    // exceeds it by more than 8 (log2 units). The probabilities are first
    // taken against the current maximum, with the scores kept; such a score
    // gives a probability above 256, so a lane whose column sum stays at most
    // 255 holds none (nor an overflow, which the first tile, with m = -1e30,
    // always has). Only when some lane of the wavefront passes that test
    // does the exact step run: per column the maximum of its lanes' scores
    // (a lane-local tree, then three lane swaps), the move and the rescale,
    // and the probabilities again. A wavefront that stays below the bound
    // ends with the values that step would give; the test on the sums
    // replaces the maximum's tree and swaps on most tiles.
    f32x4_t p[4][2];
    float st[2];
    auto probs = [&]() __attribute__((always_inline)) {
      // four exponent arguments, then their four exponentials: the empty asm
      // takes all four, so that each exponential issues three instructions
      // after the product it reads instead of right behind it
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = fmaf(s[mb][nb][e], qs, -m[nb]);
          asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
#pragma unroll
          for (int e = 0; e < 4; ++e) p[mb][nb][e] = fast_exp2(x[e]);
        }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float q4[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) q4[mb] = (p[mb][nb][0] + p[mb][nb][1]) + (p[mb][nb][2] + p[mb][nb][3]);
        st[nb] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
      }
    };
    probs();
    // (written so that a NaN sum, from an infinite probability, passes too)
    const bool big = !(st[0] <= 255.f) || !(st[1] <= 255.f);
    if (__builtin_amdgcn_ballot_w64(big)) {
      float mx[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) mx[nb] = col_max(s, nb);
      rows4_max2(mx[0], mx[1]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float t = mx[nb] * qs;  // log2 units
        const float mn = t > m[nb] + 8.f ? t : m[nb];
        const float alpha = fast_exp2(m[nb] - mn);
        m[nb] = mn;
        l[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[nb][db] *= alpha;
      }
      probs();
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      l[nb] += st[nb];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // keys 32kk + 8 g4 + j: j < 4 from M-block 2kk, j >= 4 from 2kk+1
        const f32x4_t u0 = p[2 * kk][nb], u1 = p[2 * kk + 1][nb];
        pb[nb][kk] = make_uint4(pack_bf16x2(u0[0], u0[1]), pack_bf16x2(u0[2], u0[3]),
                                pack_bf16x2(u1[0], u1[1]), pack_bf16x2(u1[2], u1[3]));
      }
    }
  }

  // The V^T operands of dim blocks db0..db0+3 of a tile, read into registers
  // in the order pv_regs uses them: va[db - db0][kk].
  __device__ __forceinline__ static void v_operands(const uint4* __restrict__ cv, const TileOffsets& o, int db0,
                                                    uint4 (&va)[4][2]) {
    const char* base = (const char*)cv;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d = 0; d < 4; ++d) va[d][kk] = vt_pair(base + o.v(db0 + d) + vkk_off(kk, 0));
  }
  // O^T += V^T P^T for dim blocks db0..db0+3 from operands in registers.
  // Key step outermost, so that the two products into one accumulator are
  // eight products apart.
  __device__ __forceinline__ void pv_regs(const uint4 (&va)[4][2], int db0, const uint4 (&pb)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][db0 + d] = mfma_bf16(va[d][kk], pb[nb][kk], acc[nb][db0 + d]);
  }
  // The K operands of M-blocks mb0, mb0 + 1 of a tile: ka[m][ks], read in the
  // order qk_regs uses them.
  __device__ __forceinline__ static void k_operands(const uint4* __restrict__ ck, const TileOffsets& o, int mb0,
                                                    uint4 (&ka)[2][4]) {
    const char* base = (const char*)ck;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int m = 0; m < 2; ++m) ka[m][ks] = *(const uint4*)(base + o.k(ks) + kmb_off(mb0 + m));
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

// Scheduling groups for the compiler's scheduler: the next n MFMAs, or the
// next n LDS reads, of the region in program order.
template <int n>
__device__ __forceinline__ void sched_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x008, n, 0);
}
template <int n>
__device__ __forceinline__ void sched_lds() {
  __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
}

// Where a 64-key tile lies: K row r at kb + 256 r, V row r at vb + vstride r;
// rows past nval repeat row nval - 1 (their keys are masked).
struct TileSrc {
  const char* kb;
  const char* vb;
  int vstride, nval;
};

// Attention of a workgroup of eight wavefronts (256 query rows, the 32 rows of
// each wavefront in wa) over ntiles 64-key tiles, on a ping-pong schedule. The
// wavefronts form two groups, wavefronts w and w + 4 sharing a SIMD, kept one
// phase apart by a workgroup barrier between phases. In a matrix phase a
// wavefront runs the previous tile's O^T += V^T P^T and then this tile's S^T =
// K Q^T (64 MFMAs); in a vector phase it runs this tile's softmax. The groups
// alternate, so each SIMD's matrix core works on one group's products while its
// vector unit runs the other group's softmax:
//   phase 2u:   group 0 matrix (PV u-1, QK u)   group 1 softmax u-1
//   phase 2u+1: group 0 softmax u               group 1 matrix (PV u-1, QK u)
// for u = 0..ntiles (the matrix phase of u = 0 adds zeros, that of u = ntiles
// runs on a repeated tile and its scores are dropped, and no softmax phase runs
// for u = ntiles). Tiles stream straight into a ring
// of four LDS buffers (32 KB each: K rows swizzled by kswz, V rows by vt_swz):
// at phase 2u each wavefront of group 0 issues its share of tile u+2 (whose
// scalar part, the tile source and buffer descriptors, it prepared in its
// softmax phase of tile u-1), and before the barrier that ends phase 2u it
// waits for its share of tile u+1.
// Tile u's buffer is read from phase 2u to 2u+3, and the load into it is
// issued at phase 2u-4, after the barrier that ends its previous tile's last
// read.
// tile_src(u) gives tile u's place; each wavefront of group 0 asks for u = 0, 1, 2, ...
// in order, once each, then for ntiles - 1 again past the end (a tile source
// may fetch ahead: it then issues kSrcLoads memory loads per call, at most 7). soft(u, s, pb) runs tile u's
// softmax (wa.softmax with the tile's masks). The ring buffers are separate
// __shared__ arrays of the kernel, so that the compiler can tell them apart.
// qload() issues the loads of the wavefront's query rows and qfinish() turns
// them into wa's query operands and initial state: the query loads go out
// between the first two tiles' and the rotation follows, so that both pass
// under the first tile's latency.
template <int kSrcLoads, class TileFn, class SoftFn, class QLoadFn, class QFinishFn>
__device__ __forceinline__ void pingpong_attention(WaveAttn& wa, int ntiles, int lane, int wave,
                                                   uint4* __restrict__ lk0, uint4* __restrict__ lk1,
                                                   uint4* __restrict__ lk2, uint4* __restrict__ lk3,
                                                   uint4* __restrict__ lv0, uint4* __restrict__ lv1,
                                                   uint4* __restrict__ lv2, uint4* __restrict__ lv3,
                                                   TileFn tile_src, SoftFn soft, QLoadFn qload,
                                                   QFinishFn qfinish) {
  static_assert(kSrcLoads >= 0 && kSrcLoads <= 7, "the wait count holds 15 loads");
  constexpr int RB = 256;  // bytes of a bf16 row of 128 dims
  const bool grp0 = wave < 4;
  // Tile t straight from global memory into LDS (buffer_load_dwordx4 ... lds,
  // the MUBUF form: the compiler's wait counting treats a FLAT load into LDS as
  // an LDS access of unknown order and then waits for every LDS read). Group 0
  // alone loads the tiles, in its matrix phases, where the address work takes
  // issue slots between the products; group 1's softmax phases then carry no
  // load work. In load j of wavefront w (w < 4), lane l fills LDS chunk 256j +
  // 64w + l, i.e. row 16j + 4w + l/16 at swizzled position l%16, so it fetches
  // the source chunk that belongs there (the V swizzle ignores bits 4 and 5 of
  // the row, the K swizzle bit 5). Rows past the tile's valid count repeat its
  // last row. Eight loads per wavefront of group 0.
  const int r_in = 4 * wave + (lane >> 4);
  const int kc0 = 16 * ((lane & 15) ^ kswz(r_in)), kc1 = 16 * ((lane & 15) ^ kswz(16 + r_in));
  const int vc = 16 * ((lane & 15) ^ vt_swz(r_in));
  // One form for every tile, without branches, so that its instructions can
  // be spread between the products: load j takes row min(16 j + r_in, nval -
  // 1) of the tile (a row of a whole tile is its own), at a per-lane offset.
  // The issue in two parts: prep (the tile source and the buffer descriptors,
  // scalar work) and fire (the eight row loads). Group 0 preps tile u+3 in its
  // softmax phase of tile u, where the scalar instructions take issue slots
  // between dependent vector ones, and fires it in its next matrix phase.
  struct Prepped {
    __amdgpu_buffer_rsrc_t rk, rv;
    int last, vstride;
  };
  auto prep = [&](int u) __attribute__((always_inline)) {
    const TileSrc ts = tile_src(min(u, ntiles - 1));
    Prepped p;
    p.last = ts.nval - 1;
    p.vstride = ts.vstride;
    // raw buffer descriptors over the tile's K and V (stride 0, a range the
    // offsets never reach; 0x00020000 is the format word of untyped data)
    p.rk = __builtin_amdgcn_make_buffer_rsrc((void*)ts.kb, 0, 0x7fffffff, 0x00020000);
    p.rv = __builtin_amdgcn_make_buffer_rsrc((void*)ts.vb, 0, 0x7fffffff, 0x00020000);
    return p;
  };
  auto fire = [&](const Prepped& p, uint4* __restrict__ dk, uint4* __restrict__ dv) __attribute__((always_inline)) {
#pragma unroll
    // (row < 64 and the strides below 2^24: 24-bit products, one multiply-add)
    for (int j = 0; j < 4; ++j) {
      const int row = min(16 * j + r_in, p.last);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rk, (__attribute__((address_space(3))) void*)(dk + 256 * j + 64 * wave),
                                               16, row * RB + ((j & 1) ? kc1 : kc0), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rv, (__attribute__((address_space(3))) void*)(dv + 256 * j + 64 * wave),
                                               16, (int)__umul24(row, p.vstride) + vc, 0, 0, 0);
    }
  };
  auto issue = [&](int u, uint4* __restrict__ dk, uint4* __restrict__ dv) __attribute__((always_inline)) {
    fire(prep(u), dk, dv);
  };
  Prepped next;  // group 0: the tile its next matrix phase issues
  // the end of a phase: the wavefront's LDS reads have returned and, at the end
  // of group 0's matrix phase, its loads older than this phase's (eight rows
  // and the tile source's own kSrcLoads, in any order) have landed; then every wavefront of the workgroup gets here (the loads of
  // group 0 are then in LDS). The signal fences keep the compiler from moving
  // LDS accesses across the barrier, the scheduling barriers any other
  // instruction (products of one phase must not sink into the next).
  auto end_phase = [&](bool wait_loads) __attribute__((always_inline)) {
    // vmcnt(8 + kSrcLoads) lgkmcnt(0): this phase's loads may fly
    if (wait_loads) __builtin_amdgcn_s_waitcnt(0x0070 | (8 + kSrcLoads));
    else __builtin_amdgcn_s_waitcnt(0xC07F);             // lgkmcnt(0): this phase's LDS reads are done
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // Carried across the barrier from a tile's softmax phase to the next matrix
  // phase: the tile's probabilities (pb) and the next tile's K operands of
  // M-blocks 0, 1 (ka). Before the first tile pb is zero and the previous V
  // buffer (lv3) holds zeros, so the first matrix phase's P V adds exact zeros
  // and needs no branch.
  uint4 pb[2][2], ka[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) pb[nb][kk] = make_uint4(0u, 0u, 0u, 0u);
  TileOffsets to = tile_offsets(lane);
  // The empty asm hides the lane offsets' values from the compiler, so that it
  // adds them to each buffer's address at the read (an immediate offset)
  // instead of keeping a register per buffer, and forms the XORed offsets of
  // each phase inside it instead of keeping them live across the loop.
  auto refresh = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(to.kb));
    asm volatile("" : "+v"(to.vb));
  };
  // matrix phase of tile u: Q K^T of tile u and P V of tile u-1, with no branch
  // (past the last tile the products run on the spare buffer's repeated tile
  // and are discarded). M-blocks 0, 1 come from registers; each group of
  // operand reads is issued one group of products ahead of its use.
  // With `loads` (group 0) the phase also issues tile u+2 (`pre`), in the same
  // scheduling region, its scalar and load instructions spread between the
  // first products instead of ahead of them.
  auto matrix = [&](auto loads, auto pre, const uint4* __restrict__ k0, const uint4* __restrict__ vm1,
                    f32x4_t (&s)[4][2]) __attribute__((always_inline)) {
    refresh();
    pre();
    uint4 vb[4][2], vc[4][2], kb[2][4];
    WaveAttn::v_operands(vm1, to, 0, vb);
    wa.qk_regs(ka, 0, s);
    WaveAttn::k_operands(k0, to, 2, kb);
    wa.pv_regs(vb, 0, pb);
    WaveAttn::v_operands(vm1, to, 4, vc);
    wa.qk_regs(kb, 2, s);
    wa.pv_regs(vc, 4, pb);
    // The order (mask 8: MFMA, 0x100: LDS read): each group of operand reads
    // goes between the products before its use, at most 14 reads in flight so
    // that the waits can name the reads a product needs (the LDS counter
    // holds 15).
    if constexpr (decltype(loads)::value) {
      // and (mask 0x20: memory load) the tile issue, prepared in the softmax
      // phase before: a row load after each product from the seventh on; the
      // per-lane offsets in between are left to the scheduler (scalar groups as
      // well make it gather all the loads in one place)
#pragma unroll
      for (int i = 0; i < 14; ++i) {
        sched_mfma<1>();
        sched_lds<1>();
        if (i >= 6) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 14; ++i) {  // Q K^T of M-blocks 0, 1 with V^T reads 1..14 of dims 0..63
        sched_mfma<1>();
        sched_lds<1>();
      }
    }
    sched_mfma<2>();
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // P V of dims 0..63 with V^T reads 15, 16 and K reads 1..6
      sched_mfma<2>();
      sched_lds<1>();
    }
    sched_lds<2>();  // K reads 7, 8
#pragma unroll
    for (int i = 0; i < 14; ++i) {  // Q K^T of M-blocks 2, 3 with V^T reads 1..14 of dims 64..127
      sched_mfma<1>();
      sched_lds<1>();
    }
    sched_mfma<2>();
    sched_mfma<2>();  // P V of dims 64..127 with V^T reads 15, 16
    sched_lds<2>();
    sched_mfma<14>();
  };
  // softmax phase of tile u, with the K operands of M-blocks 0, 1 of tile u+1
  // read from its buffer k1 (in LDS since the barrier that began this phase),
  // and (`pre`, group 0) the scalar work of the next tile issue, which the
  // scheduler spreads between the softmax's dependent vector instructions
  auto vector = [&](int u, const uint4* __restrict__ k1, f32x4_t (&s)[4][2], auto pre)
      __attribute__((always_inline)) {
    if (u >= ntiles) return;
    refresh();
    // the reads first, so that their latency passes under the softmax
    WaveAttn::k_operands(k1, to, 0, ka);
    __builtin_amdgcn_sched_barrier(0);
    pre();
    soft(u, s, pb);
  };
  // Tile u: its matrix phase, then its softmax phase; group 0 runs them as
  // phases 2u and 2u+1, group 1 one phase later. Tile u is in buffer (k0, v0),
  // tile u+1 in (k1, v1); at every even phase 2u each wavefront of group 0
  // issues its share of tile u+2 (past the end it repeats the last tile into
  // the spare buffer) and at the end of it waits for its share of tile u+1.
  // Each group runs its own copy of the loop; both pass the same number of
  // barriers.
  auto tile0 = [&](int u, const uint4* __restrict__ k0, const uint4* __restrict__ vm1,
                   const uint4* __restrict__ k1, uint4* __restrict__ k2, uint4* __restrict__ v2)
      __attribute__((always_inline)) {
    f32x4_t s[4][2];
    matrix(std::true_type{}, [&]() __attribute__((always_inline)) { fire(next, k2, v2); }, k0, vm1, s);
    end_phase(true);
    vector(u, k1, s, [&]() __attribute__((always_inline)) { next = prep(u + 3); });
    end_phase(false);
  };
  auto tile1 = [&](int u, const uint4* __restrict__ k0, const uint4* __restrict__ vm1,
                   const uint4* __restrict__ k1) __attribute__((always_inline)) {
    f32x4_t s[4][2];
    matrix(std::false_type{}, []() {}, k0, vm1, s);
    end_phase(false);
    vector(u, k1, s, []() {});
    end_phase(false);
  };

  if (ntiles <= 0) {
    qload();
    qfinish();
    return;
  }
  {
    // zeros in the V buffer that the first matrix phase reads as tile -1
    // (before any load into LDS is in flight, which a store would wait for)
    lv3[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    lv3[threadIdx.x + 512] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_sched_barrier(0);
    // tile 0, the query loads, then tile 1: a tile source that fetches its
    // next page id ahead (one load of its own) has that id ahead of the query
    // loads too, so taking it waits for none of them
    if (grp0) issue(0, lk0, lv0);
    __builtin_amdgcn_sched_barrier(0);
    qload();
    __builtin_amdgcn_sched_barrier(0);
    if (grp0) issue(1, lk1, lv1);
    __builtin_amdgcn_sched_barrier(0);
    qfinish();
    // the empty asm uses the query operands, so that the rotation is done here,
    // under the tiles' latency, not sunk below the wait that follows
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        asm volatile("" ::"v"(wa.qh[nb][ks].x), "v"(wa.qh[nb][ks].y), "v"(wa.qh[nb][ks].z), "v"(wa.qh[nb][ks].w));
    // tile 2's scalar work (its page id, fetched with tile 1's, is older than
    // tile 1's row loads, so taking it waits for those of tile 0 and the query)
    __builtin_amdgcn_sched_barrier(0);
    if (grp0) next = prep(2);
    end_phase(grp0);  // tile 0 and the zeros are in
    if (grp0) {
      WaveAttn::k_operands(lk0, to, 0, ka);
      for (int u = 0; u <= ntiles; u += 4) {
        tile0(u, lk0, lv3, lk1, lk2, lv2);
        if (u + 1 > ntiles) break;
        tile0(u + 1, lk1, lv0, lk2, lk3, lv3);
        if (u + 2 > ntiles) break;
        tile0(u + 2, lk2, lv1, lk3, lk0, lv0);
        if (u + 3 > ntiles) break;
        tile0(u + 3, lk3, lv2, lk0, lk1, lv1);
      }
      end_phase(false);  // group 1's last softmax phase
    } else {
      WaveAttn::k_operands(lk0, to, 0, ka);
      end_phase(false);  // phase 0: group 0's first matrix phase
      for (int u = 0; u <= ntiles; u += 4) {
        tile1(u, lk0, lv3, lk1);
        if (u + 1 > ntiles) break;
        tile1(u + 1, lk1, lv0, lk2);
        if (u + 2 > ntiles) break;
        tile1(u + 2, lk2, lv1, lk3);
        if (u + 3 > ntiles) break;
        tile1(u + 3, lk3, lv2, lk0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load may land in LDS after the end
  }
}

}  // namespace abk
