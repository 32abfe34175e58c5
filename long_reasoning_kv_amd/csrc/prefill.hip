// Block-mask prefill: attention of every token of a sequence laid out in
// training order (the prompt, then per block its C text tokens followed, once
// the block is complete, by its K pause tokens) under the block mask of
// Fig. 2(a) of arXiv 2610.20641, one layer. A prompt token sees the prompt
// causally; a text token sees the prompt, the kept code rows (pause k < quota)
// of earlier blocks and its own block's text causally; a pause token sees the
// same plus its whole block and its block's pause keys up to its own. Every
// token is rotated at its own position (pause k of block b at P + bC +
// bitrev(k) C/K, Fig. 2(b)). With compression off the mask is plain causal.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_mfma.h"
#include "common.h"
#include "kernels.h"

namespace abk {

// ---- staging: every key rotated once, values copied, persistent rows gathered ----
//
// Workgroup = kStageRows rows of the sequence; wavefront w takes KV heads w,
// w + 8, ... (so a head's quota is one scalar load), lane (row r, group g)
// the 16-byte group g of each half of row r: it rotates the group's dimension
// pairs (j, j + D/2) in fp64 and rounds once to bf16, like every stored key.
constexpr int kStageRows = 8;
__global__ void __launch_bounds__(512) blockmask_stage_kernel(BlockMaskArgs a) {
  constexpr int D = 128, V = 8, NJ = D / 2 / V;
  static_assert(kStageRows * NJ == 64, "one wavefront covers the workgroup's rows of one head");
  const DevPool& P = a.P;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int row = blockIdx.x * kStageRows + lane / NJ, j0 = (lane % NJ) * V;
  if (row >= a.T) return;
  // a prompt row, and a pause row k < its head's quota (a kept code row), is
  // also one of the head's persistent rows, at index pidx
  int pos, blk = 0, k = 0;
  bool pers = false, pause = false;
  if (!a.compress || row < a.prompt) {
    pos = row;  // prompt rows (all rows when compression is off) sit at their index
    pers = a.compress;
  } else {
    const int rel = row - a.prompt, off = rel % (a.C + a.Kp);
    blk = rel / (a.C + a.Kp);
    if (off < a.C) {
      pos = a.prompt + blk * a.C + off;
    } else {
      k = off - a.C;
      pause = true;
      pos = a.prompt + blk * a.C + bitrev_dev(k, a.log2Kp) * (a.C / a.Kp);
    }
  }
  const double2* rope = P.rope + (size_t)pos * (D / 2) + j0;
  for (int hh = wave; hh < a.Hkv; hh += blockDim.x / 64) {
    const int q = a.quota_h[hh];
    const int pidx = pers ? row : (pause && k < q ? a.prompt + blk * q + k : -1);
    const size_t in = ((size_t)row * a.Hkv + hh) * D;
    const uint4 kw1 = *(const uint4*)((const bf16_t*)a.k + in + j0);
    const uint4 kw2 = *(const uint4*)((const bf16_t*)a.k + in + D / 2 + j0);
    const uint4 vw1 = *(const uint4*)((const bf16_t*)a.v + in + j0);
    const uint4 vw2 = *(const uint4*)((const bf16_t*)a.v + in + D / 2 + j0);
    bf16_t x1[V], x2[V], y1[V], y2[V];
    __builtin_memcpy(x1, &kw1, 16);
    __builtin_memcpy(x2, &kw2, 16);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const double2 cs = rope[e];
      const double a1 = to_f32(x1[e]), a2 = to_f32(x2[e]);
      y1[e] = from_f64<bf16_t>(rot_first(a1, a2, cs));
      y2[e] = from_f64<bf16_t>(rot_second(a1, a2, cs));
    }
    uint4 kr1, kr2;
    __builtin_memcpy(&kr1, y1, 16);
    __builtin_memcpy(&kr2, y2, 16);
    const size_t st = ((size_t)hh * a.T + row) * D;
    *(uint4*)((bf16_t*)a.kst + st + j0) = kr1;
    *(uint4*)((bf16_t*)a.kst + st + D / 2 + j0) = kr2;
    *(uint4*)((bf16_t*)a.vst + st + j0) = vw1;
    *(uint4*)((bf16_t*)a.vst + st + D / 2 + j0) = vw2;
    if (pidx >= 0) {
      const size_t pp = ((size_t)hh * a.npers + pidx) * D;
      *(uint4*)((bf16_t*)a.kpers + pp + j0) = kr1;
      *(uint4*)((bf16_t*)a.kpers + pp + D / 2 + j0) = kr2;
      *(uint4*)((bf16_t*)a.vpers + pp + j0) = vw1;
      *(uint4*)((bf16_t*)a.vpers + pp + D / 2 + j0) = vw2;
    }
  }
}

// ---- attention on bf16 MFMA ---------------------------------------------------
//
// Workgroup = one descriptor record: a KV head and up to 64 query tokens of one
// kind inside one block (query row r is token r/4, head 4h + r%4; each of the 8
// wavefronts owns 32 rows). Its keys are two contiguous ranges: A, the layer's
// persistent rows (kpers: the prompt, then the kept code rows in block order),
// of which it sees the first nA (prompt tokens: causally); and B, its own
// block in training order (kst from the block's first text row), of which it
// sees the first nB rows, text causally and, for pause queries, pause keys up
// to their own. The ranges stream through LDS in 64-key tiles, A then B, on the
// ping-pong schedule of attn_mfma.h; a tile is masked only when one of its keys
// lies past the smallest limit of the workgroup's queries.
__global__ void __launch_bounds__(512, 1) blockmask_attn_mfma_kernel(BlockMaskArgs a) {
  constexpr int D = 128, G = 4, TK = kTileKeys, RB = D * 2;
  constexpr int TCH = TK * RB / 16;  // 16-byte chunks of a 64-row K (or V) tile
  __shared__ uint4 lk0[TCH], lk1[TCH], lk2[TCH], lk3[TCH];
  __shared__ uint4 lv0[TCH], lv1[TCH], lv2[TCH], lv3[TCH];
  const DevPool& P = a.P;
  const int lane = threadIdx.x & 63, wave = sgpr(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int32_t* rec = a.desc + (size_t)blockIdx.x * kBmRec;
  const int hk = rec[0];
  if (hk < 0) return;
  const int kind = rec[1], row0 = rec[2], ntok = rec[3], tok0 = rec[4], nA = rec[5];
  const int bstart = rec[6], nB = rec[7], blk = rec[8];
  const int rowsA = kind == 0 ? tok0 + ntok : nA;  // range A rows the workgroup reads
  const int ntA = (rowsA + TK - 1) / TK, ntB = (nB + TK - 1) / TK, ntiles = ntA + ntB;
  // smallest visibility limit of the workgroup's queries in each range
  const int minA = kind == 0 ? tok0 + 1 : nA;
  const int minB = kind == 1 ? tok0 + 1 : a.C + tok0 + 1;

  // ---- the wavefront's query rows (rotated at their positions, rounded once
  // to bf16) and their limits in both ranges; rows past the record's tokens
  // repeat its last token and are not written
  // (loaded and rotated by the schedule around the first tiles' issue)
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(d)
  WaveAttn wa;
  QueryRaw qraw[2];
  auto qload = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = wave * 32 + nb * 16 + l16;
      const int tok = min(r >> 2, ntok - 1), hh = r & 3;
      const int qi = tok0 + tok;  // the query's index in its range
      int pos;
      if (kind == 0) pos = row0 + tok;
      else if (kind == 1) pos = a.prompt + blk * a.C + qi;
      else pos = a.prompt + blk * a.C + bitrev_dev(qi, a.log2Kp) * (a.C / a.Kp);
      const bf16_t* qrow = (const bf16_t*)a.q + ((size_t)(row0 + tok) * a.Hq + hk * G + hh) * D;
      query_load(qrow, P.rope + (size_t)pos * (D / 2), g4, qraw[nb]);
    }
  };
  auto qfinish = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) query_rotate(qraw[nb], wa.qh[nb]);
    wa.init();
  };
  // the limits of query column nb in ranges A and B (recomputed on the rare
  // masked tile rather than kept in registers across the loop; the empty asm
  // keeps the compiler from hoisting them out of it)
  auto lim_ab = [&](int nb, bool in_a) __attribute__((always_inline)) {
    int l = l16;
    asm volatile("" : "+v"(l));
    const int r = wave * 32 + nb * 16 + l;
    const int qi = tok0 + min(r >> 2, ntok - 1);
    return in_a ? (kind == 0 ? qi + 1 : nA) : (kind == 1 ? qi + 1 : (kind == 2 ? a.C + qi + 1 : 0));
  };

  // ---- tile u: range A tile u (u < ntA), else range B tile u - ntA
  // Range A's rows start at the persistent list's head row, range B's at the
  // block's first staged row; both sides are computed first, so that the
  // compiler picks with selects instead of forming branches.
  const char* kbase_a = (const char*)a.kpers + (size_t)hk * a.npers * RB;
  const char* vbase_a = (const char*)a.vpers + (size_t)hk * a.npers * RB;
  const char* kbase_b = (const char*)a.kst + ((size_t)hk * a.T + bstart) * RB;
  const char* vbase_b = (const char*)a.vst + ((size_t)hk * a.T + bstart) * RB;
  auto tile_src = [&](int u) __attribute__((always_inline)) {
    const bool in_a = u < ntA;
    const int r0a = u * TK, r0b = max(u - ntA, 0) * TK;
    const int r0 = in_a ? r0a : r0b;
    const int rows = in_a ? rowsA : nB;
    TileSrc ts;
    ts.vstride = RB;
    ts.kb = (in_a ? kbase_a : kbase_b) + (size_t)r0 * RB;
    ts.vb = (in_a ? vbase_a : vbase_b) + (size_t)r0 * RB;
    ts.nval = min(TK, rows - r0);
    return ts;
  };
  auto soft = [&](int u, f32x4_t (&s)[4][2], uint4 (&pb)[2][2]) __attribute__((always_inline)) {
    const bool in_a = u < ntA;
    const int r0 = in_a ? u * TK : (u - ntA) * TK;
    const int rows = in_a ? rowsA : nB;
    auto limits = [&](int (&lim)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) lim[nb] = min(lim_ab(nb, in_a), rows) - r0 - 8 * g4;
    };
    wa.softmax(s, r0 + TK > (in_a ? minA : minB), limits, qs, lane, pb);
  };
  pingpong_attention<0>(wa, ntiles, lane, wave, lk0, lk1, lk2, lk3, lv0, lv1, lv2, lv3, tile_src, soft, qload, qfinish);

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = wave * 32 + nb * 16 + l16;
    if ((r >> 2) >= ntok) continue;
    const size_t row = (size_t)(row0 + (r >> 2)) * a.Hq + hk * G + (r & 3);
    wa.store(nb, (bf16_t*)a.out + row * D, a.lse + row, lane);
  }
}

// ---- launcher ----------------------------------------------------------------------

bool blockmask_supported(const DevPool& P, int32_t G) { return P.dtype == 1 && P.D == 128 && G == 4; }

hipError_t launch_blockmask(const BlockMaskArgs& a, int32_t nrec, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(blockmask_stage_kernel, dim3((a.T + kStageRows - 1) / kStageRows), dim3(512), 0, s, a);
  if (nrec > 0) hipLaunchKernelGGL(blockmask_attn_mfma_kernel, dim3(nrec), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace abk
