/* AbridgeKV CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 statement of what the attention hot path computes. Only
 * tests, the smoke check and the benchmark's CPU-baseline leg may call it; the
 * GPU library never links or loads it, and it shares no code with the library.
 *
 * Sources (the pages this follows):
 *  - "AbridgeKV: Compressing Long Reasoning into the KV Cache of Learned Pause
 *    Tokens" (arXiv 2610.20641) abstract: blocks of generated text are
 *    compressed into the KV entries of pause tokens, whose entries take
 *    positions inside the block they replace; the block's raw cache is freed
 *    and later tokens attend to the pause tokens' entries instead.
 *  - Figure captions of 2610.20641: Fig. 1(a) (blocks of C tokens, K pause
 *    tokens write code rows, raw rows freed), Fig. 2(a) (attention mask for
 *    two blocks), Fig. 2(b) (pause token k sits at bitrev(k)*C/K inside the
 *    block), Fig. 6(b) (per-layer quotas 256/128/64).
 *  - The AI Radio transcript of the same paper: resident cache = prompt + code
 *    rows of finished blocks + the open block; a layer never allocates rows it
 *    does not retain.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - Pause tokens attend causally among themselves in pause-index order.
 *  - Pause tokens see all C rows of their block (they run after it completes).
 *  - Layer l keeps the prefix k < quota[l] of the K pause tokens' rows.
 *  - RoPE is rotate-half with theta_i = pos * base^(-2i/d); V is not rotated.
 *  - Cached keys are RoPE(k) rounded once to the cache's storage type; the
 *    rotated query is rounded once to the same type (the attention takes
 *    storage-type operands with fp64 accumulation here, fp32 on the device).
 *  - Scores are q'.k'/sqrt(d); lse is the natural log of sum exp(score).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_PROMPT 0
#define ORC_TEXT 1
#define ORC_PAUSE 2

#define ORC_F32 0
#define ORC_BF16 1

/* One layer's view of one sequence. */
typedef struct {
  int32_t P;        /* prompt tokens */
  int32_t C;        /* block size */
  int32_t Kp;       /* pause tokens run per compression at this layer */
  int32_t quota;    /* code rows this layer keeps per compressed block */
  int32_t compress; /* 0: full-KV, blocks never close */
} orc_layer;

/* ---- positions (Fig. 2(b)) ---------------------------------------------- */

/* Reverse the low `nbits` bits of k. */
int orc_bitrev(int k, int nbits) {
  int r = 0;
  for (int i = 0; i < nbits; i++)
    if (k & (1 << i)) r |= 1 << (nbits - 1 - i);
  return r;
}

/* log2 of a power of two, else -1. */
int orc_log2_exact(int x) {
  if (x <= 0) return -1;
  int n = 0;
  while ((1 << n) < x) n++;
  return (1 << n) == x ? n : -1;
}

/* RoPE position of a logical token. Prompt token i sits at i, generated token
 * j at P + j, and pause token k of block b inside the block it replaces, at
 * P + b*C + bitrev(k)*C/Kp. */
int64_t orc_position(const orc_layer* L, int kind, int64_t a, int64_t b) {
  if (kind == ORC_PROMPT) return a;
  if (kind == ORC_TEXT) return (int64_t)L->P + a;
  int nbits = orc_log2_exact(L->Kp);
  return (int64_t)L->P + a * L->C + (int64_t)orc_bitrev((int)b, nbits) * (L->C / L->Kp);
}

/* ---- the block mask (Fig. 2(a)), applied to logical tokens --------------- */

/* Index of a token in creation order: the prompt, then per block its C text
 * tokens followed by its Kp pause tokens. */
int64_t orc_creation_index(const orc_layer* L, int kind, int64_t a, int64_t b) {
  if (kind == ORC_PROMPT) return a;
  int64_t per_block = L->compress ? (int64_t)L->C + L->Kp : (int64_t)L->C;
  if (kind == ORC_TEXT) return L->P + (a / L->C) * per_block + a % L->C;
  return L->P + a * per_block + L->C + b;
}

static int64_t orc_block_of(const orc_layer* L, int kind, int64_t a) {
  if (kind == ORC_TEXT) return a / L->C;
  if (kind == ORC_PAUSE) return a;
  return -1;
}

/* May `query` attend to `key` at this layer? R1 causal in creation order;
 * R2 prompt always; R3 raw text only inside the query's own block; R4 pause
 * rows of earlier blocks only when retained (k < quota), pause rows of the
 * query's own block causally. With compression off this is plain causal
 * attention over prompt and text. */
int orc_visible(const orc_layer* L, int qkind, int64_t qa, int64_t qb, int kkind, int64_t ka,
                int64_t kb) {
  if (orc_creation_index(L, kkind, ka, kb) > orc_creation_index(L, qkind, qa, qb)) return 0;
  if (kkind == ORC_PROMPT) return 1;
  if (!L->compress) return kkind == ORC_TEXT;
  int64_t qblock = orc_block_of(L, qkind, qa);
  if (kkind == ORC_TEXT) return orc_block_of(L, ORC_TEXT, ka) == qblock;
  if (ka < qblock) return kb < L->quota;
  if (qkind == ORC_PAUSE && ka == qblock) return kb <= qb;
  return 0;
}

/* Enumerate every logical token that exists when `query` runs (G text tokens
 * written, pause tokens of blocks < nb created, plus the query's own block's
 * pause tokens when the query is one), in creation order, and keep those the
 * mask shows. Returns the number kept (may exceed cap; only cap are stored). */
int64_t orc_visible_keys(const orc_layer* L, int64_t G, int64_t nb, int qkind, int64_t qa,
                         int64_t qb, int32_t* kind, int64_t* ka, int64_t* kb, int64_t* pos,
                         int64_t cap) {
  int64_t n = 0;
#define ORC_TRY(KI, A, B)                                               \
  do {                                                                  \
    if (orc_visible(L, qkind, qa, qb, (KI), (A), (B))) {                \
      if (n < cap) {                                                    \
        kind[n] = (KI);                                                 \
        ka[n] = (A);                                                    \
        kb[n] = (B);                                                    \
        pos[n] = orc_position(L, (KI), (A), (B));                       \
      }                                                                 \
      n++;                                                              \
    }                                                                   \
  } while (0)
  for (int64_t i = 0; i < L->P; i++) ORC_TRY(ORC_PROMPT, i, 0);
  int64_t nblocks_text = (G + L->C - 1) / L->C;
  int64_t pause_blocks = nb;
  if (qkind == ORC_PAUSE && qa + 1 > pause_blocks) pause_blocks = qa + 1;
  int64_t last = nblocks_text > pause_blocks ? nblocks_text : pause_blocks;
  for (int64_t blk = 0; blk < last; blk++) {
    for (int64_t i = 0; i < L->C; i++) {
      int64_t j = blk * L->C + i;
      if (j >= G) break;
      ORC_TRY(ORC_TEXT, j, 0);
    }
    if (L->compress && blk < pause_blocks)
      for (int64_t k = 0; k < L->Kp; k++) ORC_TRY(ORC_PAUSE, blk, k);
  }
#undef ORC_TRY
  return n;
}

/* ---- RoPE and storage rounding ------------------------------------------- */

/* Round a double once to bf16 (8 significant bits, nearest-even, fp32 range). */
double orc_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e = ilogb(x);
  if (e < -126) e = -126; /* subnormal spacing 2^-133 */
  double r = nearbyint(ldexp(x, 7 - e));
  double y = ldexp(r, e - 7);
  if (fabs(y) > 0x1.FEp127) return x > 0 ? INFINITY : -INFINITY;
  return y;
}

double orc_round(double x, int dtype) {
  return dtype == ORC_BF16 ? orc_round_bf16(x) : (double)(float)x;
}

/* Rotate-half RoPE of x[n][H][d] at pos[n]: pairs (x_i, x_{i+d/2}) turn by
 * theta_i = pos * base^(-2i/d). round_dtype < 0 keeps doubles, else rounds
 * each result once to that storage type. */
void orc_rope_rows(const double* x, const int64_t* pos, int64_t n, int H, int d, double base,
                   int round_dtype, double* y) {
  int half = d / 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++) {
    for (int h = 0; h < H; h++) {
      const double* xi = x + (r * H + h) * d;
      double* yi = y + (r * H + h) * d;
      for (int i = 0; i < half; i++) {
        double theta = (double)pos[r] * pow(base, -2.0 * i / d);
        double c = cos(theta), s = sin(theta);
        double a = xi[i], b = xi[i + half];
        double ya = a * c - b * s;
        double yb = b * c + a * s;
        if (round_dtype >= 0) {
          ya = orc_round(ya, round_dtype);
          yb = orc_round(yb, round_dtype);
        }
        yi[i] = ya;
        yi[i + half] = yb;
      }
    }
  }
}

/* ---- attention ------------------------------------------------------------ */

/* Softmax attention of q[Hq][d] (already rotated) over n keys/values
 * k,v[n][Hkv][d]; query head h reads KV head h / (Hq/Hkv). Score = q.k/sqrt(d);
 * lse = max + ln sum exp(score - max); out = sum exp(score - lse) v. */
void orc_attention(const double* q, int Hq, int Hkv, int d, int64_t n, const double* k,
                   const double* v, double* out, double* lse) {
  int g = Hq / Hkv;
  double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < Hq; h++) {
    int hk = h / g;
    const double* qh = q + (int64_t)h * d;
    double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
    double m = -INFINITY;
    for (int64_t j = 0; j < n; j++) {
      const double* kj = k + (j * Hkv + hk) * d;
      double acc = 0.0;
      for (int i = 0; i < d; i++) acc += qh[i] * kj[i];
      s[j] = acc * scale;
      if (s[j] > m) m = s[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n; j++) sum += exp(s[j] - m);
    double L = m + log(sum);
    double* oh = out + (int64_t)h * d;
    for (int i = 0; i < d; i++) oh[i] = 0.0;
    for (int64_t j = 0; j < n; j++) {
      double p = exp(s[j] - L);
      const double* vj = v + (j * Hkv + hk) * d;
      for (int i = 0; i < d; i++) oh[i] += p * vj[i];
    }
    lse[h] = L;
    free(s);
  }
}

/* Several independent queries, each with its own key list: query r uses keys
 * [off[r], off[r+1]) of k, v. Used for the pause queries of one compression,
 * whose key sets differ only in the causal pause part. */
void orc_attention_batch(const double* q, int64_t nq, int Hq, int Hkv, int d,
                         const int64_t* off, const double* k, const double* v, double* out,
                         double* lse) {
  for (int64_t r = 0; r < nq; r++) {
    int64_t a = off[r], b = off[r + 1];
    orc_attention(q + r * Hq * d, Hq, Hkv, d, b - a, k + a * Hkv * d, v + a * Hkv * d,
                  out + r * Hq * d, lse + r * Hq);
  }
}

/* Threads the oracle's parallel loops use from now on (timing on one core). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
