/* abk.h -- C ABI of the AbridgeKV attention hot path for MI355X (gfx950).
 *
 * What the library computes (sources are the pages on AbridgeKV, arXiv
 * 2610.20641):
 *  - Generated text is written in blocks of C tokens. When a block completes,
 *    K learned pause tokens attend to it and their per-layer KV entries become
 *    the block's "code rows"; then the block's raw KV rows are freed
 *    (abstract; figure captions, Fig. 1(a)).
 *  - The resident cache of a sequence at layer l is the prompt, quota[l] code
 *    rows per finished block, and the open block's raw rows (AI Radio
 *    transcript; news write-up, second and third details). Each layer has a
 *    fixed budget; rows a layer does not keep are never allocated.
 *  - Pause token k of block b is placed at RoPE position
 *    P + b*C + bitrev(k)*C/K inside the block it replaces (Fig. 2(b)).
 *  - Text tokens attend to the prompt, earlier code rows and causally to their
 *    own block; pause tokens attend to the prompt, earlier code rows, their
 *    whole block and causally to earlier pause tokens (Fig. 2(a)).
 *
 * Conventions for every call:
 *  - Device buffers (q/k/v/out/lse and the pages) are plain device pointers;
 *    the caller owns its buffers, the pool owns pages, tables and workspace.
 *  - Row layouts are contiguous, row-major, in the pool's dtype unless stated.
 *    Keys and queries are given before RoPE; the library rotates them
 *    (rotate-half, angle pos * rope_base^(-2i/d)) in fp64 from an fp64
 *    cos/sin table and rounds the result once to the pool dtype: the stored
 *    key row, and the query the scores take. Values are stored as given.
 *  - All device work is enqueued on the stream given at creation; calls
 *    return without synchronising unless stated. Host bookkeeping updates
 *    synchronously.
 *  - Every check happens before anything is enqueued: a call that returns an
 *    error has enqueued nothing and changed no state. abk_last_error() gives
 *    the reason (thread-local text).
 *  - One host thread per pool.
 *  - Scores are q.k/sqrt(d), accumulated in fp32 from the rounded operands;
 *    softmax runs in fp32; lse is the natural log of the sum of exp(score)
 *    (so out = sum exp(score - lse) v).
 */
#ifndef ABK_H
#define ABK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABK_OK = 0,
  ABK_ERR_INVALID_ARG = 1,  /* bad pointer, size, id or configuration */
  ABK_ERR_OUT_OF_PAGES = 2, /* not enough free pages or sequence slots */
  ABK_ERR_BAD_STATE = 3,    /* call out of protocol order (see each call) */
  ABK_ERR_HIP = 4,          /* a HIP runtime call failed */
  ABK_ERR_UNSUPPORTED = 5   /* valid but not built (shape/dtype), or host-only pool */
} abk_status;

typedef enum { ABK_F32 = 0, ABK_BF16 = 1 } abk_dtype;

typedef struct abk_pool abk_pool; /* opaque; owned by the library */

typedef struct {
  int32_t num_layers;   /* L */
  int32_t num_q_heads;  /* Hq; a multiple of num_kv_heads (GQA group g = Hq/Hkv in 1,2,4,8) */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d in {16, 64, 128} */
  int32_t block_tokens; /* C; a multiple of page_rows */
  int32_t num_pause;    /* K pause tokens per compression; a power of two dividing C */
  const int32_t* layer_quota; /* [L] code rows kept per block, 0 <= quota <= pause count (copied) */
  const int32_t* layer_pause; /* optional [L] pause tokens run at each layer (power of two,
                                 >= quota, divides C); NULL = num_pause at every layer */
  int32_t page_rows;    /* rows per page, 1..64 */
  int32_t max_seqs;     /* sequence slots */
  int64_t pool_bytes;   /* device bytes for K and V pages together */
  int32_t max_position; /* positions must stay below this (sizes the RoPE table) */
  int32_t dtype;        /* abk_dtype of pages, q/k/v and out */
  double rope_base;     /* e.g. 1e6 */
  int32_t compress;     /* 1: AbridgeKV; 0: full-KV, blocks never close */
  int32_t host_only;    /* 1: bookkeeping only (no device memory, no kernels; data
                           pointers are ignored) -- for capacity planning and tests */
  int32_t decode_split_rows; /* decode schedule: 0 = automatic (persistent, equal work per
                                workgroup where the shape allows, else 512-row splits);
                                > 0 = fixed split-KV work items of this many rows (whole
                                pages) */
  const int32_t* head_quota; /* optional [L][Hkv] code rows kept per block by each (layer,
                                KV head), 0 <= quota <= the layer's pause count (copied);
                                NULL = layer_quota for every head. Per-head quotas vary
                                the budget head by head (figure captions, Fig. 7: the cost
                                of halving one (layer, KV head)'s quota; AI Radio
                                transcript: a per-head schedule). With them, every (layer
                                l, KV head h) has its own rows and page table: the pool's
                                pages hold one KV head, and the `layer` argument of
                                abk_seq_query, abk_export_layout and abk_read_rows names
                                the pair as l * Hkv + h (rows [n][1][d]). The hot-path
                                calls keep their model-layer arguments and tensor
                                layouts; abk_blockmask_attention gives each KV head's
                                queries that head's own kept code rows. */
  const int64_t* budget_pool_pages; /* optional: a separate page pool per budget level (AI
                                Radio transcript: the serving engine keeps one page pool
                                per budget level). A level is one distinct quota value
                                (of layer_quota, or of head_quota when given), in
                                ascending order; entry k is the page count of level k's
                                pool, which holds page ids [sum of the earlier counts,
                                + entry k). Every (sequence, layer) takes its pages from
                                its level's pool only, lowest free id first, and a call
                                fails with OUT_OF_PAGES when any level it needs is short.
                                The counts must sum to at most the pages pool_bytes gives
                                (the rest stay unused). NULL = one pool for all levels. */
} abk_pool_config;

typedef struct {
  int32_t prompt_len;    /* P */
  int32_t generated;     /* rows appended at this layer (G) */
  int32_t blocks_done;   /* blocks compressed and freed */
  int32_t open_rows;     /* raw rows of the open block at this layer */
  int32_t resident_rows; /* P + blocks_done*quota + open (compress); P + G (full-KV) */
  int32_t n_pages;       /* pages this (sequence, layer) holds */
} abk_seq_info;

/* Create a pool: page storage, per-(sequence, layer) page tables, RoPE table.
 * Each layer has its own budget of code rows per finished block, layer_quota
 * (news write-up, the second of its three details, and figure captions,
 * Fig. 6(b): the six most valuable layers keep 256 rows, the twelve least
 * valuable 64, the rest 128, a mean of 128). A (sequence, layer) holds the
 * prompt, its code rows and the open block's raw rows (AI Radio transcript:
 * the resident cache, and a fixed budget per layer whose unkept rows are
 * never allocated), in two page lists: persistent (prompt, then code rows)
 * and open. Page layout: K pages [page][kv_head][page_rows][d] and V pages
 * likewise, plus an int32 position per (page, row). hip_stream: a hipStream_t
 * (NULL = default stream). Errors: INVALID_ARG (config), HIP (allocation). */
abk_status abk_pool_create(const abk_pool_config* cfg, void* hip_stream, abk_pool** out);
/* Synchronises the stream, then frees everything the pool owns. */
abk_status abk_pool_destroy(abk_pool* p);

/* Open a sequence with a prompt of prompt_len tokens: takes the lowest free
 * slot and reserves ceil(P/page_rows) persistent pages in every layer (layers
 * ascending, lowest page ids first). Errors: OUT_OF_PAGES (no slot or pages). */
abk_status abk_seq_create(abk_pool* p, int32_t prompt_len, int32_t* seq_id);
/* Return every page of the sequence and its slot. Enqueues nothing. */
abk_status abk_seq_release(abk_pool* p, int32_t seq_id);

/* Write the prompt rows of one layer: k, v [P, Hkv, d] device, k pre-RoPE,
 * row i at position i. BAD_STATE once generation has started at that layer. */
abk_status abk_write_prompt(abk_pool* p, int32_t seq_id, int32_t layer, const void* k,
                            const void* v);

/* Append the current token of each sequence at one layer. k, v
 * [n, Hkv, d] device (k pre-RoPE); the row lands at position P + G (G counted
 * before the call) in the open block (compress) or after the persistent rows
 * (full-KV); a new page is taken when the row starts one. seq_ids: host array
 * of n distinct ids. BAD_STATE if the prompt is not written, this layer is
 * ahead of the others, or (compress) the open block already holds C rows. */
abk_status abk_append_kv(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                         const void* k, const void* v);

/* GQA decode attention of the current token of each sequence at one layer,
 * over its resident rows: the prompt, the code rows that stand in for freed
 * blocks, and the open block (arXiv abstract: later tokens attend to the pause
 * tokens' entries in place of the freed block; figure captions, Fig. 2(a)).
 * Long chain-of-thought decoding is bound by reading this cache (arXiv
 * abstract), so the call streams each resident row once, split over the
 * device, and merges the splits (the split-KV partials and their combine).
 * q [n, Hq, d] device, pre-RoPE, rotated at position P + G - 1; query head h
 * reads KV head h / (Hq/Hkv). out [n, Hq, d] (pool dtype), lse [n, Hq] fp32.
 * BAD_STATE unless the current token is appended at this layer and the layer
 * is not between compression and free. */
abk_status abk_decode_attention(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                                const void* q, void* out, float* lse);

/* abk_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same checks, schedule and kernels, with the split partials
 * in a fixed device array of 32 MiB per GPU (kNoAllocScratchBytes) instead of
 * the pool's workspace. It calls no hipMalloc, hipFree or stream
 * synchronisation, and its results equal abk_decode_attention's. Every call on
 * one GPU shares that array: calls that overlap on one GPU (other streams,
 * other pools, other threads) race and must be ordered by the caller. A call
 * whose partials would exceed the array is refused before anything is
 * enqueued (UNSUPPORTED; the bench's 22-sequence, 36-layer step needs about
 * 6 MB per call). Other errors as for abk_decode_attention. */
abk_status abk_decode_attention_noalloc(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                                        const void* q, void* out, float* lse);

/* The append and the decode in one call: append the current token (k, v as for
 * abk_append_kv) and decode with q (as for abk_decode_attention) at one layer.
 * The result equals the two calls in sequence. For bf16 pools with d = 128,
 * four query heads per KV head, 64-row pages and the automatic schedule it is
 * one decode launch that also writes the new row (plus the split-merge
 * launch), saving the append launch per layer; other configurations issue the
 * two steps. Errors as for the two calls; on the fused path every check
 * happens before anything changes. */
abk_status abk_append_decode(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                             const void* k, const void* v, const void* q, void* out, float* lse);

/* Compress the completed open block b of each sequence at one layer: the
 * pause tokens attend to the block and their entries become its code rows
 * (figure captions, Fig. 1(a)), under the block mask of Fig. 2(a), at the
 * in-block positions of Fig. 2(b); the layer keeps the first quota[layer] of
 * them (news write-up, second detail). q_pause [n, Kp, Hq, d], k_pause and v_pause [n, Kp, Hkv, d] device,
 * pre-RoPE (Kp = the layer's pause count). Pause k is rotated at
 * P + b*C + bitrev(k)*C/Kp and attends to the prompt, the retained code rows of
 * earlier blocks, all C rows of block b, and pause keys j <= k. out [n, Kp, Hq,
 * d], lse [n, Kp, Hq] fp32. Then the rows k < quota[layer] (rotated key, value,
 * position) are appended to the layer's persistent rows in k order.
 * BAD_STATE unless the open block holds exactly C rows at this layer and was
 * not yet compressed there; BAD_STATE in full-KV mode. */
abk_status abk_compress_block(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                              const void* q_pause, const void* k_pause, const void* v_pause,
                              void* out, float* lse);

/* After every layer is compressed, return the open block's pages of every
 * layer to the free list and start the next block: once the pause tokens have
 * encoded a block, its raw cache is freed (arXiv abstract; figure captions,
 * Fig. 1(a)), so a sequence's cache falls at each compression (Fig. 1(b)). BAD_STATE unless every layer of every sequence is
 * compressed; BAD_STATE in full-KV mode. */
abk_status abk_free_block(abk_pool* p, int32_t n, const int32_t* seq_ids);

/* Host-side counters of one (sequence, layer). */
abk_status abk_seq_query(const abk_pool* p, int32_t seq_id, int32_t layer, abk_seq_info* out);

/* Read back the device page table (persistent pages, then open pages) and the
 * stored position of every resident row, in row order (host buffers).
 * Synchronises the stream. In a host-only pool returns the host mirror.
 * INVALID_ARG if a capacity is too small. */
abk_status abk_export_layout(const abk_pool* p, int32_t seq_id, int32_t layer, int32_t* page_ids,
                             int32_t cap_pages, int32_t* positions, int32_t cap_rows);

/* Copy resident rows [row0, row0 + nrows) of (sequence, layer) in row order
 * into device buffers k_out, v_out [nrows, Hkv, d] (keys as stored, i.e.
 * rotated). Enqueued on the stream. */
abk_status abk_read_rows(const abk_pool* p, int32_t seq_id, int32_t layer, int32_t row0,
                         int32_t nrows, void* k_out, void* v_out);

/* Block-mask prefill (the training-forward attention of arXiv 2610.20641,
 * Fig. 2(a) of its figure captions), one layer of one sequence. The sequence
 * is laid out in training order: prompt_len prompt rows, then for each block
 * its C text rows followed, when the block is complete (text_tokens counts
 * all text tokens; blocks b < text_tokens / C are complete), by the layer's
 * Kp pause rows; T = prompt_len + text_tokens + (text_tokens / C) * Kp rows
 * (no pause rows when compression is off). q [T, Hq, d], k/v [T, Hkv, d]:
 * device, pool dtype, pre-RoPE; every row is rotated at its own position
 * (prompt i; text j at prompt_len + j; pause k of block b at prompt_len + b C
 * + bitrev(k) C/Kp, Fig. 2(b)), keys rounded once to the pool dtype like
 * stored keys. Each row attends, with the layer's quota, to what the mask
 * shows it: prompt rows causally to the prompt; text rows to the prompt, the
 * kept code rows (pause k < quota) of earlier blocks and their own block's
 * text causally; pause rows to the same plus their whole block and their
 * block's pause rows up to their own. Compression off: plain causal
 * attention. out [T, Hq, d] (pool dtype) and lse [T, Hq] fp32 (natural log),
 * caller-owned. Uses the pool's stream, RoPE table and a library-owned
 * staging buffer (grown on demand); reads and writes no sequence state.
 * INVALID_ARG for a bad layer, negative lengths or prompt_len + text_tokens >
 * max_position; UNSUPPORTED unless the pool is bf16 with d = 128 and four
 * query heads per KV head. */
abk_status abk_blockmask_attention(abk_pool* p, int32_t layer, int32_t prompt_len, int32_t text_tokens,
                                   const void* q, const void* k, const void* v, void* out, float* lse);

/* Prompt prefill into the pool, one layer: abk_write_prompt(seq_id, layer, k,
 * v) followed by the prompt's causal attention (abk_blockmask_attention of the
 * sequence's P prompt rows and no text). q [P, Hq, d] pre-RoPE, k/v [P, Hkv,
 * d] as for abk_write_prompt; out [P, Hq, d] (pool dtype), lse [P, Hq] fp32,
 * caller-owned, device. Errors as for the two calls, all checked before
 * anything is written: INVALID_ARG (unknown sequence, bad layer, NULL
 * pointers with P > 0), UNSUPPORTED (the block-mask prefill's shapes),
 * BAD_STATE (generation has started at that layer). */
abk_status abk_prefill_prompt(abk_pool* p, int32_t seq_id, int32_t layer, const void* q, const void* k,
                              const void* v, void* out, float* lse);

/* Occupancy of one budget level's page pool (the AI Radio episode on
 * AbridgeKV: the serving engine keeps a separate pool of pages for each
 * budget level; pools are configured by abk_pool_config.budget_pool_pages).
 * Level `level` is 0 .. levels-1 in ascending quota order; with no separate
 * pools, level 0 is the one pool and *quota is -1. Writes its quota value,
 * pages in use and pages free (host counters, no stream work); *levels
 * receives the number of levels, also when `level` is out of range. Any
 * output pointer may be NULL. Errors: INVALID_ARG (NULL pool, level out of
 * range). */
abk_status abk_budget_pool_stats(const abk_pool* p, int32_t level, int32_t* levels, int32_t* quota,
                                 int64_t* pages_used, int64_t* pages_free);

/* Pool-wide counters (host, no stream work): pages in use and free over all
 * levels; resident_bytes = K+V bytes of resident rows. */
abk_status abk_pool_stats(const abk_pool* p, int64_t* pages_used, int64_t* pages_free,
                          int64_t* resident_bytes);

/* Bulk-build a fresh sequence's state after `generated` tokens with synthetic
 * rows: every completed block except the last token's is compressed and
 * freed. Row values are the seeded N(0,1) generator of the synth module (keyed
 * by seed, layer and token identity), rounded to the pool dtype; keys are
 * rotated at the row's position as by append/compress. Pages are taken per
 * layer ascending, persistent before open. BAD_STATE unless the sequence is
 * fresh (no prompt written, nothing appended). */
abk_status abk_synth_fill(abk_pool* p, int32_t seq_id, int32_t generated, uint64_t seed);

/* Test support: make a later workspace allocation of the pool fail with
 * ABK_ERR_HIP, as a failed hipMalloc or hipHostMalloc would. The call that
 * needs to grow a workspace after `after` more successful growths gets the
 * error; -1 turns the hook off. It checks that a call which fails there has
 * changed no state (the workspace is sized before any bookkeeping). Errors:
 * INVALID_ARG (NULL pool, after < -1). */
abk_status abk_debug_fail_allocs(abk_pool* p, int32_t after);

/* Thread-local text for the last non-OK status of this thread. */
const char* abk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ABK_H */
