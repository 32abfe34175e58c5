// Launch interface between the C ABI (abk_api.cpp) and the HIP kernels
// (pool_kernels.hip, decode.hip, compress.hip). Hot-path launches (append, decode, free) carry their
// per-call data by value in the kernel arguments and read the device-resident
// per-(sequence, layer) metadata and page tables, so no host-to-device copy
// sits between two layers. Rarer calls (prompt, compression, fills,
// inspection) read a small descriptor uploaded to `desc`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abk {

constexpr int kMaxBatch = 256;   // sequences per hot-path launch (larger batches are split)
constexpr int kMaxSplits = 256;  // split-KV work items per sequence (the host sizes splits to fit)

// Device view of a pool. Pages: K [page][Hkv][pr][D], V likewise; pos
// [page][pr]. ptab[(slot*L + l)*tstride + i]: persistent page i for
// i < max_pers, open page j at max_pers + j. meta[(slot*L + l)*4 + f]:
// f=0 persistent rows, f=1 open rows, f=2 position of the current token.
struct DevPool {
  void* kpool;
  void* vpool;
  int32_t* pos;
  int32_t* ptab;
  int32_t* meta;
  const double2* rope;  // [max_position][D/2] (cos, sin), fp64
  int32_t L, Hkv, D, pr, tstride, max_pers, C, dtype;
};

struct AppendArgs {
  DevPool P;
  const void* k;
  const void* v;
  int32_t layer, n, compress;
  int32_t slot[kMaxBatch];
  int32_t new_page[kMaxBatch];  // page taken for this row, or -1
};

struct DecodeArgs {
  DevPool P;
  const void* q;
  void* out;
  float* lse;
  float* part;  // split partials [work][Hkv][G][D + 2]
  int32_t layer, n, G, split_pages;
  int32_t slot[kMaxBatch];
  int32_t prefix[kMaxBatch + 1];  // work items of sequence i: [prefix[i], prefix[i+1])
};

// Persistent stream-K decode (bf16, d = 128, 4 query heads per KV head): the
// flattened work (sequence i, KV head h, 32-row unit) is cut into equal runs of
// T units, one per workgroup. useg[i] = first flattened unit of sequence i
// (its units for head h follow at useg[i] + h * units_i). A (sequence, head)
// whose units span workgroups wa..wb leaves partials in slots
// ((i * Hkv + h) * maxp + (w - wa)) for the merge kernel.
struct StreamArgs {
  DevPool P;
  const void* q;
  void* out;
  float* lse;
  float* part;  // [n][Hkv][maxp + fused][4][D + 2]
  // fused append (decode_mfma_kernel only): the current token's k, v [n][Hkv][D]
  // are written there and scored as one extra partial per head; counts in meta
  // are the ones before it, and decode_stream_merge_kernel advances them
  const void* k;
  const void* v;
  int32_t fused, compress;
  int32_t layer, n, T, U, maxp;
  int32_t slot[kMaxBatch];
  int32_t useg[kMaxBatch + 1];
  int32_t new_page[kMaxBatch];  // fused: page taken for the current row, or -1
};

struct FreeArgs {
  DevPool P;
  int32_t n;
  int32_t slot[kMaxBatch];
};

// Prompt write: rows 0..P-1 of (slot, layer); pages from desc. Row r's P.Hkv
// heads are read at k + r * kv_stride (elements).
struct PromptArgs {
  DevPool P;
  const void* k;
  const void* v;
  const int32_t* pages;  // ceil(P/pr) ids (device)
  int32_t slot, layer, prompt_len, kv_stride;
};

// Query rows (pause tokens x query heads of a KV head) per workgroup of the
// MFMA compression kernel.
constexpr int kCompressRows = 256;

// One compression record per entry in desc (ints): {slot, block, pers_before,
// prompt_len, pages_off, npages, first_new, quota}. An entry is a sequence
// (hsplit = 1) or one (sequence, KV head) of a pool with per-head quotas
// (hsplit = the caller's KV heads, the pool's P.Hkv = 1): entry i is then the
// caller's sequence i / hsplit, KV heads (i % hsplit) * P.Hkv + 0..P.Hkv-1.
// The caller's q/k/v/out/lse keep their [sequence][pause][head][D] layouts.
// The records are followed by the n * P.Hkv pairs (entry * P.Hkv + KV head) in
// the order the MFMA kernel launches them, then by the page lists.
constexpr int kCompRec = 8;
struct CompressArgs {
  DevPool P;
  const void* qp;        // [n / hsplit][Kp][Hq][D]
  const void* kp;        // [n / hsplit][Kp][P.Hkv * hsplit][D]
  const void* vp;
  void* out;
  float* lse;
  void* kp_rot;          // workspace [n][P.Hkv][Kp][D]: rotated pause keys
  const int32_t* desc;   // n records, the pairs in launch order, then page lists
  float* part;           // nsplit > 1: [n][P.Hkv][query tiles][nsplit][kCompressRows][D + 2] partials
  int32_t layer, n, hsplit, Hq, G, Kp, log2Kp;  // Hq: the caller's query heads
  int32_t nsplit;        // MFMA path: context splits per query tile (1 = none)
};

// Block-mask prefill of one sequence in training order (T rows: the prompt,
// then per block C text rows and, for complete blocks, Kp pause rows), one
// layer. The staging pass rotates every key once into kst [Hkv][T][D] (values
// into vst) and gathers the prompt and the kept code rows (pause k < quota of
// every complete block) into kpers/vpers [Hkv][npers][D]: the layer's
// persistent rows. With a quota per KV head, head h keeps pause k < quota_h[h]
// at rows [prompt + blk * quota_h[h] + k] of its [npers] slab (npers sized for
// the largest). The attention pass takes one workgroup per record of desc
// (kBmRec ints): {KV head (-1: none), kind (0 prompt, 1 text, 2 pause), first
// query row, query tokens (<= kBmTokens), index of the first query in its range
// (prompt, text-in-block or pause index), persistent rows it sees, first row
// of its block in kst, rows of the block it sees, block}.
constexpr int kBmRec = 9;
constexpr int kBmTokens = 64;  // query tokens per record (256 query rows)
constexpr int kMaxPrefillHeads = 16;
struct BlockMaskArgs {
  DevPool P;
  const void* q;   // [T][Hq][D] pre-RoPE
  const void* k;   // [T][Hkv][D] pre-RoPE
  const void* v;   // [T][Hkv][D]
  void* out;       // [T][Hq][D]
  float* lse;      // [T][Hq]
  void* kst;       // [Hkv][T][D]
  void* vst;       // [Hkv][T][D]
  void* kpers;     // [Hkv][npers][D] (the staging buffers themselves when compression is off)
  void* vpers;
  const int32_t* desc;
  int32_t Hq, Hkv, T, prompt, C, Kp, log2Kp, npers, compress;
  int32_t quota_h[kMaxPrefillHeads];  // code rows each KV head keeps per block
};

// Fill: desc holds per layer {pers_off, npers_pages, open_off, nopen_pages}
// then the page lists.
// Rows are keyed for the generator by the model's (layer, KV head): pool
// layer l with hsplit > 1 (per-head quotas) is layer l / hsplit, head l % hsplit.
struct FillArgs {
  DevPool P;
  const int32_t* desc;
  const int32_t* quota;  // [L] device
  const int32_t* pause;  // [L] device
  uint64_t seed;
  int32_t slot, prompt_len, G, nb, compress, hsplit;
};

// Gather rows [row0, row0+nrows) of (slot, layer) through the device page
// table into k_out, v_out [nrows][Hkv][D].
struct ReadArgs {
  DevPool P;
  void* k_out;
  void* v_out;
  int32_t slot, layer, row0, nrows;
};

// Export: writes {n_pers, n_open, qpos, npages, pages..., positions...}.
struct ExportArgs {
  DevPool P;
  int32_t* dst;
  int32_t slot, layer;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int32_t total_work, hipStream_t s);
// stream-K path: shapes it serves, workgroups per CU it keeps resident, launch
bool decode_stream_supported(const DevPool& P, int32_t G);
int32_t decode_stream_blocks_per_cu(const DevPool& P);
hipError_t launch_decode_stream(const StreamArgs& a, int32_t nwg, hipStream_t s);
// bf16, d = 128, four query heads per KV head, 64-row pages: MFMA decode with
// wavefront-level stream-K over 32-row tiles (U, T, useg in tiles; T per wavefront)
bool decode_mfma_supported(const DevPool& P, int32_t G);
int32_t decode_mfma_waves_per_cu();
hipError_t launch_decode_mfma(const StreamArgs& a, int32_t nwaves, hipStream_t s);  // + merge (always when fused)
hipError_t launch_free(const FreeArgs& a, hipStream_t s);
hipError_t launch_prompt(const PromptArgs& a, hipStream_t s);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
bool compress_mfma_supported(const DevPool& P, int32_t G);
hipError_t launch_fill(const FillArgs& a, int32_t max_rows, hipStream_t s);
// block-mask prefill (bf16, d = 128, four query heads per KV head): staging pass
// then one attention workgroup per descriptor record
bool blockmask_supported(const DevPool& P, int32_t G);
hipError_t launch_blockmask(const BlockMaskArgs& a, int32_t nrec, hipStream_t s);
hipError_t launch_read(const ReadArgs& a, hipStream_t s);
// Fixed device workspace of the allocation-free decode entry point: the split
// partials live in a file-scope device array of this many bytes, one per GPU,
// shared by every such call on that GPU. noalloc_scratch gives its address on
// the current device (resolved once per device; the address is what host code
// passes to kernels, never the array's name).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_export(const ExportArgs& a, hipStream_t s);

}  // namespace abk
