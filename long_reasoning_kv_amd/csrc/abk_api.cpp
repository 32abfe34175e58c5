// C ABI of the AbridgeKV attention hot path (declared in include/abk.h).
//
// Each call: check arguments, let the host pool validate the protocol and do
// its bookkeeping (nothing changes on failure), then enqueue the device work
// on the pool's stream. Hot-path calls (append, decode, free) pass their
// per-call data in kernel arguments; the others upload a small descriptor
// through a ring of pinned host buffers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <climits>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/abk.h"
#include "kernels.h"
#include "pool.h"

namespace {

thread_local std::string g_err;

abk_status set_err(abk_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

abk_status from_host(abk::Status st, const std::string& msg) {
  return set_err((abk_status)st, msg);
}

#define ABK_HIP(call)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess)                                                                \
      return set_err(ABK_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));    \
  } while (0)

constexpr int kRing = 8;

struct PinnedSlot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

}  // namespace

struct abk_pool {
  abk::HostPool host;
  abk::Shape shape;  // as the host pool and the kernels see it (per-head quotas: see hs)
  // Per-head quotas: hs = the model's KV heads, and every (layer l, KV head h)
  // is layer l * hs + h of the pool, with one KV head (pages of one head, g
  // query heads). Otherwise hs = 1.
  int32_t hs = 1;
  bool host_only = false;
  int32_t split_rows = 0;  // 0: automatic schedule; > 0: fixed split-KV work items of this many rows
  int32_t stream_wgs = 0;  // resident workgroups of the stream-K decode (0: not used)
  int32_t mfma_waves = 0;  // resident wavefronts of the MFMA decode (0: not used)
  int32_t cus = 0;         // compute units of the device
  hipStream_t stream = nullptr;
  abk::DevPool dev{};
  int32_t* quota_d = nullptr;
  int32_t* pause_d = nullptr;
  float* part = nullptr;
  size_t part_bytes = 0;
  void* kp_rot = nullptr;
  size_t kp_rot_bytes = 0;
  void* bm_stage = nullptr;  // block-mask prefill: staged keys/values, persistent rows
  size_t bm_stage_bytes = 0;
  void* desc = nullptr;
  size_t desc_bytes = 0;
  int32_t* export_d = nullptr;
  size_t export_ints = 0;
  PinnedSlot ring[kRing];
  int ring_next = 0;
  std::vector<int32_t> scratch;  // host staging for descriptors
  int32_t fail_allocs = -1;      // test hook: workspace allocations left before one fails (-1: off)
  float* noalloc_part = nullptr;  // the allocation-free decode's fixed workspace on this device
};

namespace {

// The test hook's count-down: true when this workspace allocation is the one
// made to fail.
bool injected_failure(abk_pool* p) {
  if (p->fail_allocs < 0) return false;
  if (p->fail_allocs-- > 0) return false;
  p->fail_allocs = -1;
  return true;
}

abk_status grow(abk_pool* p, void** buf, size_t* have, size_t need) {
  if (need <= *have) return ABK_OK;
  if (injected_failure(p)) return set_err(ABK_ERR_HIP, "workspace allocation failed (injected)");
  ABK_HIP(hipStreamSynchronize(p->stream));
  if (*buf) ABK_HIP(hipFree(*buf));
  *buf = nullptr;
  *have = 0;
  size_t cap = std::max(need, (size_t)1 << 20);
  ABK_HIP(hipMalloc(buf, cap));
  *have = cap;
  return ABK_OK;
}

// Make the next descriptor upload of up to `bytes` allocation-free: the device
// buffer and the next pinned slot of the ring are grown (the slot once its
// previous copy has finished). Calls that change host state reserve first, so
// that a failed allocation leaves the state as it was.
abk_status reserve_desc(abk_pool* p, size_t bytes) {
  if (bytes == 0) return ABK_OK;
  if (abk_status st = grow(p, &p->desc, &p->desc_bytes, bytes)) return st;
  PinnedSlot& s = p->ring[p->ring_next];
  if (s.pending) ABK_HIP(hipEventSynchronize(s.ev));
  s.pending = false;
  if (s.cap < bytes) {
    if (injected_failure(p)) return set_err(ABK_ERR_HIP, "pinned staging allocation failed (injected)");
    if (s.host) ABK_HIP(hipHostFree(s.host));
    s.host = nullptr;
    s.cap = 0;
    size_t cap = std::max(bytes * 2, (size_t)1 << 16);
    ABK_HIP(hipHostMalloc(&s.host, cap, hipHostMallocDefault));
    s.cap = cap;
  }
  if (!s.ev) ABK_HIP(hipEventCreateWithFlags(&s.ev, hipEventDisableTiming));
  return ABK_OK;
}

// Copy `bytes` of host data to the pool's device descriptor buffer, in stream
// order, through a pinned slot that is reused only after its copy finished.
abk_status upload_desc(abk_pool* p, const void* src, size_t bytes) {
  if (bytes == 0) return ABK_OK;
  if (abk_status st = reserve_desc(p, bytes)) return st;
  PinnedSlot& s = p->ring[p->ring_next];
  p->ring_next = (p->ring_next + 1) % kRing;
  std::memcpy(s.host, src, bytes);
  ABK_HIP(hipMemcpyAsync(p->desc, s.host, bytes, hipMemcpyHostToDevice, p->stream));
  ABK_HIP(hipEventRecord(s.ev, p->stream));
  s.pending = true;
  return ABK_OK;
}

abk_status check_pool(const abk_pool* p) {
  return p ? ABK_OK : set_err(ABK_ERR_INVALID_ARG, "pool is NULL");
}

size_t row_elems(const abk::Shape& s) { return (size_t)s.Hkv * s.D; }

// The model layer `layer` as pool layers [layer * hs, layer * hs + hs).
abk_status check_model_layer(const abk_pool* p, int32_t layer) {
  if (layer < 0 || layer >= p->shape.L / p->hs) return set_err(ABK_ERR_INVALID_ARG, "bad layer");
  return ABK_OK;
}

// Entries of a hot-path call: (sequence i, head j) at index i * hs + j, each a
// (sequence, pool layer) with its own page table. Kernels address an entry's
// metadata and page table through one combined index sid * L + pool layer
// with a device view whose layer count is 1 (flat_view).
struct Entries {
  std::vector<int32_t> sid, lay, cslot;
};
Entries entries(const abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids) {
  Entries e;
  const size_t m = (size_t)n * p->hs;
  e.sid.resize(m);
  e.lay.resize(m);
  e.cslot.resize(m);
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < p->hs; ++j) {
      const size_t x = (size_t)i * p->hs + j;
      e.sid[x] = seq_ids[i];
      e.lay[x] = layer * p->hs + j;
      e.cslot[x] = seq_ids[i] * p->shape.L + e.lay[x];
    }
  return e;
}
abk::DevPool flat_view(const abk_pool* p) {
  abk::DevPool d = p->dev;
  d.L = 1;
  return d;
}

}  // namespace

extern "C" {

const char* abk_last_error(void) { return g_err.c_str(); }

abk_status abk_pool_create(const abk_pool_config* cfg, void* hip_stream, abk_pool** out) {
  if (!cfg || !out) return set_err(ABK_ERR_INVALID_ARG, "cfg/out is NULL");
  *out = nullptr;
  if (cfg->num_layers < 1 || cfg->num_layers > 4096) return set_err(ABK_ERR_INVALID_ARG, "num_layers");
  if (!cfg->layer_quota) return set_err(ABK_ERR_INVALID_ARG, "layer_quota is NULL");
  abk::Shape s;
  s.L = cfg->num_layers;
  s.Hq = cfg->num_q_heads;
  s.Hkv = cfg->num_kv_heads;
  s.D = cfg->head_dim;
  s.C = cfg->block_tokens;
  s.pr = cfg->page_rows;
  s.max_seqs = cfg->max_seqs;
  s.max_position = cfg->max_position;
  s.dtype = cfg->dtype;
  s.compress = cfg->compress ? 1 : 0;
  s.rope_base = cfg->rope_base;
  s.quota.assign(cfg->layer_quota, cfg->layer_quota + s.L);
  if (cfg->layer_pause) s.pause.assign(cfg->layer_pause, cfg->layer_pause + s.L);
  else s.pause.assign(s.L, cfg->num_pause);
  if (s.Hkv < 1 || s.D < 1 || s.pr < 1 || (s.dtype != 0 && s.dtype != 1))
    return set_err(ABK_ERR_INVALID_ARG, "bad shape or dtype");
  int32_t hs = 1;
  if (cfg->head_quota) {
    // per-(layer, KV head) quotas: one pool layer per pair, one KV head each
    if (s.Hq < 1 || s.Hq % s.Hkv) return set_err(ABK_ERR_INVALID_ARG, "bad head counts");
    if ((int64_t)s.L * s.Hkv > 4096) return set_err(ABK_ERR_INVALID_ARG, "num_layers * num_kv_heads above 4096");
    hs = s.Hkv;
    std::vector<int32_t> q, k;
    for (int32_t l = 0; l < s.L; ++l)
      for (int32_t h = 0; h < hs; ++h) {
        q.push_back(cfg->head_quota[(size_t)l * hs + h]);
        k.push_back(s.pause[l]);
      }
    s.quota = q;
    s.pause = k;
    s.L *= hs;
    s.Hq /= hs;
    s.Hkv = 1;
  }
  if (cfg->budget_pool_pages) {
    std::vector<int32_t> lq = s.quota;
    std::sort(lq.begin(), lq.end());
    lq.erase(std::unique(lq.begin(), lq.end()), lq.end());
    s.level_pages.assign(cfg->budget_pool_pages, cfg->budget_pool_pages + lq.size());
  }
  const int64_t page_bytes = (int64_t)s.Hkv * s.pr * s.D * s.esize();
  s.num_pages = cfg->pool_bytes / (2 * page_bytes);
  abk_pool* p = new abk_pool();
  std::string e;
  if (abk::Status st = p->host.init(s, &e)) {
    delete p;
    return set_err((abk_status)st, e);
  }
  if (s.Hkv * s.D > 2048) {
    delete p;
    return set_err(ABK_ERR_UNSUPPORTED, "num_kv_heads * head_dim above 2048");
  }
  p->shape = s;
  p->hs = hs;
  p->host_only = cfg->host_only != 0;
  if (cfg->decode_split_rows < 0) {
    delete p;
    return set_err(ABK_ERR_INVALID_ARG, "decode_split_rows is negative");
  }
  p->split_rows = cfg->decode_split_rows;
  p->stream = (hipStream_t)hip_stream;
  if (p->host_only) {
    *out = p;
    return ABK_OK;
  }
  auto fail = [&](hipError_t err, const char* what) {
    abk_pool_destroy(p);
    return set_err(ABK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
  };
  hipError_t err;
  const size_t pages = (size_t)s.num_pages;
  const size_t tab_ints = (size_t)s.max_seqs * s.L * s.table_stride();
  const size_t meta_ints = (size_t)s.max_seqs * s.L * 4;
  const size_t rope_n = (size_t)s.max_position * (s.D / 2);
  abk::DevPool& d = p->dev;
  if ((err = hipMalloc(&d.kpool, pages * page_bytes))) return fail(err, "pages");
  if ((err = hipMalloc(&d.vpool, pages * page_bytes))) return fail(err, "pages");
  if ((err = hipMalloc(&d.pos, pages * s.pr * sizeof(int32_t)))) return fail(err, "positions");
  if ((err = hipMalloc(&d.ptab, tab_ints * sizeof(int32_t)))) return fail(err, "page table");
  if ((err = hipMalloc(&d.meta, meta_ints * sizeof(int32_t)))) return fail(err, "meta");
  double2* rope = nullptr;
  if ((err = hipMalloc(&rope, rope_n * sizeof(double2)))) return fail(err, "rope");
  d.rope = rope;
  if ((err = hipMalloc(&p->quota_d, s.L * sizeof(int32_t)))) return fail(err, "quota");
  if ((err = hipMalloc(&p->pause_d, s.L * sizeof(int32_t)))) return fail(err, "pause");
  p->export_ints = 4 + (size_t)s.table_stride() + s.max_position + s.C;
  if ((err = hipMalloc(&p->export_d, p->export_ints * sizeof(int32_t)))) return fail(err, "export");
  if ((err = hipMemset(d.kpool, 0, pages * page_bytes))) return fail(err, "memset");
  if ((err = hipMemset(d.vpool, 0, pages * page_bytes))) return fail(err, "memset");
  if ((err = hipMemset(d.pos, 0xff, pages * s.pr * sizeof(int32_t)))) return fail(err, "memset");
  if ((err = hipMemset(d.ptab, 0xff, tab_ints * sizeof(int32_t)))) return fail(err, "memset");
  if ((err = hipMemset(d.meta, 0, meta_ints * sizeof(int32_t)))) return fail(err, "memset");
  // RoPE (cos, sin) of the angles pos * base^(-2i/d), in fp64
  {
    std::vector<double2> h(rope_n);
    const int half = s.D / 2;
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(s.rope_base, -2.0 * i / s.D);
    for (int64_t pos = 0; pos < s.max_position; ++pos)
      for (int i = 0; i < half; ++i) {
        double th = (double)pos * inv[i];
        h[pos * half + i] = make_double2(std::cos(th), std::sin(th));
      }
    if ((err = hipMemcpy(rope, h.data(), rope_n * sizeof(double2), hipMemcpyHostToDevice)))
      return fail(err, "rope upload");
  }
  if ((err = hipMemcpy(p->quota_d, s.quota.data(), s.L * sizeof(int32_t), hipMemcpyHostToDevice)))
    return fail(err, "quota upload");
  if ((err = hipMemcpy(p->pause_d, s.pause.data(), s.L * sizeof(int32_t), hipMemcpyHostToDevice)))
    return fail(err, "pause upload");
  if ((err = hipDeviceSynchronize())) return fail(err, "init sync");
  // the allocation-free decode's workspace: its address on this device
  {
    void* ws = nullptr;
    if ((err = abk::noalloc_scratch(&ws))) return fail(err, "allocation-free workspace address");
    p->noalloc_part = (float*)ws;
  }
  {
    int dev = 0, cus = 0;
    if ((err = hipGetDevice(&dev))) return fail(err, "device");
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)))
      return fail(err, "device attributes");
    abk::DevPool probe = d;
    probe.pr = s.pr;
    probe.D = s.D;
    probe.dtype = s.dtype;
    p->cus = cus;
    if (abk::decode_mfma_supported(probe, s.Hq / s.Hkv))
      p->mfma_waves = cus * abk::decode_mfma_waves_per_cu();
    else if (abk::decode_stream_supported(probe, s.Hq / s.Hkv))
      p->stream_wgs = cus * abk::decode_stream_blocks_per_cu(probe);
  }
  d.L = s.L;
  d.Hkv = s.Hkv;
  d.D = s.D;
  d.pr = s.pr;
  d.tstride = s.table_stride();
  d.max_pers = s.max_pers_pages();
  d.C = s.C;
  d.dtype = s.dtype;
  *out = p;
  return ABK_OK;
}

abk_status abk_pool_destroy(abk_pool* p) {
  if (!p) return ABK_OK;
  if (!p->host_only) {
    (void)hipStreamSynchronize(p->stream);
    abk::DevPool& d = p->dev;
    for (void* b : {(void*)d.kpool, (void*)d.vpool, (void*)d.pos, (void*)d.ptab, (void*)d.meta,
                    (void*)d.rope, (void*)p->quota_d, (void*)p->pause_d, (void*)p->part,
                    p->kp_rot, p->bm_stage, p->desc, (void*)p->export_d})
      if (b) (void)hipFree(b);
    for (auto& s : p->ring) {
      if (s.host) (void)hipHostFree(s.host);
      if (s.ev) (void)hipEventDestroy(s.ev);
    }
  }
  delete p;
  return ABK_OK;
}

abk_status abk_seq_create(abk_pool* p, int32_t prompt_len, int32_t* seq_id) {
  if (abk_status st = check_pool(p)) return st;
  if (abk::Status st = p->host.seq_create(prompt_len, seq_id)) return from_host(st, p->host.err);
  return ABK_OK;
}

abk_status abk_seq_release(abk_pool* p, int32_t seq_id) {
  if (abk_status st = check_pool(p)) return st;
  if (abk::Status st = p->host.seq_release(seq_id)) return from_host(st, p->host.err);
  return ABK_OK;
}

abk_status abk_write_prompt(abk_pool* p, int32_t seq_id, int32_t layer, const void* k,
                            const void* v) {
  if (abk_status st = check_pool(p)) return st;
  if (p->host.check_seq(seq_id)) return set_err(ABK_ERR_INVALID_ARG, "unknown sequence id");
  if (abk_status st = check_model_layer(p, layer)) return st;
  const int32_t P = p->host.seq(seq_id).P;
  if (!p->host_only && P > 0 && (!k || !v)) return set_err(ABK_ERR_INVALID_ARG, "k/v is NULL");
  if (abk::Status st = p->host.write_prompt(seq_id, layer * p->hs, p->hs)) return from_host(st, p->host.err);
  if (p->host_only) return ABK_OK;
  const int32_t np = (P + p->shape.pr - 1) / p->shape.pr;
  const size_t hb = (size_t)p->shape.Hkv * p->shape.D * p->shape.esize();  // one pool layer's heads
  for (int32_t j = 0; j < p->hs; ++j) {
    const int32_t lv = layer * p->hs + j;
    const auto& pages = p->host.seq(seq_id).layers[lv].pers_pages;
    if (abk_status st = upload_desc(p, pages.data(), np * sizeof(int32_t))) return st;
    abk::PromptArgs a;
    a.P = flat_view(p);
    a.k = (const char*)k + j * hb;
    a.v = (const char*)v + j * hb;
    a.kv_stride = p->hs * p->shape.Hkv * p->shape.D;  // elements between the caller's rows
    a.pages = (const int32_t*)p->desc;
    a.slot = seq_id * p->shape.L + lv;
    a.layer = 0;
    a.prompt_len = P;
    ABK_HIP(abk::launch_prompt(a, p->stream));
  }
  return ABK_OK;
}

abk_status abk_append_kv(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                         const void* k, const void* v) {
  if (abk_status st = check_pool(p)) return st;
  if (abk_status st = check_model_layer(p, layer)) return st;
  if (!p->host_only && n > 0 && (!k || !v)) return set_err(ABK_ERR_INVALID_ARG, "k/v is NULL");
  std::vector<int32_t> new_page;
  if (abk::Status st = p->host.append(layer * p->hs, p->hs, n, seq_ids, &new_page))
    return from_host(st, p->host.err);
  if (p->host_only) return ABK_OK;
  const Entries e = entries(p, layer, n, seq_ids);
  const int32_t ne = (int32_t)e.sid.size();
  const size_t rb = row_elems(p->shape) * p->shape.esize();  // one entry's row
  for (int32_t c0 = 0; c0 < ne; c0 += abk::kMaxBatch) {
    const int32_t m = std::min(ne - c0, abk::kMaxBatch);
    abk::AppendArgs a;
    a.P = flat_view(p);
    a.k = (const char*)k + c0 * rb;
    a.v = (const char*)v + c0 * rb;
    a.layer = 0;
    a.n = m;
    a.compress = p->shape.compress;
    for (int32_t i = 0; i < m; ++i) {
      a.slot[i] = e.cslot[c0 + i];
      a.new_page[i] = new_page[c0 + i];
    }
    ABK_HIP(abk::launch_append(a, p->stream));
  }
  return ABK_OK;
}

namespace {

// MFMA decode schedule: equal runs of 32-row tiles per wavefront over the
// flattened (sequence, head, tile) work; a sequence's tiles cover its
// persistent rows, then its open rows. `before_append`: counts exclude the
// token a fused call is about to append (which the kernel handles itself), and
// a sequence with no rows yet gets one empty tile. Runs are lengthened where a
// head would otherwise span more than kMaxSplits of them (one long sequence
// among few heads).
abk_status mfma_schedule(abk_pool* p, const Entries& e, bool before_append,
                         std::vector<abk::StreamArgs>* chunks) {
  const abk::Shape& s = p->shape;
  constexpr int32_t TK = 32;
  const int32_t n = (int32_t)e.sid.size();
  chunks->clear();
  for (int32_t c0 = 0; c0 < n; c0 += abk::kMaxBatch) {
    const int32_t m = std::min(n - c0, abk::kMaxBatch);
    chunks->emplace_back();
    abk::StreamArgs& a = chunks->back();
    a.useg[0] = 0;
    for (int32_t i = 0; i < m; ++i) {
      const int32_t id = e.sid[c0 + i], lv = e.lay[c0 + i];
      const int32_t pers = p->host.seq(id).layers[lv].pers_rows;
      const int32_t open = p->host.open_rows(id, lv);
      int32_t units = (pers + TK - 1) / TK + (open + TK - 1) / TK;
      if (before_append && units == 0) units = 1;
      a.slot[i] = e.cslot[c0 + i];
      a.useg[i + 1] = a.useg[i] + units * s.Hkv;
    }
    const int32_t U = a.useg[m];
    const int32_t kMinUnits = 4;  // per wavefront, to amortise its set-up
    int32_t W = std::max(1, std::min(p->mfma_waves, (U + kMinUnits - 1) / kMinUnits));
    int32_t umax = 0;  // the longest head's tiles
    for (int32_t i = 0; i < m; ++i) umax = std::max(umax, (a.useg[i + 1] - a.useg[i]) / s.Hkv);
    // a head of u tiles spans at most ceil(u / T) + 1 runs
    const int32_t T = std::max((U + W - 1) / W, (umax + abk::kMaxSplits - 3) / (abk::kMaxSplits - 2));
    int32_t maxp = 1;
    for (int32_t i = 0; i < m; ++i) {
      const int32_t units = (a.useg[i + 1] - a.useg[i]) / s.Hkv;
      for (int32_t h = 0; h < s.Hkv; ++h) {
        const int32_t S = a.useg[i] + h * units;
        maxp = std::max(maxp, (S + units - 1) / T - S / T + 1);
      }
    }
    if (maxp > abk::kMaxSplits) return set_err(ABK_ERR_UNSUPPORTED, "too many partials per head");
    a.n = m;
    a.T = T;
    a.U = U;
    a.maxp = maxp;
  }
  return ABK_OK;
}

// Bytes of split partials the scheduled chunks need (the chunks run one after
// another on the stream and share the buffer); `fused`: a fused call's
// partial of the current token per head.
size_t mfma_part_bytes(const abk_pool* p, const std::vector<abk::StreamArgs>& chunks, bool fused) {
  const abk::Shape& s = p->shape;
  const int32_t G = s.Hq / s.Hkv;
  size_t need = 0;
  for (const auto& a : chunks)
    need = std::max(need, (size_t)a.n * s.Hkv * (a.maxp + (fused ? 1 : 0)) * G * (s.D + 2));
  return need * sizeof(float);
}

// Launch the scheduled chunks with partials in `part` (at least
// mfma_part_bytes); k/v/new_page non-null: fused append of the current token.
abk_status launch_mfma_chunks(abk_pool* p, const void* q, void* out, float* lse, const void* k, const void* v,
                              const int32_t* new_page, float* part, std::vector<abk::StreamArgs>* chunks) {
  const abk::Shape& s = p->shape;
  const size_t qb = (size_t)s.Hq * s.D * s.esize();
  const size_t kb = (size_t)s.Hkv * s.D * s.esize();
  for (size_t c = 0; c < chunks->size(); ++c) {
    abk::StreamArgs& a = (*chunks)[c];
    const int32_t c0 = (int32_t)c * abk::kMaxBatch;
    const int32_t W = (a.U + a.T - 1) / a.T;
    a.P = flat_view(p);
    a.q = (const char*)q + c0 * qb;
    a.out = (char*)out + c0 * qb;
    a.lse = lse + (size_t)c0 * s.Hq;
    a.part = part;
    a.layer = 0;
    a.compress = s.compress;
    a.fused = k != nullptr;
    a.k = k ? (const char*)k + c0 * kb : nullptr;
    a.v = v ? (const char*)v + c0 * kb : nullptr;
    for (int32_t i = 0; i < a.n; ++i) a.new_page[i] = new_page ? new_page[c0 + i] : -1;
    ABK_HIP(abk::launch_decode_mfma(a, W, p->stream));
  }
  return ABK_OK;
}

}  // namespace

namespace {

// The split partials of a decode call: the pool's buffer, grown to `bytes`,
// or, for the allocation-free entry point, the fixed device array `fixed` of
// `cap` bytes (a call that needs more is refused before anything is enqueued).
abk_status decode_part(abk_pool* p, size_t bytes, float* fixed, size_t cap, float** part) {
  if (fixed) {
    if (bytes > cap)
      return set_err(ABK_ERR_UNSUPPORTED, "split partials need " + std::to_string(bytes) +
                                              " bytes; the allocation-free decode holds " + std::to_string(cap));
    *part = fixed;
    return ABK_OK;
  }
  if (abk_status st = grow(p, (void**)&p->part, &p->part_bytes, bytes)) return st;
  *part = p->part;
  return ABK_OK;
}

// Decode attention of one layer (checks, schedule, launches) with the split
// partials as decode_part gives them.
abk_status decode_into(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids, const void* q, void* out,
                       float* lse, float* fixed, size_t cap) {
  if (abk_status st = check_pool(p)) return st;
  if (abk_status st = check_model_layer(p, layer)) return st;
  if (!p->host_only && n > 0 && (!q || !out || !lse))
    return set_err(ABK_ERR_INVALID_ARG, "q/out/lse is NULL");
  if (abk::Status st = p->host.check_decode(layer * p->hs, p->hs, n, seq_ids)) return from_host(st, p->host.err);
  if (p->host_only || n == 0) return ABK_OK;
  const abk::Shape& s = p->shape;
  const int32_t G = s.Hq / s.Hkv;
  const size_t qb = (size_t)s.Hq * s.D * s.esize();  // one entry's queries
  const Entries e = entries(p, layer, n, seq_ids);
  const int32_t ne = (int32_t)e.sid.size();
  float* part = nullptr;
  if (p->mfma_waves > 0 && p->split_rows == 0) {
    std::vector<abk::StreamArgs> chunks;
    if (abk_status st = mfma_schedule(p, e, false, &chunks)) return st;
    if (abk_status st = decode_part(p, mfma_part_bytes(p, chunks, false), fixed, cap, &part)) return st;
    return launch_mfma_chunks(p, q, out, lse, nullptr, nullptr, nullptr, part, &chunks);
  }
  if (p->stream_wgs > 0 && p->split_rows == 0) {
    // stream-K: equal runs of 32-row units over the flattened (sequence, head,
    // unit) work; every chunk is scheduled, and the partials sized, first
    const int32_t nq = s.pr / 32;
    std::vector<abk::StreamArgs> chunks;
    std::vector<int32_t> waves;
    size_t need = 0;
    for (int32_t c0 = 0; c0 < ne; c0 += abk::kMaxBatch) {
      const int32_t m = std::min(ne - c0, abk::kMaxBatch);
      chunks.emplace_back();
      abk::StreamArgs& a = chunks.back();
      a.fused = 0;
      a.compress = s.compress;
      a.k = a.v = nullptr;
      a.useg[0] = 0;
      for (int32_t i = 0; i < m; ++i) {
        const auto& lay = p->host.seq(e.sid[c0 + i]).layers[e.lay[c0 + i]];
        const int32_t units = (int32_t)(lay.pers_pages.size() + lay.open_pages.size()) * nq;
        a.slot[i] = e.cslot[c0 + i];
        a.useg[i + 1] = a.useg[i] + units * s.Hkv;
      }
      const int32_t U = a.useg[m];
      const int32_t kMinUnits = 8;  // per workgroup, to amortise its set-up
      int32_t W = std::max(1, std::min(p->stream_wgs, (U + kMinUnits - 1) / kMinUnits));
      int32_t umax = 0;  // the longest head's units; it spans at most ceil(u / T) + 1 runs
      for (int32_t i = 0; i < m; ++i) umax = std::max(umax, (a.useg[i + 1] - a.useg[i]) / s.Hkv);
      const int32_t T = std::max((U + W - 1) / W, (umax + abk::kMaxSplits - 3) / (abk::kMaxSplits - 2));
      W = (U + T - 1) / T;
      int32_t maxp = 1;
      for (int32_t i = 0; i < m; ++i) {
        const int32_t units = (a.useg[i + 1] - a.useg[i]) / s.Hkv;
        for (int32_t h = 0; h < s.Hkv; ++h) {
          const int32_t S = a.useg[i] + h * units;
          maxp = std::max(maxp, (S + units - 1) / T - S / T + 1);
        }
      }
      if (maxp > abk::kMaxSplits) return set_err(ABK_ERR_UNSUPPORTED, "too many partials per head");
      need = std::max(need, (size_t)m * s.Hkv * maxp * G * (s.D + 2) * sizeof(float));
      a.P = flat_view(p);
      a.q = (const char*)q + c0 * qb;
      a.out = (char*)out + c0 * qb;
      a.lse = lse + (size_t)c0 * s.Hq;
      a.layer = 0;
      a.n = m;
      a.T = T;
      a.U = U;
      a.maxp = maxp;
      waves.push_back(W);
    }
    if (abk_status st = decode_part(p, need, fixed, cap, &part)) return st;
    for (size_t c = 0; c < chunks.size(); ++c) {
      chunks[c].part = part;
      ABK_HIP(abk::launch_decode_stream(chunks[c], waves[c], p->stream));
    }
    return ABK_OK;
  }
  // pages per split-KV work item; widened when a sequence would need more
  // than kMaxSplits of them
  int32_t split_pages = std::max(1, (p->split_rows > 0 ? p->split_rows : 512) / s.pr);
  std::vector<int32_t> splits(ne);
  int32_t max_nvp = 0;
  for (int32_t i = 0; i < ne; ++i) {
    const auto& lay = p->host.seq(e.sid[i]).layers[e.lay[i]];
    splits[i] = (int32_t)(lay.pers_pages.size() + lay.open_pages.size());
    max_nvp = std::max(max_nvp, splits[i]);
  }
  split_pages = std::max(split_pages, (max_nvp + abk::kMaxSplits - 1) / abk::kMaxSplits);
  for (int32_t i = 0; i < ne; ++i) splits[i] = (splits[i] + split_pages - 1) / split_pages;
  // size the partials for the whole call first (growing synchronises)
  size_t need = 0;
  for (int32_t c0 = 0; c0 < ne; c0 += abk::kMaxBatch) {
    size_t t = 0;
    for (int32_t i = c0; i < std::min(ne, c0 + abk::kMaxBatch); ++i) t += splits[i];
    need = std::max(need, t);
  }
  if (abk_status st = decode_part(p, need * s.Hkv * G * (s.D + 2) * sizeof(float), fixed, cap, &part)) return st;
  for (int32_t c0 = 0; c0 < ne; c0 += abk::kMaxBatch) {
    const int32_t m = std::min(ne - c0, abk::kMaxBatch);
    abk::DecodeArgs a;
    a.P = flat_view(p);
    a.q = (const char*)q + c0 * qb;
    a.out = (char*)out + c0 * qb;
    a.lse = lse + (size_t)c0 * s.Hq;
    a.part = part;
    a.layer = 0;
    a.n = m;
    a.G = G;
    a.split_pages = split_pages;
    a.prefix[0] = 0;
    for (int32_t i = 0; i < m; ++i) {
      a.slot[i] = e.cslot[c0 + i];
      a.prefix[i + 1] = a.prefix[i] + splits[c0 + i];
    }
    ABK_HIP(abk::launch_decode(a, a.prefix[m], p->stream));
  }
  return ABK_OK;
}

}  // namespace

abk_status abk_decode_attention(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                                const void* q, void* out, float* lse) {
  return decode_into(p, layer, n, seq_ids, q, out, lse, nullptr, 0);
}

abk_status abk_decode_attention_noalloc(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                                        const void* q, void* out, float* lse) {
  if (abk_status st = check_pool(p)) return st;
  if (!p->host_only && !p->noalloc_part)
    return set_err(ABK_ERR_BAD_STATE, "the allocation-free workspace was not resolved at pool creation");
  return decode_into(p, layer, n, seq_ids, q, out, lse, p->noalloc_part, abk::kNoAllocScratchBytes);
}

abk_status abk_append_decode(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                             const void* k, const void* v, const void* q, void* out, float* lse) {
  if (abk_status st = check_pool(p)) return st;
  if (!p->host_only && n > 0 && (!k || !v || !q || !out || !lse))
    return set_err(ABK_ERR_INVALID_ARG, "k/v/q/out/lse is NULL");
  if (p->host_only || n == 0 || p->mfma_waves == 0 || p->split_rows != 0) {
    // other shapes and schedules: the two steps as separate launches
    if (abk_status st = abk_append_kv(p, layer, n, seq_ids, k, v)) return st;
    return abk_decode_attention(p, layer, n, seq_ids, q, out, lse);
  }
  if (abk_status st = check_model_layer(p, layer)) return st;
  if (abk::Status st = p->host.check_batch(n, seq_ids)) return from_host(st, p->host.err);
  const Entries e = entries(p, layer, n, seq_ids);
  std::vector<abk::StreamArgs> chunks;
  if (abk_status st = mfma_schedule(p, e, true, &chunks)) return st;
  // the workspace before the append changes any state
  if (abk_status st = grow(p, (void**)&p->part, &p->part_bytes, mfma_part_bytes(p, chunks, true))) return st;
  std::vector<int32_t> new_page;
  if (abk::Status st = p->host.append(layer * p->hs, p->hs, n, seq_ids, &new_page))
    return from_host(st, p->host.err);
  return launch_mfma_chunks(p, q, out, lse, k, v, new_page.data(), p->part, &chunks);
}

abk_status abk_compress_block(abk_pool* p, int32_t layer, int32_t n, const int32_t* seq_ids,
                              const void* q_pause, const void* k_pause, const void* v_pause,
                              void* out, float* lse) {
  if (abk_status st = check_pool(p)) return st;
  if (abk_status st = check_model_layer(p, layer)) return st;
  if (!p->host_only && n > 0 && (!q_pause || !k_pause || !v_pause || !out || !lse))
    return set_err(ABK_ERR_INVALID_ARG, "a pause/out/lse pointer is NULL");
  const abk::Shape& s = p->shape;
  const int32_t l0 = layer * p->hs;
  if (abk::Status st = p->host.check_compress(l0, p->hs, n, seq_ids)) return from_host(st, p->host.err);
  const int32_t Kp = s.pause[l0];
  const int32_t ne = n * p->hs;
  const int32_t npair = ne * s.Hkv;
  const int32_t G = s.Hq / s.Hkv;
  // Workspace sizes from the counts before the call (the descriptor: records,
  // launch order, then each entry's pages of its new code rows), grown before
  // the host pool changes so that a failed allocation changes nothing.
  size_t desc_ints = (size_t)ne * abk::kCompRec + npair;
  int32_t min_ntc = INT32_MAX;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < p->hs; ++j) {
      const int32_t pers = p->host.seq(seq_ids[i]).layers[l0 + j].pers_rows, qn = s.quota[l0 + j];
      if (qn > 0) desc_ints += (pers + qn - 1) / s.pr - pers / s.pr + 1;
      min_ntc = std::min(min_ntc, (pers + 63) / 64 + s.C / 64);
    }
  int32_t nsplit = 1, ntq = 0;
  const bool mfma = !p->host_only && abk::compress_mfma_supported(p->dev, G);
  if (mfma && n > 0) {
    // few sequences: split each query tile's context over several workgroups so
    // that about one per CU runs, keeping at least 4 context tiles per split
    ntq = (4 * Kp + abk::kCompressRows - 1) / abk::kCompressRows;
    const int32_t wgs = (npair + 7) / 8 * 8 * ntq;
    const int32_t target = std::max(1, p->cus);
    if (wgs < target) nsplit = std::max(1, std::min({(target + wgs - 1) / wgs, min_ntc / 4, 16}));
  }
  if (!p->host_only && n > 0) {
    if (abk_status st = grow(p, &p->kp_rot, &p->kp_rot_bytes, (size_t)npair * Kp * s.D * s.esize())) return st;
    if (nsplit > 1)
      if (abk_status st = grow(p, (void**)&p->part, &p->part_bytes,
                               (size_t)npair * ntq * nsplit * abk::kCompressRows * (s.D + 2) * sizeof(float)))
        return st;
    if (abk_status st = reserve_desc(p, desc_ints * sizeof(int32_t))) return st;
  }
  std::vector<abk::CompressPlan> plan;  // one per (sequence, head) entry
  if (abk::Status st = p->host.compress(l0, p->hs, n, seq_ids, &plan)) return from_host(st, p->host.err);
  if (p->host_only || n == 0) return ABK_OK;
  std::vector<int32_t>& d = p->scratch;
  // records, then the (entry, KV head) pairs in launch order: longest context
  // first, so that the short ones fill in behind the long ones at the end of
  // the launch; then the page lists
  d.assign((size_t)ne * abk::kCompRec + npair, 0);
  {
    std::vector<int32_t> ord(ne);
    for (int32_t i = 0; i < ne; ++i) ord[i] = i;
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) {
      return plan[x].pers_before > plan[y].pers_before;
    });
    int32_t* o = &d[(size_t)ne * abk::kCompRec];
    for (int32_t r = 0; r < ne; ++r)
      for (int32_t h = 0; h < s.Hkv; ++h) o[r * s.Hkv + h] = ord[r] * s.Hkv + h;
  }
  for (int32_t i = 0; i < ne; ++i) {
    int32_t* r = &d[(size_t)i * abk::kCompRec];
    r[0] = plan[i].slot * s.L + plan[i].layer;  // combined index (flat device view)
    r[1] = plan[i].block;
    r[2] = plan[i].pers_before;
    r[3] = p->host.seq(plan[i].slot).P;
    r[4] = (int32_t)d.size();
    r[5] = (int32_t)plan[i].pages.size();
    r[6] = plan[i].first_new;
    r[7] = plan[i].quota;
    d.insert(d.end(), plan[i].pages.begin(), plan[i].pages.end());
  }
  if (abk_status st = upload_desc(p, d.data(), d.size() * sizeof(int32_t))) return st;
  abk::CompressArgs a;
  a.P = flat_view(p);
  a.qp = q_pause;
  a.kp = k_pause;
  a.vp = v_pause;
  a.out = out;
  a.lse = lse;
  a.kp_rot = p->kp_rot;
  a.desc = (const int32_t*)p->desc;
  a.layer = 0;
  a.n = ne;
  a.hsplit = p->hs;
  a.Hq = s.Hq * p->hs;  // the caller's query heads
  a.G = G;
  a.Kp = Kp;
  a.log2Kp = abk::log2_exact(Kp);
  a.nsplit = nsplit;
  a.part = nsplit > 1 ? p->part : nullptr;
  ABK_HIP(abk::launch_compress(a, p->stream));
  return ABK_OK;
}

abk_status abk_free_block(abk_pool* p, int32_t n, const int32_t* seq_ids) {
  if (abk_status st = check_pool(p)) return st;
  if (abk::Status st = p->host.free_block(n, seq_ids)) return from_host(st, p->host.err);
  if (p->host_only) return ABK_OK;
  for (int32_t c0 = 0; c0 < n; c0 += abk::kMaxBatch) {
    abk::FreeArgs a;
    a.P = p->dev;
    a.n = std::min(n - c0, abk::kMaxBatch);
    for (int32_t i = 0; i < a.n; ++i) a.slot[i] = seq_ids[c0 + i];
    ABK_HIP(abk::launch_free(a, p->stream));
  }
  return ABK_OK;
}

abk_status abk_blockmask_attention(abk_pool* p, int32_t layer, int32_t prompt_len, int32_t text_tokens,
                                   const void* q, const void* k, const void* v, void* out, float* lse) {
  if (abk_status st = check_pool(p)) return st;
  if (abk_status st = check_model_layer(p, layer)) return st;
  const abk::Shape& s = p->shape;
  if (prompt_len < 0 || text_tokens < 0) return set_err(ABK_ERR_INVALID_ARG, "negative length");
  if ((int64_t)prompt_len + text_tokens > s.max_position)
    return set_err(ABK_ERR_INVALID_ARG, "positions reach max_position");
  // the model's KV heads and each one's quota (per-head quotas: pool layers
  // layer * hs + h)
  const int32_t Hkv = s.Hkv * p->hs, Hq = s.Hq * p->hs;
  if (Hkv > abk::kMaxPrefillHeads) return set_err(ABK_ERR_UNSUPPORTED, "block-mask prefill above 16 KV heads");
  std::vector<int32_t> qh(Hkv);
  for (int32_t h = 0; h < Hkv; ++h) qh[h] = s.quota[layer * p->hs + (p->hs > 1 ? h : 0)];
  const int32_t C = s.C, Kp = s.pause[layer * p->hs], qmax = *std::max_element(qh.begin(), qh.end());
  const bool comp = s.compress != 0;
  const int32_t nb = comp ? text_tokens / C : 0;  // complete blocks: followed by their pause rows
  const int64_t T64 = (int64_t)prompt_len + text_tokens + (int64_t)nb * Kp;
  if (T64 > (1 << 30)) return set_err(ABK_ERR_INVALID_ARG, "sequence too long");
  const int32_t T = (int32_t)T64;
  if (!(s.dtype == 1 && s.D == 128 && s.Hq == 4 * s.Hkv))
    return set_err(ABK_ERR_UNSUPPORTED, "block-mask prefill needs bf16, d = 128, four query heads per KV head");
  if (T == 0) return ABK_OK;
  if (!p->host_only && (!q || !k || !v || !out || !lse))
    return set_err(ABK_ERR_INVALID_ARG, "q/k/v/out/lse is NULL");
  if (p->host_only) return ABK_OK;

  // query tiles of up to kBmTokens tokens of one kind in one block; per KV
  // head, a text or pause tile sees nA = prompt + blk * that head's quota
  // persistent rows
  struct Tile {
    int32_t kind, row0, ntok, tok0, bstart, nB, blk;
    int64_t work;  // keys seen by its last query beyond the persistent rows
  };
  std::vector<Tile> tiles;
  const int32_t P0 = comp ? prompt_len : T;  // rows attended causally from the start
  for (int32_t t0 = 0; t0 < P0; t0 += abk::kBmTokens) {
    const int32_t n = std::min(abk::kBmTokens, P0 - t0);
    tiles.push_back({0, t0, n, t0, 0, 0, -1, t0 + n});
  }
  if (comp) {
    const int32_t nblk = (text_tokens + C - 1) / C;
    for (int32_t blk = 0; blk < nblk; ++blk) {
      const int32_t bstart = prompt_len + blk * (C + Kp), ctext = std::min(C, text_tokens - blk * C);
      for (int32_t i0 = 0; i0 < ctext; i0 += abk::kBmTokens) {
        const int32_t n = std::min(abk::kBmTokens, ctext - i0);
        tiles.push_back({1, bstart + i0, n, i0, bstart, i0 + n, blk, (int64_t)i0 + n});
      }
      if (blk < nb)
        for (int32_t j0 = 0; j0 < Kp; j0 += abk::kBmTokens) {
          const int32_t n = std::min(abk::kBmTokens, Kp - j0);
          tiles.push_back({2, bstart + C + j0, n, j0, bstart, C + j0 + n, blk, (int64_t)C + j0 + n});
        }
    }
  }
  // Workgroups of one (KV head, block) share blockIdx mod 8, i.e. one XCD and
  // its L2, since they read the same keys; each XCD's list runs heaviest first.
  const int32_t nblk_all = (comp ? (text_tokens + C - 1) / C : 0) + 1;
  std::vector<std::vector<std::pair<int64_t, std::array<int32_t, abk::kBmRec>>>> lists(8);
  for (int32_t h = 0; h < Hkv; ++h)
    for (const Tile& t : tiles) {
      const int32_t x = (h * nblk_all + (t.blk + 1)) % 8;
      const int32_t nA = t.kind == 0 ? 0 : prompt_len + t.blk * qh[h];
      lists[x].push_back({t.work + nA, {h, t.kind, t.row0, t.ntok, t.tok0, nA, t.bstart, t.nB, t.blk}});
    }
  size_t maxlen = 0;
  for (auto& l : lists) {
    std::stable_sort(l.begin(), l.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
    maxlen = std::max(maxlen, l.size());
  }
  std::vector<int32_t>& d = p->scratch;
  d.assign(maxlen * 8 * abk::kBmRec, 0);
  for (size_t j = 0; j < maxlen; ++j)
    for (int32_t x = 0; x < 8; ++x) {
      int32_t* r = &d[(j * 8 + x) * abk::kBmRec];
      if (j < lists[x].size())
        std::copy(lists[x][j].second.begin(), lists[x][j].second.end(), r);
      else
        r[0] = -1;  // no work
    }
  const int32_t nrec = (int32_t)(maxlen * 8);

  const int32_t npers = comp ? prompt_len + nb * qmax : T;
  const size_t row_bytes = (size_t)Hkv * s.D * s.esize();
  const size_t stage = 2 * (size_t)T * row_bytes, pers = comp ? 2 * (size_t)npers * row_bytes : 0;
  if (abk_status st = grow(p, &p->bm_stage, &p->bm_stage_bytes, stage + pers)) return st;
  if (abk_status st = upload_desc(p, d.data(), d.size() * sizeof(int32_t))) return st;
  abk::BlockMaskArgs a;
  a.P = p->dev;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.kst = p->bm_stage;
  a.vst = (char*)p->bm_stage + (size_t)T * row_bytes;
  a.kpers = comp ? (char*)p->bm_stage + stage : a.kst;
  a.vpers = comp ? (char*)p->bm_stage + stage + (size_t)npers * row_bytes : a.vst;
  a.desc = (const int32_t*)p->desc;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T = T;
  a.prompt = prompt_len;
  a.C = C;
  a.Kp = Kp;
  int32_t lg = 0;
  while ((1 << lg) < Kp) ++lg;
  a.log2Kp = lg;
  for (int32_t h = 0; h < abk::kMaxPrefillHeads; ++h) a.quota_h[h] = h < Hkv ? qh[h] : 0;
  a.npers = npers;
  a.compress = comp ? 1 : 0;
  ABK_HIP(abk::launch_blockmask(a, nrec, p->stream));
  return ABK_OK;
}

abk_status abk_prefill_prompt(abk_pool* p, int32_t seq_id, int32_t layer, const void* q, const void* k,
                              const void* v, void* out, float* lse) {
  if (abk_status st = check_pool(p)) return st;
  if (p->host.check_seq(seq_id)) return set_err(ABK_ERR_INVALID_ARG, "unknown sequence id");
  if (abk_status st = check_model_layer(p, layer)) return st;
  const abk::Shape& s = p->shape;
  if (!(s.dtype == 1 && s.D == 128 && s.Hq == 4 * s.Hkv))
    return set_err(ABK_ERR_UNSUPPORTED, "prompt prefill needs bf16, d = 128, four query heads per KV head");
  // the block-mask prefill's own checks, before the prompt is written
  if (s.Hkv * p->hs > abk::kMaxPrefillHeads)
    return set_err(ABK_ERR_UNSUPPORTED, "block-mask prefill above 16 KV heads");
  const int32_t P = p->host.seq(seq_id).P;
  if (!p->host_only && P > 0 && (!q || !out || !lse))
    return set_err(ABK_ERR_INVALID_ARG, "q/out/lse is NULL");
  // the rows into the pool (every check before anything changes), then the
  // prompt's causal attention from the same inputs
  if (abk_status st = abk_write_prompt(p, seq_id, layer, k, v)) return st;
  return abk_blockmask_attention(p, layer, P, 0, q, k, v, out, lse);
}

abk_status abk_seq_query(const abk_pool* p, int32_t seq_id, int32_t layer, abk_seq_info* out) {
  if (abk_status st = check_pool(p)) return st;
  if (!out) return set_err(ABK_ERR_INVALID_ARG, "out is NULL");
  if (p->host.check_seq(seq_id) || p->host.check_layer(layer))
    return set_err(ABK_ERR_INVALID_ARG, "unknown sequence or layer");
  const abk::SeqState& q = p->host.seq(seq_id);
  const abk::LayerState& lay = q.layers[layer];
  out->prompt_len = q.P;
  out->generated = lay.G;
  out->blocks_done = q.nb;
  out->open_rows = p->host.open_rows(seq_id, layer);
  out->resident_rows = p->host.resident_rows(seq_id, layer);
  out->n_pages = (int32_t)(lay.pers_pages.size() + lay.open_pages.size());
  return ABK_OK;
}

abk_status abk_export_layout(const abk_pool* cp, int32_t seq_id, int32_t layer, int32_t* page_ids,
                             int32_t cap_pages, int32_t* positions, int32_t cap_rows) {
  abk_pool* p = const_cast<abk_pool*>(cp);
  if (abk_status st = check_pool(p)) return st;
  if (p->host.check_seq(seq_id) || p->host.check_layer(layer))
    return set_err(ABK_ERR_INVALID_ARG, "unknown sequence or layer");
  const abk::LayerState& lay = p->host.seq(seq_id).layers[layer];
  const int32_t npages = (int32_t)(lay.pers_pages.size() + lay.open_pages.size());
  const int32_t rows = p->host.resident_rows(seq_id, layer);
  if ((npages > 0 && (!page_ids || cap_pages < npages)) || (rows > 0 && (!positions || cap_rows < rows)))
    return set_err(ABK_ERR_INVALID_ARG, "capacity too small");
  if (p->host_only) {
    int32_t j = 0;
    for (int32_t pg : lay.pers_pages) page_ids[j++] = pg;
    for (int32_t pg : lay.open_pages) page_ids[j++] = pg;
    for (int32_t r = 0; r < rows; ++r) positions[r] = (int32_t)p->host.row_position(seq_id, layer, r);
    return ABK_OK;
  }
  abk::ExportArgs a;
  a.P = p->dev;
  a.dst = p->export_d;
  a.slot = seq_id;
  a.layer = layer;
  ABK_HIP(abk::launch_export(a, p->stream));
  std::vector<int32_t> h(4 + npages + rows);
  ABK_HIP(hipMemcpyAsync(h.data(), p->export_d, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                         p->stream));
  ABK_HIP(hipStreamSynchronize(p->stream));
  if (h[0] + h[1] != rows || h[3] != npages)
    return set_err(ABK_ERR_BAD_STATE, "device layout disagrees with the host mirror");
  std::memcpy(page_ids, h.data() + 4, npages * sizeof(int32_t));
  std::memcpy(positions, h.data() + 4 + npages, rows * sizeof(int32_t));
  return ABK_OK;
}

abk_status abk_read_rows(const abk_pool* cp, int32_t seq_id, int32_t layer, int32_t row0,
                         int32_t nrows, void* k_out, void* v_out) {
  abk_pool* p = const_cast<abk_pool*>(cp);
  if (abk_status st = check_pool(p)) return st;
  if (p->host.check_seq(seq_id) || p->host.check_layer(layer))
    return set_err(ABK_ERR_INVALID_ARG, "unknown sequence or layer");
  const int32_t rows = p->host.resident_rows(seq_id, layer);
  if (row0 < 0 || nrows < 0 || (int64_t)row0 + nrows > rows)
    return set_err(ABK_ERR_INVALID_ARG, "rows out of range");
  if (p->host_only) return set_err(ABK_ERR_UNSUPPORTED, "host-only pool has no rows");
  if (nrows > 0 && (!k_out || !v_out)) return set_err(ABK_ERR_INVALID_ARG, "k_out/v_out is NULL");
  abk::ReadArgs a;
  a.P = p->dev;
  a.k_out = k_out;
  a.v_out = v_out;
  a.slot = seq_id;
  a.layer = layer;
  a.row0 = row0;
  a.nrows = nrows;
  ABK_HIP(abk::launch_read(a, p->stream));
  return ABK_OK;
}

abk_status abk_budget_pool_stats(const abk_pool* p, int32_t level, int32_t* levels, int32_t* quota,
                                 int64_t* pages_used, int64_t* pages_free) {
  if (abk_status st = check_pool(p)) return st;
  if (levels) *levels = p->host.levels();
  if (level < 0 || level >= p->host.levels()) return set_err(ABK_ERR_INVALID_ARG, "budget level out of range");
  const int64_t fr = p->host.level_free(level);
  if (quota) *quota = p->host.level_quota(level);
  if (pages_used) *pages_used = p->host.level_pages(level) - fr;
  if (pages_free) *pages_free = fr;
  return ABK_OK;
}

abk_status abk_debug_fail_allocs(abk_pool* p, int32_t after) {
  if (abk_status st = check_pool(p)) return st;
  if (after < -1) return set_err(ABK_ERR_INVALID_ARG, "after must be >= -1");
  p->fail_allocs = after;
  return ABK_OK;
}

abk_status abk_pool_stats(const abk_pool* p, int64_t* pages_used, int64_t* pages_free,
                          int64_t* resident_bytes) {
  if (abk_status st = check_pool(p)) return st;
  const int64_t fr = p->host.pages_free();
  if (pages_used) *pages_used = p->shape.num_pages - fr;
  if (pages_free) *pages_free = fr;
  if (resident_bytes)
    *resident_bytes = p->host.resident_rows_total() * 2 * (int64_t)row_elems(p->shape) * p->shape.esize();
  return ABK_OK;
}

abk_status abk_synth_fill(abk_pool* p, int32_t seq_id, int32_t generated, uint64_t seed) {
  if (abk_status st = check_pool(p)) return st;
  if (abk::Status st = p->host.fill(seq_id, generated)) return from_host(st, p->host.err);
  if (p->host_only) return ABK_OK;
  const abk::Shape& s = p->shape;
  const abk::SeqState& q = p->host.seq(seq_id);
  std::vector<int32_t>& d = p->scratch;
  d.assign((size_t)4 * s.L, 0);
  int32_t max_rows = 0;
  for (int32_t l = 0; l < s.L; ++l) {
    const auto& lay = q.layers[l];
    d[4 * l + 0] = (int32_t)d.size();
    d[4 * l + 1] = (int32_t)lay.pers_pages.size();
    d.insert(d.end(), lay.pers_pages.begin(), lay.pers_pages.end());
    d[4 * l + 2] = (int32_t)d.size();
    d[4 * l + 3] = (int32_t)lay.open_pages.size();
    d.insert(d.end(), lay.open_pages.begin(), lay.open_pages.end());
    max_rows = std::max(max_rows, p->host.resident_rows(seq_id, l));
  }
  if (abk_status st = upload_desc(p, d.data(), d.size() * sizeof(int32_t))) return st;
  abk::FillArgs a;
  a.P = p->dev;
  a.desc = (const int32_t*)p->desc;
  a.quota = p->quota_d;
  a.pause = p->pause_d;
  a.seed = seed;
  a.slot = seq_id;
  a.prompt_len = q.P;
  a.G = generated;
  a.nb = q.nb;
  a.compress = s.compress;
  a.hsplit = p->hs;
  ABK_HIP(abk::launch_fill(a, max_rows, p->stream));
  return ABK_OK;
}

}  // extern "C"
