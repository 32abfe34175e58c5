// Host bookkeeping of the paged AbridgeKV cache (see pool.h).
#include "pool.h"

#include <algorithm>

namespace abk {

static int32_t cdiv(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

int32_t bitrev(int32_t k, int32_t nbits) {
  int32_t r = 0;
  for (int32_t i = 0; i < nbits; ++i) r = (r << 1) | ((k >> i) & 1);
  return r;
}

int32_t log2_exact(int32_t x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int32_t n = 0;
  while ((1 << n) != x) ++n;
  return n;
}

Status HostPool::init(const Shape& s, std::string* e) {
  auto bad = [&](const char* m) {
    *e = m;
    return kInvalidArg;
  };
  if (s.L < 1 || s.Hkv < 1 || s.Hq < 1 || s.Hq % s.Hkv) return bad("bad head counts");
  int32_t g = s.Hq / s.Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return bad("GQA group must be 1, 2, 4 or 8");
  if (s.D != 16 && s.D != 64 && s.D != 128) return bad("head_dim must be 16, 64 or 128");
  if (s.pr < 1 || s.pr > 64) return bad("page_rows must be in 1..64");
  if (s.C < 1 || s.C % s.pr) return bad("block_tokens must be a positive multiple of page_rows");
  if ((int32_t)s.quota.size() != s.L || (int32_t)s.pause.size() != s.L)
    return bad("layer tables missing");
  for (int32_t l = 0; l < s.L; ++l) {
    int32_t K = s.pause[l];
    if (log2_exact(K) < 0 || K > s.C || s.C % K) return bad("pause count must be a power of two dividing C");
    if (s.quota[l] < 0 || s.quota[l] > K) return bad("quota must be in 0..pause count");
  }
  if (s.max_seqs < 1 || s.max_position < 1) return bad("max_seqs and max_position must be positive");
  if (s.num_pages < 1 || s.num_pages > INT32_MAX) return bad("pool_bytes gives no pages (or too many)");
  if (!(s.rope_base > 0.0)) return bad("rope_base must be positive");
  if (s.dtype != 0 && s.dtype != 1) return bad("dtype must be ABK_F32 or ABK_BF16");
  // budget levels: one per distinct quota value when separate pools are asked for
  std::vector<int32_t> lq;
  if (!s.level_pages.empty()) {
    lq = s.quota;
    std::sort(lq.begin(), lq.end());
    lq.erase(std::unique(lq.begin(), lq.end()), lq.end());
    if (s.level_pages.size() != lq.size()) return bad("budget_pool_pages needs one count per distinct quota");
    int64_t tot = 0;
    for (int64_t n : s.level_pages) {
      if (n < 0) return bad("negative budget pool size");
      tot += n;
    }
    if (tot > s.num_pages) return bad("budget pools hold more pages than pool_bytes gives");
  } else {
    lq.assign(1, -1);
  }
  s_ = s;
  level_quota_ = lq;
  free_.assign(lq.size(), MinHeap());
  level_start_.assign(lq.size() + 1, 0);
  for (size_t k = 0; k < lq.size(); ++k)
    level_start_[k + 1] = level_start_[k] + (s.level_pages.empty() ? s.num_pages : s.level_pages[k]);
  for (size_t k = 0; k < lq.size(); ++k)
    for (int64_t p = level_start_[k]; p < level_start_[k + 1]; ++p) free_[k].push((int32_t)p);
  level_of_.assign(s.L, 0);
  if (!s.level_pages.empty())
    for (int32_t l = 0; l < s.L; ++l)
      level_of_[l] = (int32_t)(std::lower_bound(lq.begin(), lq.end(), s.quota[l]) - lq.begin());
  seqs_.assign(s.max_seqs, SeqState());
  for (int32_t i = 0; i < s.max_seqs; ++i) free_slots_.push(i);
  mark_.assign(s.max_seqs, 0);
  return kOk;
}

int32_t HostPool::take_page(int32_t l) {
  MinHeap& h = free_[level_of_[l]];
  int32_t p = h.top();
  h.pop();
  return p;
}

void HostPool::give_page(int32_t p) {
  const size_t k = std::upper_bound(level_start_.begin(), level_start_.end(), (int64_t)p) - level_start_.begin() - 1;
  free_[k].push(p);
}

int64_t HostPool::pages_free() const {
  int64_t t = 0;
  for (const auto& h : free_) t += (int64_t)h.size();
  return t;
}

Status HostPool::check_need(const std::vector<int64_t>& need, const char* what) {
  for (size_t k = 0; k < need.size(); ++k)
    if (need[k] > (int64_t)free_[k].size())
      return fail(kOutOfPages, std::string("not enough free pages ") + what +
                                   (free_.size() > 1 ? " in budget pool " + std::to_string(k) : std::string()));
  return kOk;
}

int32_t HostPool::gmin(const SeqState& q) const {
  int32_t m = INT32_MAX;
  for (const auto& x : q.layers) m = std::min(m, x.G);
  return m;
}

int32_t HostPool::gmax(const SeqState& q) const {
  int32_t m = 0;
  for (const auto& x : q.layers) m = std::max(m, x.G);
  return m;
}

int32_t HostPool::open_rows(int32_t id, int32_t l) const {
  const SeqState& q = seqs_[id];
  return s_.compress ? q.layers[l].G - q.nb * s_.C : 0;
}

int32_t HostPool::resident_rows(int32_t id, int32_t l) const {
  return seqs_[id].layers[l].pers_rows + open_rows(id, l);
}

int64_t HostPool::resident_rows_total() const {
  int64_t t = 0;
  for (int32_t i = 0; i < s_.max_seqs; ++i)
    if (seqs_[i].live)
      for (int32_t l = 0; l < s_.L; ++l) t += resident_rows(i, l);
  return t;
}

Status HostPool::check_seq(int32_t id) const {
  if (id < 0 || id >= s_.max_seqs || !seqs_[id].live) return kInvalidArg;
  return kOk;
}

Status HostPool::check_layer(int32_t l) const { return (l < 0 || l >= s_.L) ? kInvalidArg : kOk; }
Status HostPool::check_layers(int32_t l0, int32_t nl) const {
  return (nl < 1 || l0 < 0 || (int64_t)l0 + nl > s_.L) ? kInvalidArg : kOk;
}

Status HostPool::check_batch(int32_t n, const int32_t* ids) {
  if (n < 0) return fail(kInvalidArg, "negative batch size");
  if (n > 0 && !ids) return fail(kInvalidArg, "seq_ids is NULL");
  if (++stamp_ == 0) {
    std::fill(mark_.begin(), mark_.end(), 0);
    stamp_ = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (check_seq(ids[i])) return fail(kInvalidArg, "unknown sequence id " + std::to_string(ids[i]));
    if (mark_[ids[i]] == stamp_) return fail(kInvalidArg, "duplicate sequence id in batch");
    mark_[ids[i]] = stamp_;
  }
  return kOk;
}

Status HostPool::seq_create(int32_t P, int32_t* id) {
  if (!id) return fail(kInvalidArg, "seq_id is NULL");
  if (P < 0 || P > s_.max_position) return fail(kInvalidArg, "prompt length out of range");
  if (free_slots_.empty()) return fail(kOutOfPages, "no free sequence slot");
  std::vector<int64_t> need(levels(), 0);
  for (int32_t l = 0; l < s_.L; ++l) need[level_of_[l]] += cdiv(P, s_.pr);
  if (Status st = check_need(need, "for the prompt")) return st;
  int32_t sid = free_slots_.top();
  free_slots_.pop();
  SeqState& q = seqs_[sid];
  q = SeqState();
  q.live = true;
  q.P = P;
  q.layers.assign(s_.L, LayerState());
  for (int32_t l = 0; l < s_.L; ++l) {
    LayerState& lay = q.layers[l];
    for (int32_t i = 0; i < cdiv(P, s_.pr); ++i) lay.pers_pages.push_back(take_page(l));
    lay.pers_rows = P;
  }
  *id = sid;
  return kOk;
}

Status HostPool::seq_release(int32_t id) {
  if (check_seq(id)) return fail(kInvalidArg, "unknown sequence id");
  SeqState& q = seqs_[id];
  for (auto& lay : q.layers) {
    for (int32_t p : lay.pers_pages) give_page(p);
    for (int32_t p : lay.open_pages) give_page(p);
  }
  q = SeqState();
  free_slots_.push(id);
  return kOk;
}

Status HostPool::write_prompt(int32_t id, int32_t l0, int32_t nl) {
  if (check_seq(id)) return fail(kInvalidArg, "unknown sequence id");
  if (check_layers(l0, nl)) return fail(kInvalidArg, "bad layer");
  for (int32_t j = 0; j < nl; ++j)
    if (seqs_[id].layers[l0 + j].G != 0) return fail(kBadState, "prompt rewritten after generation began");
  for (int32_t j = 0; j < nl; ++j) seqs_[id].layers[l0 + j].prompt_written = true;
  return kOk;
}

Status HostPool::append(int32_t l0, int32_t nl, int32_t n, const int32_t* ids, std::vector<int32_t>* new_page) {
  if (check_layers(l0, nl)) return fail(kInvalidArg, "bad layer");
  if (Status st = check_batch(n, ids)) return st;
  std::vector<int64_t> need(levels(), 0);
  for (int32_t i = 0; i < n; ++i) {
    const SeqState& q = seqs_[ids[i]];
    const int32_t g0 = gmin(q);
    for (int32_t j = 0; j < nl; ++j) {
      const LayerState& lay = q.layers[l0 + j];
      if (!lay.prompt_written) return fail(kBadState, "prompt not written at this layer");
      if (lay.G != g0) return fail(kBadState, "layer is ahead of the current token");
      if ((int64_t)q.P + lay.G >= s_.max_position) return fail(kInvalidArg, "position reaches max_position");
      if (s_.compress) {
        int32_t op = lay.G - q.nb * s_.C;
        if (op >= s_.C) return fail(kBadState, "open block is full: compress and free it first");
        need[level_of_[l0 + j]] += (op % s_.pr == 0);
      } else {
        need[level_of_[l0 + j]] += (lay.pers_rows % s_.pr == 0);
      }
    }
  }
  if (Status st = check_need(need, "to append")) return st;
  new_page->assign((size_t)n * nl, -1);
  for (int32_t i = 0; i < n; ++i) {
    SeqState& q = seqs_[ids[i]];
    for (int32_t j = 0; j < nl; ++j) {
      LayerState& lay = q.layers[l0 + j];
      int32_t& np = (*new_page)[(size_t)i * nl + j];
      if (s_.compress) {
        if ((lay.G - q.nb * s_.C) % s_.pr == 0) {
          np = take_page(l0 + j);
          lay.open_pages.push_back(np);
        }
      } else {
        if (lay.pers_rows % s_.pr == 0) {
          np = take_page(l0 + j);
          lay.pers_pages.push_back(np);
        }
        lay.pers_rows += 1;
      }
      lay.G += 1;
    }
  }
  return kOk;
}

Status HostPool::check_decode(int32_t l0, int32_t nl, int32_t n, const int32_t* ids) {
  if (check_layers(l0, nl)) return fail(kInvalidArg, "bad layer");
  if (Status st = check_batch(n, ids)) return st;
  for (int32_t i = 0; i < n; ++i) {
    const SeqState& q = seqs_[ids[i]];
    for (int32_t j = 0; j < nl; ++j) {
      const LayerState& lay = q.layers[l0 + j];
      if (!lay.prompt_written || lay.G == 0 || lay.G != gmax(q))
        return fail(kBadState, "current token not appended at this layer");
      if (lay.compressed) return fail(kBadState, "block compressed at this layer but not freed");
    }
  }
  return kOk;
}

Status HostPool::check_compress(int32_t l0, int32_t nl, int32_t n, const int32_t* ids) {
  if (check_layers(l0, nl)) return fail(kInvalidArg, "bad layer");
  if (!s_.compress) return fail(kBadState, "compression is off (full-KV pool)");
  if (Status st = check_batch(n, ids)) return st;
  std::vector<int64_t> need(levels(), 0);
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < nl; ++j) {
      const int32_t l = l0 + j;
      const LayerState& lay = seqs_[ids[i]].layers[l];
      if (open_rows(ids[i], l) != s_.C) return fail(kBadState, "open block is not complete");
      if (lay.compressed) return fail(kBadState, "block already compressed at this layer");
      need[level_of_[l]] += cdiv(lay.pers_rows + s_.quota[l], s_.pr) - cdiv(lay.pers_rows, s_.pr);
    }
  return check_need(need, "for code rows");
}

Status HostPool::compress(int32_t l0, int32_t nl, int32_t n, const int32_t* ids, std::vector<CompressPlan>* plan) {
  if (Status st = check_compress(l0, nl, n, ids)) return st;
  plan->clear();
  for (int32_t i = 0; i < n; ++i) {
    SeqState& q = seqs_[ids[i]];
    for (int32_t j = 0; j < nl; ++j) {
      const int32_t l = l0 + j, qn = s_.quota[l];
      LayerState& lay = q.layers[l];
      CompressPlan cp;
      cp.slot = ids[i];
      cp.layer = l;
      cp.quota = qn;
      cp.block = q.nb;
      cp.pers_before = lay.pers_rows;
      cp.first_new = 0;
      int32_t have = cdiv(lay.pers_rows, s_.pr);
      int32_t want = cdiv(lay.pers_rows + qn, s_.pr);
      for (int32_t k = have; k < want; ++k) lay.pers_pages.push_back(take_page(l));
      if (qn > 0) {
        int32_t first = lay.pers_rows / s_.pr, last = (lay.pers_rows + qn - 1) / s_.pr;
        cp.pages.assign(lay.pers_pages.begin() + first, lay.pers_pages.begin() + last + 1);
        cp.first_new = have - first;
      }
      lay.pers_rows += qn;
      lay.compressed = true;
      plan->push_back(std::move(cp));
    }
  }
  return kOk;
}

Status HostPool::free_block(int32_t n, const int32_t* ids) {
  if (!s_.compress) return fail(kBadState, "compression is off (full-KV pool)");
  if (Status st = check_batch(n, ids)) return st;
  for (int32_t i = 0; i < n; ++i)
    for (const auto& lay : seqs_[ids[i]].layers)
      if (!lay.compressed) return fail(kBadState, "not every layer is compressed");
  for (int32_t i = 0; i < n; ++i) {
    SeqState& q = seqs_[ids[i]];
    for (auto& lay : q.layers) {
      for (int32_t p : lay.open_pages) give_page(p);
      lay.open_pages.clear();
      lay.compressed = false;
    }
    q.nb += 1;
  }
  return kOk;
}

Status HostPool::fill(int32_t id, int32_t G) {
  if (check_seq(id)) return fail(kInvalidArg, "unknown sequence id");
  if (G < 0) return fail(kInvalidArg, "negative length");
  SeqState& q = seqs_[id];
  for (const auto& lay : q.layers)
    if (lay.G || lay.prompt_written) return fail(kBadState, "fill needs a fresh sequence");
  if (G > 0 && (int64_t)q.P + G - 1 >= s_.max_position)
    return fail(kInvalidArg, "position reaches max_position");
  int32_t nb = (s_.compress && G > 0) ? (G - 1) / s_.C : 0;
  int32_t opn = s_.compress ? G - nb * s_.C : 0;
  std::vector<int64_t> need(levels(), 0);
  for (int32_t l = 0; l < s_.L; ++l) {
    int64_t r1 = q.P + (s_.compress ? (int64_t)nb * s_.quota[l] : G);
    need[level_of_[l]] += cdiv(r1, s_.pr) - cdiv(q.P, s_.pr) + cdiv(opn, s_.pr);
  }
  if (Status st = check_need(need, "for the fill")) return st;
  for (int32_t l = 0; l < s_.L; ++l) {
    LayerState& lay = q.layers[l];
    int32_t r1 = q.P + (s_.compress ? nb * s_.quota[l] : G);
    for (int32_t k = cdiv(q.P, s_.pr); k < cdiv(r1, s_.pr); ++k) lay.pers_pages.push_back(take_page(l));
    for (int32_t k = 0; k < cdiv(opn, s_.pr); ++k) lay.open_pages.push_back(take_page(l));
    lay.pers_rows = r1;
    lay.G = G;
    lay.prompt_written = true;
  }
  q.nb = nb;
  return kOk;
}

int64_t HostPool::row_position(int32_t id, int32_t l, int32_t r) const {
  const SeqState& q = seqs_[id];
  const LayerState& lay = q.layers[l];
  if (r < q.P) return r;
  if (r < lay.pers_rows) {
    if (!s_.compress) return r;  // generated token j = r - P sits at P + j
    int32_t c = r - q.P, qn = s_.quota[l], K = s_.pause[l];
    int32_t b = c / qn, k = c % qn;
    return (int64_t)q.P + (int64_t)b * s_.C + (int64_t)bitrev(k, log2_exact(K)) * (s_.C / K);
  }
  return (int64_t)q.P + (int64_t)q.nb * s_.C + (r - lay.pers_rows);
}

}  // namespace abk
