// Host bookkeeping of the paged AbridgeKV cache: page allocator, sequence
// slots, per-(sequence, layer) row counts and page lists, protocol checks.
// Plain C++ with no device calls; the C ABI drives it and mirrors its results
// to the device. Every operation validates first and changes nothing on
// failure.
//
// Cache structure (arXiv 2610.20641, abstract and Fig. 1 captions; AI Radio
// transcript): per layer the resident rows are the prompt, quota[l] code rows
// per finished block, and the open block's raw rows; rows a layer does not
// keep are never allocated, and a finished block's raw rows are freed.
#pragma once

#include <cstdint>
#include <functional>
#include <queue>
#include <string>
#include <vector>

namespace abk {

enum Status : int32_t {
  kOk = 0,
  kInvalidArg = 1,
  kOutOfPages = 2,
  kBadState = 3,
  kHipError = 4,
  kUnsupported = 5,
};

struct Shape {
  int32_t L = 0, Hq = 0, Hkv = 0, D = 0;
  int32_t C = 0, pr = 0;  // block tokens, page rows
  int32_t max_seqs = 0, max_position = 0, dtype = 0, compress = 1;
  int64_t num_pages = 0;
  double rope_base = 0.0;
  std::vector<int32_t> quota, pause;  // per layer
  // Optional separate page pools per budget level (a level = one distinct
  // quota value, ascending): pages of level k are ids [sum of earlier counts,
  // + level_pages[k]). Empty: one pool for every layer.
  std::vector<int64_t> level_pages;
  int32_t esize() const { return dtype == 0 ? 4 : 2; }
  int32_t max_pers_pages() const { return (max_position + pr - 1) / pr; }
  int32_t max_open_pages() const { return compress ? C / pr : 0; }
  int32_t table_stride() const { return max_pers_pages() + max_open_pages(); }
};

struct LayerState {
  int32_t G = 0;          // generated rows appended at this layer
  int32_t pers_rows = 0;  // prompt + code rows (compress) or prompt + text (full-KV)
  std::vector<int32_t> pers_pages, open_pages;
  bool compressed = false;  // current block compressed here, not yet freed
  bool prompt_written = false;
};

struct SeqState {
  bool live = false;
  int32_t P = 0;
  int32_t nb = 0;  // blocks compressed and freed
  std::vector<LayerState> layers;
};

// What one (sequence, layer) of a compress call needs on the device.
struct CompressPlan {
  int32_t slot, layer, quota, block, pers_before;
  std::vector<int32_t> pages;  // pages covering rows [pers_before, pers_before + quota)
  int32_t first_new;           // index in `pages` of the first newly taken page
};

class HostPool {
 public:
  Status init(const Shape& s, std::string* err);

  const Shape& shape() const { return s_; }
  const SeqState& seq(int32_t id) const { return seqs_[id]; }
  int64_t pages_free() const;
  // budget levels: count, the level of a layer, a level's quota and pages
  int32_t levels() const { return (int32_t)free_.size(); }
  int32_t level_of(int32_t l) const { return level_of_[l]; }
  int32_t level_quota(int32_t k) const { return level_quota_[k]; }
  int64_t level_pages(int32_t k) const { return level_start_[k + 1] - level_start_[k]; }
  int64_t level_free(int32_t k) const { return (int64_t)free_[k].size(); }
  int32_t open_rows(int32_t id, int32_t l) const;
  int32_t resident_rows(int32_t id, int32_t l) const;
  int64_t resident_rows_total() const;

  // Checks shared by the ABI.
  Status check_seq(int32_t id) const;
  Status check_layer(int32_t l) const;
  Status check_layers(int32_t l0, int32_t nl) const;
  Status check_batch(int32_t n, const int32_t* ids);

  // The calls below act on the layers [l0, l0 + nl) together (one layer, or
  // the per-head layers of one model layer): every check passes for all of
  // them before anything changes. Per-(sequence, layer) outputs are ordered
  // sequence-major: entry i * nl + j is sequence ids[i] at layer l0 + j.
  Status seq_create(int32_t P, int32_t* id);
  Status seq_release(int32_t id);
  Status write_prompt(int32_t id, int32_t l0, int32_t nl = 1);
  // new_page[e] = page taken for entry e's row, or -1.
  Status append(int32_t l0, int32_t nl, int32_t n, const int32_t* ids, std::vector<int32_t>* new_page);
  Status check_decode(int32_t l0, int32_t nl, int32_t n, const int32_t* ids);
  // the checks of compress alone (nothing changes)
  Status check_compress(int32_t l0, int32_t nl, int32_t n, const int32_t* ids);
  Status compress(int32_t l0, int32_t nl, int32_t n, const int32_t* ids, std::vector<CompressPlan>* plan);
  Status free_block(int32_t n, const int32_t* ids);
  Status fill(int32_t id, int32_t G);

  // Position of resident row r of (id, l), from the host mirror.
  int64_t row_position(int32_t id, int32_t l, int32_t r) const;

  std::string err;  // reason of the last failure

 private:
  Status fail(Status st, const std::string& msg) {
    err = msg;
    return st;
  }
  int32_t take_page(int32_t l);  // from layer l's budget pool
  void give_page(int32_t p);
  // pages a call needs per budget level; fails unless every level has them
  Status check_need(const std::vector<int64_t>& need, const char* what);
  int32_t gmin(const SeqState& q) const;
  int32_t gmax(const SeqState& q) const;

  Shape s_;
  std::vector<SeqState> seqs_;
  using MinHeap = std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>>;
  std::vector<MinHeap> free_;         // per budget level
  std::vector<int64_t> level_start_;  // first page id of each level, then the end
  std::vector<int32_t> level_of_;     // per layer
  std::vector<int32_t> level_quota_;  // per level (-1: one pool for all quotas)
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_slots_;
  std::vector<uint32_t> mark_;  // duplicate detection, stamped per call
  uint32_t stamp_ = 0;
};

int32_t bitrev(int32_t k, int32_t nbits);
int32_t log2_exact(int32_t x);  // -1 unless x is a power of two

}  // namespace abk
