// Host-side model of an R-SWA handle (see host_state.hpp).  No HIP here.
#include "host_state.hpp"

#include <iterator>

#include <algorithm>
#include <cmath>
#include <numeric>

namespace rswa {

namespace {

int fail(std::string *err, int code, const std::string &msg) {
  if (err) *err = msg;
  return code;
}

std::string S(int64_t v) { return std::to_string(v); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int resolve_config(const rswa_config &in, Config *out, std::string *err) {
  Config c;
  c.num_layers = in.num_layers;
  c.num_heads = in.num_heads;
  c.head_dim = in.head_dim;
  c.window = in.window;
  c.max_positions = in.max_positions == 0 ? kDefaultMaxPositions : in.max_positions;
  c.max_requests = in.max_requests;
  c.num_slots = in.num_slots;
  c.dtype = in.dtype;
  c.max_splits = in.max_splits == 0 ? std::max(16384, 4 * std::max(in.max_requests, 0))
                                    : in.max_splits;
  c.max_prefill_tokens =
      in.max_prefill_tokens == 0 ? kDefaultMaxPrefillTokens : in.max_prefill_tokens;
  c.decode_split_tokens = in.decode_split_tokens;
  c.attention = in.attention;
  c.rope_base = in.rope_base == 0 ? 10000.0 : in.rope_base;
  c.softmax_scale = in.softmax_scale > 0 ? in.softmax_scale : 0.0;
  c.has_table = in.slot_table != nullptr;
  c.slot_table_len = in.slot_table_len;

  if (c.num_layers < 1) return fail(err, RSWA_E_ARG, "num_layers must be >= 1");
  if (c.num_heads < 1 || c.num_heads > 512) return fail(err, RSWA_E_ARG, "num_heads must be in [1, 512]");
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(err, RSWA_E_UNSUPPORTED, "head_dim must be 64 or 128, got " + S(c.head_dim));
  if (c.dtype != RSWA_DTYPE_BF16 && c.dtype != RSWA_DTYPE_F32)
    return fail(err, RSWA_E_UNSUPPORTED, "dtype must be RSWA_DTYPE_BF16 or RSWA_DTYPE_F32");
  if (c.window < 1) return fail(err, RSWA_E_ARG, "window must be >= 1");
  if (c.max_positions < 1 || c.max_positions > (1 << 22))
    return fail(err, RSWA_E_ARG, "max_positions must be in [1, 4194304]");
  if (c.window > c.max_positions) return fail(err, RSWA_E_ARG, "window exceeds max_positions");
  if (c.max_requests < 1 || c.max_requests > (1 << 20))
    return fail(err, RSWA_E_ARG, "max_requests must be in [1, 1048576]");
  if (c.num_slots < 1 || c.num_slots > INT32_MAX)
    return fail(err, RSWA_E_ARG, "num_slots must be in [1, 2^31-1]");
  if (c.max_splits < c.max_requests || c.max_splits > (1 << 24))
    return fail(err, RSWA_E_ARG, "max_splits must be in [max_requests, 2^24]");
  if ((int64_t)c.max_splits * c.num_heads > (int64_t(1) << 28))
    return fail(err, RSWA_E_ARG, "max_splits * num_heads must be <= 2^28");
  if (c.max_prefill_tokens < 1 || c.max_prefill_tokens > (int64_t(1) << 31))
    return fail(err, RSWA_E_ARG, "max_prefill_tokens must be in [1, 2^31]");
  if (c.decode_split_tokens < 0 || c.decode_split_tokens % kSplitQuantum != 0)
    return fail(err, RSWA_E_ARG, "decode_split_tokens must be a non-negative multiple of 64");
  if (c.attention != RSWA_ATTENTION_RSWA && c.attention != RSWA_ATTENTION_SWA)
    return fail(err, RSWA_E_ARG, "attention must be RSWA_ATTENTION_RSWA or RSWA_ATTENTION_SWA");
  if (!(c.rope_base > 0) || !std::isfinite(c.rope_base))
    return fail(err, RSWA_E_ARG, "rope_base must be positive");
  if (!std::isfinite(in.softmax_scale)) return fail(err, RSWA_E_ARG, "softmax_scale must be finite");
  if (c.softmax_scale == 0) c.softmax_scale = 1.0 / std::sqrt((double)c.head_dim);
  // Decode addresses a request's rows (and, with a slot table, a whole layer)
  // through 32-bit buffer offsets.
  const int64_t row_bytes = (int64_t)c.num_heads * c.head_dim * c.elem_bytes();
  if (((int64_t)c.max_positions + c.window) * row_bytes > (int64_t)UINT32_MAX)
    return fail(err, RSWA_E_UNSUPPORTED, "(max_positions + window) * heads * head_dim * elem_bytes "
                                         "must be < 2^32");
  if (c.has_table && c.num_slots * row_bytes > (int64_t)UINT32_MAX - 64)
    return fail(err, RSWA_E_UNSUPPORTED, "with a slot table, one layer of a pool "
                                         "(num_slots * heads * head_dim * elem_bytes) must be < 2^32 - 64 bytes");
  if (c.has_table) {
    if (c.slot_table_len < 1 || c.slot_table_len > INT32_MAX)
      return fail(err, RSWA_E_ARG, "slot_table_len must be in [1, 2^31-1] with a slot table");
  } else if (in.slot_table_len != 0) {
    return fail(err, RSWA_E_ARG, "slot_table_len given without a slot table");
  }
  *out = c;
  return RSWA_OK;
}

BatchBlob BatchBlob::make(int n, int k) {
  BatchBlob b;
  b.req = 0;
  b.split_off = align_up(sizeof(int32_t) * n, 16);
  b.splits = b.split_off + align_up(sizeof(int32_t) * (n + 1), 32);
  b.bytes = b.splits + sizeof(SplitDesc) * (size_t)k;
  return b;
}

size_t BatchBlob::capacity(const Config &c) { return make(c.max_requests, c.max_splits).bytes; }

PrefillBlob PrefillBlob::make(int n, int64_t t) {
  PrefillBlob b;
  b.req = 0;
  b.plen = align_up(sizeof(int32_t) * n, 16);
  b.qoff = b.plen + align_up(sizeof(int32_t) * n, 16);
  b.ptot = b.qoff + align_up(sizeof(int32_t) * n, 16);
  b.cu = b.ptot + align_up(sizeof(int32_t) * n, 16);
  b.base = b.cu + align_up(sizeof(int64_t) * (n + 1), 16);
  b.tiles = b.base + align_up(sizeof(int64_t) * n, 16);
  b.bytes = b.tiles + align_up(sizeof(int32_t) * 2 * (size_t)t, 16);
  return b;
}

size_t PrefillBlob::capacity(const Config &c) {
  return make(c.max_requests, c.max_prefill_blocks()).bytes;
}

Layout make_layout(const Config &c) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.rope = take(sizeof(float) * 2 * (size_t)c.max_positions * (c.head_dim / 2));
  L.req_p = take(sizeof(int32_t) * c.max_requests);
  L.req_t = take(sizeof(int32_t) * c.max_requests);
  L.req_base = take(sizeof(int64_t) * c.max_requests);
  L.batch_bytes = BatchBlob::capacity(c);
  L.batch = take(L.batch_bytes);
  L.part_o = take(sizeof(float) * (size_t)c.max_splits * c.num_heads * c.head_dim);
  L.part_ml = take(sizeof(float) * 2 * (size_t)c.max_splits * c.num_heads);
  L.merge_cnt = take(sizeof(int32_t) * (size_t)c.max_requests * c.num_heads);
  L.step_cnt = take(sizeof(int32_t) * (size_t)c.max_requests);
  L.prefill_bytes = PrefillBlob::capacity(c);
  L.prefill = take(L.prefill_bytes);
  L.total = off;
  return L;
}

HostState::HostState(const Config &c)
    : cfg_(c),
      req_(c.max_requests),
      done_((size_t)c.max_requests * c.num_layers, 0),
      admitted_(c.max_requests, {0, 0}),
      in_batch_(c.max_requests, 0),
      written_(c.num_layers, 0),
      decoded_(c.num_layers, 0) {
  free_[0] = c.row_capacity();
}

bool HostState::fully_prefilled(int32_t id) const {
  const RequestState &r = req_[id];
  if (r.plen < 0) return false;
  for (int l = 0; l < cfg_.num_layers; ++l)
    if (prefilled(id, l) != r.plen) return false;
  return true;
}

bool HostState::step_open() const {
  for (int l = 0; l < cfg_.num_layers; ++l)
    if (written_[l] || decoded_[l]) return true;
  return false;
}

int HostState::check_prefill(int32_t layer, int32_t n, const int32_t *ids, const int32_t *plen,
                             const int64_t *base, std::string *err, const int32_t *start,
                             const int32_t *len) const {
  if (layer < 0 || layer >= cfg_.num_layers)
    return fail(err, RSWA_E_ARG, "layer " + S(layer) + " out of range");
  if (n < 0 || n > cfg_.max_requests) return fail(err, RSWA_E_ARG, "n out of range");
  if (n > 0 && (!ids || !plen || !base)) return fail(err, RSWA_E_ARG, "null host array");
  if ((start == nullptr) != (len == nullptr)) return fail(err, RSWA_E_ARG, "chunk_start / chunk_len: both or neither");
  std::vector<uint8_t> seen(cfg_.max_requests, 0);
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= cfg_.max_requests)
      return fail(err, RSWA_E_ARG, "request id " + S(id) + " out of range");
    if (seen[id]) return fail(err, RSWA_E_ARG, "request id " + S(id) + " repeated");
    seen[id] = 1;
    if (plen[i] < 0) return fail(err, RSWA_E_ARG, "negative prefill_len");
    if (plen[i] > cfg_.max_positions)
      return fail(err, RSWA_E_POSITION, "prefill_len " + S(plen[i]) + " exceeds max_positions");
    if (base[i] < 0) return fail(err, RSWA_E_ARG, "negative slot_base");
    if (base[i] + plen[i] + cfg_.window > cfg_.row_capacity())
      return fail(err, RSWA_E_CAPACITY, "request " + S(id) + " needs rows up to " +
                                            S(base[i] + plen[i] + cfg_.window) + " but the " +
                                            (cfg_.has_table ? "slot table" : "pool") + " has " +
                                            S(cfg_.row_capacity()));
    const int32_t s0 = start ? start[i] : 0;
    const int32_t ln = len ? len[i] : plen[i];
    if (s0 < 0 || ln < 0 || (int64_t)s0 + ln > plen[i])
      return fail(err, RSWA_E_ARG, "request " + S(id) + ": chunk " + S(s0) + " + " + S(ln) +
                                       " outside prefill_len " + S(plen[i]));
    total += ln;
    if (in_batch_[id])
      return fail(err, RSWA_E_STATE, "request " + S(id) + " is in the active decode batch");
    const std::pair<int64_t, int64_t> &adm = admitted_[id];
    if (adm.second && (base[i] != adm.first || (int64_t)plen[i] + cfg_.window > adm.second))
      return fail(err, RSWA_E_ARG, "request " + S(id) + " was admitted with rows " + S(adm.first) +
                                       " .. " + S(adm.first + adm.second - 1));
    const RequestState &r = req_[id];
    if (layer == 0 && s0 == 0) continue;  // (re)registers the request
    if (r.plen < 0) return fail(err, RSWA_E_STATE, "request " + S(id) + " not registered (layer 0, chunk at 0)");
    if (r.plen != plen[i] || r.base != base[i])
      return fail(err, RSWA_E_STATE, "request " + S(id) + " prefill_len/slot_base differ from its registration");
    if (prefilled(id, layer) != s0)
      return fail(err, RSWA_E_STATE, "request " + S(id) + " layer " + S(layer) + " holds " +
                                         S(prefilled(id, layer)) + " prefill rows, chunk starts at " + S(s0));
    if (layer > 0 && prefilled(id, layer - 1) < s0 + ln)
      return fail(err, RSWA_E_STATE, "request " + S(id) + ": layer " + S(layer - 1) + " holds " +
                                         S(prefilled(id, layer - 1)) + " rows; layers must go in order");
  }
  if (total > cfg_.max_prefill_tokens)
    return fail(err, RSWA_E_CAPACITY, "prefill tokens " + S(total) + " exceed max_prefill_tokens");
  return RSWA_OK;
}

void HostState::commit_prefill(int32_t layer, int32_t n, const int32_t *ids, const int32_t *plen,
                               const int64_t *base, const int32_t *start, const int32_t *len) {
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    RequestState &r = req_[id];
    const int32_t s0 = start ? start[i] : 0;
    const int32_t ln = len ? len[i] : plen[i];
    if (layer == 0 && s0 == 0) {
      r.plen = plen[i];
      r.base = base[i];
      r.t = 0;
      std::fill(done_.begin() + (size_t)id * cfg_.num_layers,
                done_.begin() + (size_t)(id + 1) * cfg_.num_layers, 0);
    }
    done_[(size_t)id * cfg_.num_layers + layer] = s0 + ln;
  }
}

PrefillPlan HostState::plan_prefill(int32_t n, const int32_t *plen, int32_t tile,
                                    const int32_t *qoff) const {
  PrefillPlan p;
  p.tile = tile;
  p.cu.assign(n + 1, 0);
  for (int b = 0; b < n; ++b) {
    p.cu[b + 1] = p.cu[b] + plen[b];
    p.max_len = std::max(p.max_len, plen[b]);
  }
  p.total_tokens = p.cu[n];
  const int heads = cfg_.num_heads;
  // Work of query tile qt of request b, in key tiles: the rows before the
  // chunk (qoff / tile) plus the causal part.
  struct Item { int32_t b, qt, h; int64_t work; };
  struct Group { int32_t b, h, tiles; int64_t work; };
  auto lead = [&](int b) -> int64_t { return qoff ? qoff[b] / tile : 0; };
  std::vector<Group> groups;
  int64_t n_items = 0;
  for (int b = 0; b < n; ++b) {
    const int32_t nt = (int32_t)ceil_div(plen[b], tile);
    if (nt == 0) continue;
    const int64_t work = (int64_t)nt * (nt + 1) / 2 + (int64_t)nt * lead(b);
    for (int h = 0; h < heads; ++h) groups.push_back({b, h, nt, work});
    n_items += (int64_t)nt * heads;
  }
  // Longest-processing-time assignment to XCDs, by whole (request, head)
  // group when there are enough groups, else by single block.
  std::vector<std::vector<Item>> xcd(kNumXcds);
  std::vector<int64_t> load(kNumXcds, 0);
  auto least = [&]() {
    return (int)(std::min_element(load.begin(), load.end()) - load.begin());
  };
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group &x, const Group &y) { return x.work > y.work; });
  bool affinity = groups.size() >= (size_t)kXcdAffinityGroups;
  if (affinity) {
    for (const Group &g : groups) {
      const int x = least();
      for (int32_t qt = g.tiles - 1; qt >= 0; --qt) xcd[x].push_back({g.b, qt, g.h, 0});
      load[x] += g.work;
    }
    size_t longest = 0;
    for (auto &l : xcd) longest = std::max(longest, l.size());
    if ((int64_t)longest * kNumXcds > 2 * n_items + 64) {  // too much padding
      affinity = false;
      for (auto &l : xcd) l.clear();
      std::fill(load.begin(), load.end(), 0);
    }
  }
  if (!affinity) {
    std::vector<Item> items;
    items.reserve(n_items);
    for (const Group &g : groups)
      for (int32_t qt = 0; qt < g.tiles; ++qt) items.push_back({g.b, qt, g.h, qt + 1 + lead(g.b)});
    std::stable_sort(items.begin(), items.end(),
                     [](const Item &x, const Item &y) { return x.work > y.work; });
    for (const Item &it : items) {
      const int x = least();
      xcd[x].push_back(it);
      load[x] += it.work;
    }
  }
  size_t longest = 0;
  for (auto &l : xcd) longest = std::max(longest, l.size());
  p.tiles.reserve(2 * longest * kNumXcds);
  for (size_t k = 0; k < longest; ++k)
    for (int x = 0; x < kNumXcds; ++x) {
      if (k < xcd[x].size()) {
        const Item &it = xcd[x][k];
        p.tiles.push_back(it.b);
        p.tiles.push_back((int32_t)(((uint32_t)it.qt << 16) | (uint32_t)it.h));
      } else {
        p.tiles.push_back(-1);
        p.tiles.push_back(0);
      }
    }
  // Trailing empty slots need no launch.
  while (p.tiles.size() >= 2 && p.tiles[p.tiles.size() - 2] < 0) p.tiles.resize(p.tiles.size() - 2);
  return p;
}

int HostState::check_set_batch(int32_t n, const int32_t *ids, std::string *err) const {
  if (step_open())
    return fail(err, RSWA_E_STATE, "rswa_set_batch inside a step (after a ring write, before advance)");
  if (n < 0 || n > cfg_.max_requests) return fail(err, RSWA_E_ARG, "n out of range");
  if (n > 0 && !ids) return fail(err, RSWA_E_ARG, "null req_ids");
  std::vector<uint8_t> seen(cfg_.max_requests, 0);
  for (int i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= cfg_.max_requests)
      return fail(err, RSWA_E_ARG, "request id " + S(id) + " out of range");
    if (seen[id]) return fail(err, RSWA_E_ARG, "request id " + S(id) + " repeated");
    seen[id] = 1;
    if (!fully_prefilled(id))
      return fail(err, RSWA_E_STATE, "request " + S(id) + " is not prefilled in every layer");
  }
  if (n > 0) {
    DecodePlan p = plan_decode(n, ids);
    if (p.num_splits() > cfg_.max_splits)
      return fail(err, RSWA_E_CAPACITY, "batch needs " + S(p.num_splits()) +
                                            " split work items; max_splits is " + S(cfg_.max_splits));
  }
  return RSWA_OK;
}

DecodePlan HostState::plan_decode(int32_t n, const int32_t *ids) const {
  DecodePlan p;
  // Key range a request's decode steps can reach: logical slots
  // decode_key0(P) .. P + W - 1 (all of 0 .. P + W - 1 for R-SWA).
  std::vector<int64_t> lmax(n);
  int64_t longest = 0;
  for (int b = 0; b < n; ++b) {
    const int32_t pl = req_[ids[b]].plen;
    lmax[b] = (int64_t)pl + cfg_.window - decode_key0(pl);
    longest = std::max(longest, lmax[b]);
  }
  const int64_t heads = cfg_.num_heads;
  auto splits_of = [&](int64_t sz) {
    int64_t k = 0;
    for (int b = 0; b < n; ++b) k += ceil_div(lmax[b], sz);
    return k;
  };
  int64_t keys = 0;
  for (int b = 0; b < n; ++b) keys += lmax[b];
  int64_t sz = cfg_.decode_split_tokens;
  if (sz <= 0) {
    if (keys * heads <= kOneRoundKeys) {
      sz = kSplitQuantum;
      while (splits_of(sz) * heads > kDecodeWaves) sz += kSplitQuantum;
    } else {
      sz = kLongSplitKeys;
      while (splits_of(sz) * heads > resident_waves_ && sz < longest) sz += kSplitQuantum;
    }
    while (splits_of(sz) > cfg_.max_splits) sz += kSplitQuantum;
  }
  p.split_tokens = (int32_t)std::min<int64_t>(sz, longest);
  p.split_off.assign(n + 1, 0);
  for (int b = 0; b < n; ++b) {
    const int32_t id = ids[b];
    const RequestState &rq = req_[id];
    const int64_t k = ceil_div(lmax[b], sz);
    const int64_t key0 = decode_key0(rq.plen);
    p.split_off[b + 1] = p.split_off[b] + (int32_t)k;
    for (int64_t j = 0; j < k; ++j) {
      SplitDesc d{};
      d.b = b;
      d.r = id;
      d.k0 = (int32_t)(key0 + j * sz);
      d.k1 = (int32_t)std::min(key0 + (j + 1) * sz, key0 + lmax[b]);
      d.p = rq.plen;
      d.base = rq.base;
      p.splits.push_back(d);
    }
  }
  // Launch shape: the fewest waves per block that give every CU at most one
  // block, within what a CU holds.
  const int64_t tasks = (int64_t)p.num_splits() * heads;
  const int64_t per_cu = std::clamp<int64_t>(resident_waves_ / kDecodeCUs, 1, kDecodeMaxWavesPerBlock);
  p.waves_per_block = (int32_t)std::clamp<int64_t>(ceil_div(tasks, kDecodeCUs), 1, per_cu);
  return p;
}

void HostState::commit_set_batch(int32_t n, const int32_t *ids, DecodePlan plan) {
  for (int32_t id : batch_) in_batch_[id] = 0;
  batch_.assign(ids, ids + n);
  for (int32_t id : batch_) in_batch_[id] = 1;
  plan_ = std::move(plan);
  ++epoch_;
}

int HostState::check_ring_write(int32_t layer, std::string *err) const {
  if (layer < 0 || layer >= cfg_.num_layers)
    return fail(err, RSWA_E_ARG, "layer " + S(layer) + " out of range");
  if (batch_.empty()) return fail(err, RSWA_E_STATE, "no active batch (rswa_set_batch)");
  if (written_[layer])
    return fail(err, RSWA_E_STATE, "layer " + S(layer) + " already written in this step");
  for (int32_t id : batch_) {
    const RequestState &r = req_[id];
    if ((int64_t)r.plen + r.t >= cfg_.max_positions)
      return fail(err, RSWA_E_POSITION, "request " + S(id) + " reached position " +
                                            S((int64_t)r.plen + r.t) + " = max_positions");
  }
  return RSWA_OK;
}

void HostState::commit_ring_write(int32_t layer) { written_[layer] = 1; }

int HostState::check_decode(int32_t layer, std::string *err) const {
  if (layer < 0 || layer >= cfg_.num_layers)
    return fail(err, RSWA_E_ARG, "layer " + S(layer) + " out of range");
  if (batch_.empty()) return fail(err, RSWA_E_STATE, "no active batch (rswa_set_batch)");
  if (!written_[layer])
    return fail(err, RSWA_E_STATE, "layer " + S(layer) + ": rswa_ring_write must come first");
  if (decoded_[layer])
    return fail(err, RSWA_E_STATE, "layer " + S(layer) + " already decoded in this step");
  return RSWA_OK;
}

void HostState::commit_decode(int32_t layer) { decoded_[layer] = 1; }

int HostState::check_fused(int32_t layer, std::string *err) const {
  return check_ring_write(layer, err);  // not written this step implies not decoded
}

void HostState::commit_fused(int32_t layer) {
  written_[layer] = 1;
  decoded_[layer] = 1;
}

int HostState::check_advance(std::string *err) const {
  if (batch_.empty()) return fail(err, RSWA_E_STATE, "no active batch (rswa_set_batch)");
  for (int l = 0; l < cfg_.num_layers; ++l)
    if (!decoded_[l])
      return fail(err, RSWA_E_STATE, "layer " + S(l) + " not decoded in this step");
  return RSWA_OK;
}

bool HostState::completes_step(int32_t layer) const {
  for (int l = 0; l < cfg_.num_layers; ++l)
    if (l != layer && !decoded_[l]) return false;
  return !decoded_[layer];
}

bool HostState::step_decoded() const {
  for (int l = 0; l < cfg_.num_layers; ++l)
    if (!decoded_[l]) return false;
  return !batch_.empty();
}

void HostState::commit_advance() {
  for (int32_t id : batch_) req_[id].t += 1;
  std::fill(written_.begin(), written_.end(), 0);
  std::fill(decoded_.begin(), decoded_.end(), 0);
}

int HostState::check_note_steps(int32_t steps, std::string *err) const {
  if (steps < 0) return fail(err, RSWA_E_ARG, "steps must be >= 0");
  if (batch_.empty()) return fail(err, RSWA_E_STATE, "no active batch (rswa_set_batch)");
  if (step_open()) return fail(err, RSWA_E_STATE, "a decode step is half done");
  if (captured_epoch_ != (int64_t)epoch_)
    return fail(err, RSWA_E_STATE, "no decode step of the current batch was captured "
                                   "(rswa_set_batch since the capture invalidates the graph)");
  for (int32_t id : batch_) {
    const RequestState &r = req_[id];
    if ((int64_t)r.plen + r.t + steps > cfg_.max_positions)
      return fail(err, RSWA_E_POSITION, "request " + S(id) + " would pass max_positions");
  }
  return RSWA_OK;
}

void HostState::commit_note_steps(int32_t steps) {
  for (int32_t id : batch_) req_[id].t += steps;
}

int HostState::check_admit(int32_t id, int32_t plen, int64_t *base, std::string *err) const {
  if (id < 0 || id >= cfg_.max_requests) return fail(err, RSWA_E_ARG, "request id out of range");
  if (plen < 0) return fail(err, RSWA_E_ARG, "negative prefill_len");
  if (plen > cfg_.max_positions)
    return fail(err, RSWA_E_POSITION, "prefill_len " + S(plen) + " exceeds max_positions");
  if (req_[id].plen >= 0 || admitted_[id].second)
    return fail(err, RSWA_E_STATE, "request " + S(id) + " is registered or admitted (retire it first)");
  const int64_t need = (int64_t)plen + cfg_.window;
  for (const auto &f : free_)
    if (f.second >= need) {
      *base = f.first;
      return RSWA_OK;
    }
  return fail(err, RSWA_E_CAPACITY, "no " + S(need) + " free consecutive rows (" + S(free_rows()) +
                                        " free in all)");
}

void HostState::commit_admit(int32_t id, int32_t plen, int64_t base) {
  const int64_t need = (int64_t)plen + cfg_.window;
  auto it = free_.find(base);
  const int64_t len = it->second;
  free_.erase(it);
  if (len > need) free_[base + need] = len - need;
  admitted_[id] = {base, need};
}

int HostState::check_retire(int32_t n, const int32_t *ids, std::string *err) const {
  if (n < 0 || n > cfg_.max_requests) return fail(err, RSWA_E_ARG, "n out of range");
  if (n > 0 && !ids) return fail(err, RSWA_E_ARG, "null req_ids");
  std::vector<uint8_t> seen(cfg_.max_requests, 0);
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= cfg_.max_requests) return fail(err, RSWA_E_ARG, "request id out of range");
    if (seen[id]) return fail(err, RSWA_E_ARG, "request id " + S(id) + " repeated");
    seen[id] = 1;
    if (in_batch_[id]) return fail(err, RSWA_E_STATE, "request " + S(id) + " is in the active decode batch");
  }
  return RSWA_OK;
}

void HostState::commit_retire(int32_t n, const int32_t *ids) {
  for (int i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    req_[id] = RequestState{};
    std::fill(done_.begin() + (size_t)id * cfg_.num_layers,
              done_.begin() + (size_t)(id + 1) * cfg_.num_layers, 0);
    auto [start, len] = admitted_[id];
    admitted_[id] = {0, 0};
    if (!len) continue;
    // return the range, merging with free neighbours
    auto next = free_.lower_bound(start);
    if (next != free_.end() && start + len == next->first) {
      len += next->second;
      next = free_.erase(next);
    }
    if (next != free_.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == start) {
        prev->second += len;
        continue;
      }
    }
    free_[start] = len;
  }
}

int64_t HostState::free_rows() const {
  int64_t total = 0;
  for (const auto &f : free_) total += f.second;
  return total;
}

}  // namespace rswa
