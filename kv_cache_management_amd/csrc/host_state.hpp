// Host-side model of an R-SWA cache handle: config validation, workspace
// layout, the per-request ring state mirror, the call-order state machine and
// the split-KV / prefill work planning.  Pure C++17, no HIP: the same code is
// linked into the HIP library and into a CPU-only test program.
//
// Ring state follows page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘"
// (www.gtnt.cn/news/146005), section 2.1: a request holds its prefill_len
// prefill rows plus a W-row ring written at prefill_len + ring_pos, so its
// cache never exceeds prefill_len + W rows.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "rswa.h"

namespace rswa {

constexpr int kAlign = 256;
constexpr int kSplitQuantum = 64;      // forced split sizes are multiples of this
// Split-KV planning (measured on MI355X).  A decode step streams at the
// rate its busiest CU allows, and each wave adds a fixed start-up and merge
// latency.  Splits are kSplitQuantum-multiples (the last split of a request
// takes the remainder; equal splits at arbitrary key offsets measured
// slower).  Batches of at most kOneRoundKeys key-heads run as one round of
// at most kDecodeWaves waves (one per SIMD, blocks of four, at most one
// block per CU), with the shortest split length that fits; larger batches use
// kLongSplitKeys-key splits, lengthened until every wave of the launch is
// resident at once: blocks that do not fit start only when others finish
// and then stream alone, at the end of the step.  A launch is shaped as one
// block per CU with the fewest waves per block that allows (single waves
// for at most one wave per CU, four for a full one-round batch, twelve for
// one of every resident wave): blocks of four landed two or three to a CU,
// unevenly, and streamed ~3 % slower.
constexpr int kDecodeWaves = 1024;          // 256 CUs x 4 SIMDs
constexpr int kDecodeWavesPerBlock = 4;
constexpr int kDecodeMaxWavesPerBlock = 12; // 3 waves per SIMD x 4 SIMDs
constexpr int kDecodeCUs = 256;
constexpr int kLongSplitKeys = 1024;
constexpr int64_t kOneRoundKeys = (int64_t)kDecodeWaves * 1280;
// Decode waves the GPU holds at once when the device was not asked (three
// per SIMD: the kernel's register count); rswa_cache_init sets the measured
// figure.
constexpr int64_t kDefaultResidentWaves = 3 * (int64_t)kDecodeWaves;
constexpr int kDefaultMaxPositions = 32768;
constexpr int64_t kDefaultMaxPrefillTokens = 262144;
constexpr int kPrefillTileMin = 64;    // smallest prefill query tile of any kernel

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Config with defaults resolved.
struct Config {
  int32_t num_layers = 0, num_heads = 0, head_dim = 0, window = 0;
  int32_t max_positions = 0, max_requests = 0, dtype = 0, max_splits = 0;
  int32_t decode_split_tokens = 0, attention = 0;
  int64_t num_slots = 0, max_prefill_tokens = 0, slot_table_len = 0;
  double rope_base = 0, softmax_scale = 0;
  bool has_table = false;
  int elem_bytes() const { return dtype == RSWA_DTYPE_BF16 ? 2 : 4; }
  int64_t row_capacity() const { return has_table ? slot_table_len : num_slots; }
  int64_t max_prefill_tiles() const {
    return max_prefill_tokens / kPrefillTileMin + max_requests;
  }
  // Launch slots of one prefill call: every (query tile, head) block plus
  // the padding the XCD interleave may add.
  int64_t max_prefill_blocks() const { return 2 * max_prefill_tiles() * num_heads + 64; }
};

// Byte offsets of each workspace region (all 256-byte aligned).
struct Layout {
  size_t rope = 0;        // float2 [max_positions][head_dim/2] (cos, sin)
  size_t req_p = 0;       // int32 [max_requests]  prefill_len
  size_t req_t = 0;       // int32 [max_requests]  generated tokens
  size_t req_base = 0;    // int64 [max_requests]  slot_base
  size_t batch = 0;       // batch blob (see BatchBlob)
  size_t batch_bytes = 0;
  size_t part_o = 0;      // float [max_splits][num_heads][head_dim]
  size_t part_ml = 0;     // float2 [max_splits][num_heads]  (max, sum)
  size_t merge_cnt = 0;   // int32 [max_requests][num_heads]  splits finished per (entry, head)
  size_t step_cnt = 0;    // int32 [max_requests]  heads merged per entry (step's last layer)
  size_t prefill = 0;     // prefill blob (see PrefillBlob)
  size_t prefill_bytes = 0;
  size_t total = 0;
};

// Validates cfg and resolves defaults.  Returns RSWA_OK or an error code
// with a message in *err.
int resolve_config(const rswa_config &in, Config *out, std::string *err);
Layout make_layout(const Config &c);

// One split-KV work item: keys [k0, k1) (logical slots) of batch entry b,
// request r with prefill_len p and first pool row / table index base.
// k1 <= p + W; the keys a step reads are the part below p + min(t + 1, W).
struct SplitDesc {
  int32_t b, r, k0, k1, p, pad;
  int64_t base;
};
static_assert(sizeof(SplitDesc) == 32, "split descriptor is one 32-byte scalar load");

// Offsets inside a packed blob uploaded in one copy.
struct BatchBlob {   // for n active requests and k split work items
  size_t req = 0;        // int32 [n]      request id of batch entry b
  size_t split_off = 0;  // int32 [n + 1]  first split of batch entry b
  size_t splits = 0;     // SplitDesc [k]
  size_t bytes = 0;
  static BatchBlob make(int n, int k);
  static size_t capacity(const Config &c);
};

struct PrefillBlob {  // for n requests and t query tiles
  size_t req = 0;        // int32 [n]
  size_t plen = 0;       // int32 [n]      rows of this call (the chunk length)
  size_t qoff = 0;       // int32 [n]      position of the chunk's first row
  size_t ptot = 0;       // int32 [n]      the request's whole prefill_len
  size_t cu = 0;         // int64 [n + 1]  packed token offset of request b
  size_t base = 0;       // int64 [n]
  size_t tiles = 0;      // int32 [2t]     launch slots: (b, qt << 16 | head as uint32), b < 0 = empty
  size_t bytes = 0;
  static PrefillBlob make(int n, int64_t t);
  static size_t capacity(const Config &c);
};

struct RequestState {
  int32_t plen = -1;     // -1: not registered
  int64_t base = 0;
  int32_t t = 0;         // generated tokens already cached
};

struct DecodePlan {
  int32_t split_tokens = 0;        // keys of the longest split
  int32_t waves_per_block = kDecodeWavesPerBlock;  // launch shape, 1 .. kDecodeMaxWavesPerBlock
  std::vector<int32_t> split_off;  // n + 1
  std::vector<SplitDesc> splits;   // num_splits, entry-major
  int32_t num_splits() const { return (int32_t)splits.size(); }
};

constexpr int kNumXcds = 8;            // MI355X: workgroup i runs on XCD i mod 8
constexpr int kXcdAffinityGroups = 32; // (request, head) groups needed for affinity

struct PrefillPlan {
  int32_t tile = 0;
  int64_t total_tokens = 0;
  int32_t max_len = 0;
  std::vector<int64_t> cu;         // n + 1
  // Launch order of (query tile, head) blocks: slot i holds
  // (b, qt << 16 | head, packed unsigned), or b = -1 for an empty slot.  Slot i runs on XCD
  // i mod 8; each XCD's slots hold whole (request, head) groups (when there
  // are enough of them) with the longest query tiles first, so blocks that
  // share keys and values run on the same L2.
  std::vector<int32_t> tiles;
  int64_t num_tiles() const { return (int64_t)tiles.size() / 2; }
};

// Call-order and ring bookkeeping of one handle.  Every check_* leaves the
// state untouched; the matching commit_* applies a checked call.
class HostState {
 public:
  explicit HostState(const Config &c);
  const Config &config() const { return cfg_; }

  // Prefill of rows start[i] .. start[i] + len[i] - 1 of each request's
  // prefill_len plen[i] (start / len null: the whole prefill).  Layer 0 at
  // start 0 registers the request (prefill_len, slot_base, t = 0); later
  // chunks continue where the layer stopped, and layer l needs layer l - 1
  // to have reached the chunk's end.
  int check_prefill(int32_t layer, int32_t n, const int32_t *ids, const int32_t *plen,
                    const int64_t *base, std::string *err, const int32_t *start = nullptr,
                    const int32_t *len = nullptr) const;
  void commit_prefill(int32_t layer, int32_t n, const int32_t *ids, const int32_t *plen,
                      const int64_t *base, const int32_t *start = nullptr,
                      const int32_t *len = nullptr);
  // Plans the packed offsets and the query tiles (of `tile` rows) of a
  // checked prefill call: len[b] rows per request starting at position
  // qoff[b] (null: 0).
  PrefillPlan plan_prefill(int32_t n, const int32_t *len, int32_t tile,
                           const int32_t *qoff = nullptr) const;
  // Rows of request id's prefill already in the cache at layer l.
  int32_t prefilled(int32_t id, int32_t layer) const { return done_[(size_t)id * cfg_.num_layers + layer]; }
  bool fully_prefilled(int32_t id) const;

  // Admission and retirement.  admit reserves P + W consecutive rows of the
  // pool (or slot-table) index space, first fit, for a request not yet
  // registered; retire unregisters requests outside the decode batch and
  // returns their reserved rows.
  int check_admit(int32_t id, int32_t plen, int64_t *base, std::string *err) const;
  void commit_admit(int32_t id, int32_t plen, int64_t base);
  int check_retire(int32_t n, const int32_t *ids, std::string *err) const;
  void commit_retire(int32_t n, const int32_t *ids);
  int64_t free_rows() const;
  // First logical slot any decode step of a request with prefill_len p may
  // attend to: 0, or with the standard-window baseline p - W + 1.
  int32_t decode_key0(int32_t p) const {
    return cfg_.attention == RSWA_ATTENTION_SWA ? std::max(0, p - cfg_.window + 1) : 0;
  }

  int check_set_batch(int32_t n, const int32_t *ids, std::string *err) const;
  DecodePlan plan_decode(int32_t n, const int32_t *ids) const;
  // Decode waves the device keeps resident at once (> 0).
  void set_resident_waves(int64_t w) { resident_waves_ = w > 0 ? w : kDefaultResidentWaves; }
  int64_t resident_waves() const { return resident_waves_; }
  void commit_set_batch(int32_t n, const int32_t *ids, DecodePlan plan);

  int check_ring_write(int32_t layer, std::string *err) const;
  void commit_ring_write(int32_t layer);
  int check_decode(int32_t layer, std::string *err) const;
  void commit_decode(int32_t layer);
  // Ring write and decode of one layer in one call.
  int check_fused(int32_t layer, std::string *err) const;
  void commit_fused(int32_t layer);
  int check_advance(std::string *err) const;
  void commit_advance();
  // The decode of `layer` completes this step's set of decoded layers, so
  // its kernel also advances the device copy of t (rswa_advance then only
  // updates the host view).
  bool completes_step(int32_t layer) const;
  // Every layer of the open step is decoded: the device t of the batch is
  // already one ahead of the host's until rswa_advance.
  bool step_decoded() const;
  // `steps` whole decode steps of the current batch ran outside the
  // library's calls (a replayed graph of them).  Needs a capture of decode
  // work since the last rswa_set_batch: a graph captured before it holds the
  // old batch's size, split count and tables.
  int check_note_steps(int32_t steps, std::string *err) const;
  void commit_note_steps(int32_t steps);
  // Decode work of the current batch was enqueued on a capturing stream.
  void note_capture() { captured_epoch_ = (int64_t)epoch_; }
  // Number of rswa_set_batch calls committed so far.
  uint64_t batch_epoch() const { return epoch_; }

  const RequestState &request(int32_t id) const { return req_[id]; }
  const std::vector<int32_t> &batch() const { return batch_; }
  const DecodePlan &plan() const { return plan_; }
  bool step_open() const;

  // Closed forms of the ring bookkeeping for a request with t generated
  // tokens already cached.
  static int32_t ring_pos(int32_t t, int32_t w) { return t % w; }
  static int32_t cache_len(int32_t p, int32_t t, int32_t w) { return p + (t < w ? t : w); }
  static int32_t next_pos(int32_t p, int32_t t) { return p + t; }

 private:
  Config cfg_;
  std::vector<RequestState> req_;
  std::vector<int32_t> done_;                  // [max_requests][num_layers] rows prefilled
  std::map<int64_t, int64_t> free_;            // free row ranges: start -> length
  std::vector<std::pair<int64_t, int64_t>> admitted_;  // per id: (start, length), length 0 = none
  std::vector<uint8_t> in_batch_;
  std::vector<int32_t> batch_;
  DecodePlan plan_;
  std::vector<uint8_t> written_, decoded_;
  int64_t resident_waves_ = kDefaultResidentWaves;
  uint64_t epoch_ = 0;           // committed rswa_set_batch calls
  int64_t captured_epoch_ = -1;  // epoch of the last captured decode work
};

}  // namespace rswa
