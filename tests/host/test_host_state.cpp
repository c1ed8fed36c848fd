// CPU test of the host-side R-SWA state machine and planners (no HIP).
// Built with g++ and AddressSanitizer/UBSan by tests/test_host_state.py.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <map>
#include <tuple>
#include <set>
#include <string>
#include <vector>

#include "host_state.hpp"

using namespace rswa;

static int g_fail = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "%s:%d CHECK failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static rswa_config base_cfg() {
  rswa_config c{};
  c.num_layers = 2;
  c.num_heads = 10;
  c.head_dim = 128;
  c.window = 8;
  c.max_positions = 1000;
  c.max_requests = 4;
  c.num_slots = 4000;
  c.dtype = RSWA_DTYPE_BF16;
  return c;
}

static Config resolved(const rswa_config &in) {
  Config c;
  std::string err;
  int rc = resolve_config(in, &c, &err);
  if (rc != RSWA_OK) std::fprintf(stderr, "resolve: %s\n", err.c_str());
  CHECK(rc == RSWA_OK);
  return c;
}

static void test_config() {
  std::string err;
  Config out;
  auto bad = [&](auto mut, int code) {
    rswa_config c = base_cfg();
    mut(c);
    int rc = resolve_config(c, &out, &err);
    CHECK(rc == code);
    CHECK(!err.empty());
    err.clear();
  };
  bad([](rswa_config &c) { c.num_layers = 0; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.num_heads = 0; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.head_dim = 96; }, RSWA_E_UNSUPPORTED);
  bad([](rswa_config &c) { c.dtype = 7; }, RSWA_E_UNSUPPORTED);
  bad([](rswa_config &c) { c.window = 0; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.window = 2000; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.max_requests = 0; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.num_slots = 0; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.max_splits = 2; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.decode_split_tokens = 100; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.rope_base = -1; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.slot_table_len = 5; }, RSWA_E_ARG);
  bad([](rswa_config &c) { c.slot_table = (const int32_t *)16; c.slot_table_len = 0; }, RSWA_E_ARG);
  rswa_config c = base_cfg();
  c.max_positions = 0;
  c.rope_base = 0;
  c.softmax_scale = 0;
  Config r = resolved(c);
  CHECK(r.max_positions == 32768);
  CHECK(r.rope_base == 10000.0);
  CHECK(r.softmax_scale > 0.0883 && r.softmax_scale < 0.0884);
  CHECK(r.max_splits == 16384);
}

static void test_layout() {
  Config c = resolved(base_cfg());
  Layout L = make_layout(c);
  struct R { size_t off, len; };
  std::vector<R> rs = {
      {L.rope, sizeof(float) * 2 * c.max_positions * (c.head_dim / 2)},
      {L.req_p, 4u * c.max_requests},
      {L.req_t, 4u * c.max_requests},
      {L.req_base, 8u * c.max_requests},
      {L.batch, L.batch_bytes},
      {L.part_o, sizeof(float) * c.max_splits * c.num_heads * c.head_dim},
      {L.part_ml, sizeof(float) * 2 * c.max_splits * c.num_heads},
      {L.merge_cnt, 4u * c.max_requests * c.num_heads},
      {L.step_cnt, 4u * c.max_requests},
      {L.prefill, L.prefill_bytes}};
  std::sort(rs.begin(), rs.end(), [](R a, R b) { return a.off < b.off; });
  for (size_t i = 0; i < rs.size(); ++i) {
    CHECK(rs[i].off % kAlign == 0);
    CHECK(rs[i].off + rs[i].len <= (i + 1 < rs.size() ? rs[i + 1].off : L.total));
  }
  // blobs fit their regions at capacity
  CHECK(BatchBlob::make(c.max_requests, c.max_splits).bytes <= L.batch_bytes);
  CHECK(PrefillBlob::make(c.max_requests, c.max_prefill_tiles()).bytes <= L.prefill_bytes);
}

static void test_prefill_order_and_errors() {
  Config c = resolved(base_cfg());
  HostState st(c);
  std::string err;
  int32_t ids[2] = {0, 3};
  int32_t pl[2] = {100, 0};
  int64_t base[2] = {0, 200};
  CHECK(st.check_prefill(1, 2, ids, pl, base, &err) == RSWA_E_STATE);  // not registered
  CHECK(st.check_prefill(2, 2, ids, pl, base, &err) == RSWA_E_ARG);    // layer out of range
  int32_t dup[2] = {1, 1};
  CHECK(st.check_prefill(0, 2, dup, pl, base, &err) == RSWA_E_ARG);
  int32_t badid[2] = {0, 4};
  CHECK(st.check_prefill(0, 2, badid, pl, base, &err) == RSWA_E_ARG);
  int32_t plbig[2] = {1001, 0};
  CHECK(st.check_prefill(0, 2, ids, plbig, base, &err) == RSWA_E_POSITION);
  int64_t basebig[2] = {0, 4000 - 8 + 1};
  CHECK(st.check_prefill(0, 2, ids, pl, basebig, &err) == RSWA_E_CAPACITY);
  int64_t baseedge[2] = {0, 4000 - 8};
  CHECK(st.check_prefill(0, 2, ids, pl, baseedge, &err) == RSWA_OK);
  int32_t plneg[2] = {-1, 0};
  CHECK(st.check_prefill(0, 2, ids, plneg, base, &err) == RSWA_E_ARG);
  // a failed check changed nothing
  CHECK(st.request(0).plen == -1);

  CHECK(st.check_prefill(0, 2, ids, pl, base, &err) == RSWA_OK);
  st.commit_prefill(0, 2, ids, pl, base);
  CHECK(st.request(0).plen == 100 && st.prefilled(0, 0) == 100 && st.prefilled(0, 1) == 0 &&
        st.request(0).t == 0);
  int32_t pl2[2] = {101, 0};
  CHECK(st.check_prefill(1, 2, ids, pl2, base, &err) == RSWA_E_STATE);  // P differs
  CHECK(st.check_set_batch(2, ids, &err) == RSWA_E_STATE);              // layer 1 missing
  CHECK(st.check_prefill(1, 2, ids, pl, base, &err) == RSWA_OK);
  st.commit_prefill(1, 2, ids, pl, base);
  CHECK(st.check_prefill(1, 2, ids, pl, base, &err) == RSWA_E_STATE);   // layer 1 again
  CHECK(st.check_set_batch(2, ids, &err) == RSWA_OK);
  // prefill plan: every (query tile, head) block once, empty slots marked
  PrefillPlan pp = st.plan_prefill(2, pl, 64);
  CHECK(pp.total_tokens == 100 && pp.cu[1] == 100 && pp.cu[2] == 100);
  std::set<std::tuple<int, int, int>> seen;
  for (int64_t i = 0; i < pp.num_tiles(); ++i) {
    const int b = pp.tiles[2 * i];
    if (b < 0) continue;
    CHECK(seen.insert({b, pp.tiles[2 * i + 1] >> 16, pp.tiles[2 * i + 1] & 0xffff}).second);
  }
  CHECK(seen.size() == 2 * 10);  // request 0: 2 tiles x 10 heads; request 3 is empty
  CHECK(pp.num_tiles() <= 24);
}

// With many (request, head) groups every group stays on one XCD (slot i runs
// on XCD i mod 8), its query tiles longest first, and XCD work is balanced.
static void test_prefill_xcd_plan() {
  rswa_config rc = base_cfg();
  rc.max_requests = 64;
  rc.max_positions = 32768;
  rc.num_slots = 64 * 9000;
  rc.max_prefill_tokens = 1 << 20;
  Config c = resolved(rc);
  HostState st(c);
  std::vector<int32_t> pl(64);
  for (int i = 0; i < 64; ++i) pl[i] = 272 + (i * 7919) % 8000;
  PrefillPlan pp = st.plan_prefill(64, pl.data(), 128);
  std::map<std::pair<int, int>, std::vector<std::pair<int64_t, int>>> where;
  std::vector<int64_t> work(8, 0);
  int64_t items = 0;
  for (int64_t i = 0; i < pp.num_tiles(); ++i) {
    const int b = pp.tiles[2 * i];
    if (b < 0) continue;
    const int qt = pp.tiles[2 * i + 1] >> 16, h = pp.tiles[2 * i + 1] & 0xffff;
    where[{b, h}].push_back({i, qt});
    work[i % 8] += qt + 1;
    ++items;
  }
  int64_t expect = 0;
  for (int i = 0; i < 64; ++i) expect += 10 * ((pl[i] + 127) / 128);
  CHECK(items == expect);
  CHECK((int64_t)where.size() == 640);
  for (auto &kv : where) {
    const auto &v = kv.second;
    CHECK((int)v.size() == (pl[kv.first.first] + 127) / 128);
    for (size_t k = 0; k < v.size(); ++k) {
      CHECK(v[k].first % 8 == v[0].first % 8);      // one XCD
      CHECK(v[k].second == (int)(v.size() - 1 - k));  // longest first
    }
  }
  const int64_t mx = *std::max_element(work.begin(), work.end());
  const int64_t mn = *std::min_element(work.begin(), work.end());
  CHECK(mx - mn <= mx / 50);  // within 2 %
  CHECK(pp.num_tiles() <= c.max_prefill_blocks());
}

static void register_all(HostState &st, int n, const int32_t *ids, const int32_t *pl,
                         const int64_t *base) {
  std::string err;
  for (int l = 0; l < st.config().num_layers; ++l) {
    CHECK(st.check_prefill(l, n, ids, pl, base, &err) == RSWA_OK);
    st.commit_prefill(l, n, ids, pl, base);
  }
}

static void test_step_machine_and_ring() {
  rswa_config rc = base_cfg();
  rc.max_positions = 120;
  Config c = resolved(rc);
  HostState st(c);
  std::string err;
  int32_t ids[2] = {2, 0};
  int32_t pl[2] = {5, 100};
  int64_t base[2] = {0, 50};
  register_all(st, 2, ids, pl, base);
  CHECK(st.check_ring_write(0, &err) == RSWA_E_STATE);  // no batch
  CHECK(st.check_set_batch(2, ids, &err) == RSWA_OK);
  st.commit_set_batch(2, ids, st.plan_decode(2, ids));
  // in-batch requests cannot be re-prefilled
  CHECK(st.check_prefill(0, 2, ids, pl, base, &err) == RSWA_E_STATE);

  std::deque<int> fifo;  // generated indices resident in request 2's ring
  for (int s = 0; s < 20; ++s) {
    const RequestState &r = st.request(2);
    // closed forms against a FIFO of generated tokens
    CHECK(HostState::ring_pos(r.t, c.window) == s % c.window);
    CHECK(HostState::next_pos(r.plen, r.t) == 5 + s);
    CHECK(HostState::cache_len(r.plen, r.t, c.window) == 5 + (int)fifo.size());
    CHECK(st.check_decode(0, &err) == RSWA_E_STATE);  // write first
    CHECK(st.check_advance(&err) == RSWA_E_STATE);
    CHECK(st.check_ring_write(0, &err) == RSWA_OK);
    st.commit_ring_write(0);
    CHECK(st.check_ring_write(0, &err) == RSWA_E_STATE);  // twice
    CHECK(st.check_set_batch(2, ids, &err) == RSWA_E_STATE);  // mid-step
    CHECK(st.check_decode(0, &err) == RSWA_OK);
    st.commit_decode(0);
    CHECK(st.check_decode(0, &err) == RSWA_E_STATE);
    CHECK(st.check_advance(&err) == RSWA_E_STATE);  // layer 1 missing
    CHECK(st.check_ring_write(1, &err) == RSWA_OK);
    st.commit_ring_write(1);
    CHECK(st.check_decode(1, &err) == RSWA_OK);
    st.commit_decode(1);
    CHECK(st.check_advance(&err) == RSWA_OK);
    st.commit_advance();
    fifo.push_back(s);
    if ((int)fifo.size() > c.window) fifo.pop_front();
  }
  CHECK(st.request(2).t == 20 && st.request(0).t == 20);
  CHECK(HostState::cache_len(5, 20, 8) == 13);
  // request 0 (P = 100) reaches position 120 = max_positions after 20 steps
  CHECK(st.check_ring_write(0, &err) == RSWA_E_POSITION);
  CHECK(st.check_fused(0, &err) == RSWA_E_POSITION);
  CHECK(st.request(0).t == 20);
}

// A fused ring write + decode counts as both calls for its layer.
static void test_fused_step() {
  Config c = resolved(base_cfg());
  HostState st(c);
  std::string err;
  int32_t ids[1] = {1};
  int32_t pl[1] = {7};
  int64_t base[1] = {0};
  register_all(st, 1, ids, pl, base);
  st.commit_set_batch(1, ids, st.plan_decode(1, ids));
  CHECK(st.check_fused(0, &err) == RSWA_OK);
  st.commit_fused(0);
  CHECK(st.check_fused(0, &err) == RSWA_E_STATE);
  CHECK(st.check_decode(0, &err) == RSWA_E_STATE);
  CHECK(st.check_ring_write(0, &err) == RSWA_E_STATE);
  CHECK(st.check_advance(&err) == RSWA_E_STATE);  // layer 1 missing
  CHECK(st.check_ring_write(1, &err) == RSWA_OK);
  st.commit_ring_write(1);
  CHECK(st.check_fused(1, &err) == RSWA_E_STATE);  // already written
  CHECK(st.check_decode(1, &err) == RSWA_OK);
  st.commit_decode(1);
  CHECK(st.check_advance(&err) == RSWA_OK);
  st.commit_advance();
  CHECK(st.request(1).t == 1);
  // graph replay bookkeeping: whole steps only, positions checked, and only
  // for a graph captured since the last rswa_set_batch
  CHECK(st.check_note_steps(3, &err) == RSWA_E_STATE);  // nothing captured
  st.note_capture();
  CHECK(st.check_note_steps(3, &err) == RSWA_OK);
  st.commit_note_steps(3);
  CHECK(st.request(1).t == 4);
  CHECK(st.check_note_steps(-1, &err) == RSWA_E_ARG);
  CHECK(st.check_ring_write(0, &err) == RSWA_OK);
  st.commit_ring_write(0);
  CHECK(st.check_note_steps(1, &err) == RSWA_E_STATE);  // step half done
  st.commit_decode(0);
  st.commit_fused(1);
  st.commit_advance();
  CHECK(st.request(1).t == 5);
  const int32_t room = st.config().max_positions - (7 + 5);
  CHECK(st.check_note_steps(room, &err) == RSWA_OK);
  CHECK(st.check_note_steps(room + 1, &err) == RSWA_E_POSITION);
  // a new batch (even the same ids) invalidates the captured graph
  const uint64_t e0 = st.batch_epoch();
  CHECK(st.check_set_batch(1, ids, &err) == RSWA_OK);
  st.commit_set_batch(1, ids, st.plan_decode(1, ids));
  CHECK(st.batch_epoch() == e0 + 1);
  CHECK(st.check_note_steps(1, &err) == RSWA_E_STATE);
  st.note_capture();
  CHECK(st.check_note_steps(1, &err) == RSWA_OK);
}

// Query-tile indices up to 65535 (64-row tiles of a 4194304-position prefill)
// survive the (qt << 16 | head) packing when unpacked unsigned.
static void test_prefill_tile_index_limit() {
  rswa_config rc = base_cfg();
  rc.num_heads = 1;
  rc.head_dim = 64;
  rc.dtype = RSWA_DTYPE_F32;
  rc.window = 1;
  rc.max_requests = 1;
  rc.max_positions = 1 << 22;
  rc.num_slots = (1 << 22) + 1;
  rc.max_prefill_tokens = 1 << 22;
  Config c = resolved(rc);
  HostState st(c);
  int32_t len[1] = {1 << 22};
  PrefillPlan pp = st.plan_prefill(1, len, 64);
  std::vector<uint8_t> seen(65536, 0);
  int64_t items = 0;
  for (int64_t i = 0; i < pp.num_tiles(); ++i) {
    if (pp.tiles[2 * i] < 0) continue;
    const uint32_t slot = (uint32_t)pp.tiles[2 * i + 1];
    const uint32_t qt = slot >> 16, h = slot & 0xffffu;
    CHECK(h == 0);
    CHECK(qt < 65536);
    if (qt < 65536) seen[qt] += 1;
    ++items;
  }
  CHECK(items == 65536);
  CHECK(std::count(seen.begin(), seen.end(), 1) == 65536);
  CHECK(pp.num_tiles() <= c.max_prefill_blocks());
}

// Splits of request i tile its key range [key0, P + W) exactly, in order:
// split_tokens keys each (a multiple of 64), the last one the remainder.
static void check_tiling(const DecodePlan &p, int n, const int32_t *pl, const int64_t *base,
                         int window, int32_t (*key0)(int32_t)) {
  CHECK((int)p.split_off.size() == n + 1 && p.split_off[n] == p.num_splits());
  int32_t longest = 0;
  for (int i = 0; i < n; ++i) {
    int32_t next = key0(pl[i]);
    for (int j = p.split_off[i]; j < p.split_off[i + 1]; ++j) {
      const SplitDesc &d = p.splits[j];
      CHECK(d.b == i && d.p == pl[i] && d.base == base[i]);
      CHECK(d.k0 == next && d.k1 > d.k0);
      CHECK(d.k1 - d.k0 == p.split_tokens || j + 1 == p.split_off[i + 1]);
      CHECK(d.k1 - d.k0 <= p.split_tokens);
      longest = std::max(longest, d.k1 - d.k0);
      next = d.k1;
    }
    CHECK(next == pl[i] + window);
  }
  CHECK(p.split_tokens == longest);
}

static int32_t rswa_key0(int32_t) { return 0; }
static int32_t swa_key0(int32_t p) { return std::max(0, p - 127); }

static void test_decode_plan() {
  rswa_config rc = base_cfg();
  rc.max_positions = 32768;
  rc.max_requests = 64;
  rc.num_slots = 64 * 40000;
  rc.window = 128;
  rc.max_prefill_tokens = 1 << 20;
  Config c = resolved(rc);
  HostState st(c);
  std::vector<int32_t> ids(64), pl(64);
  std::vector<int64_t> base(64);
  int64_t b = 0;
  for (int i = 0; i < 64; ++i) {
    ids[i] = i;
    pl[i] = 272 + (i * 7919) % 8000;
    base[i] = b;
    b += pl[i] + 128;
  }
  register_all(st, 64, ids.data(), pl.data(), base.data());
  DecodePlan p = st.plan_decode(64, ids.data());
  check_tiling(p, 64, pl.data(), base.data(), 128, rswa_key0);
  for (int j = 0; j < p.num_splits(); ++j) CHECK(p.splits[j].r == ids[p.splits[j].b]);
  // 64 requests x ~4.4k keys x 10 heads is beyond one round: 1024-key
  // splits, lengthened (in 64-key steps) until every wave is resident at once.
  CHECK(st.resident_waves() == kDefaultResidentWaves);
  CHECK(p.split_tokens > kLongSplitKeys && p.split_tokens % kSplitQuantum == 0);
  CHECK(p.num_splits() * 10 <= st.resident_waves());
  // all resident: blocks of as many waves as a CU holds, one block per CU
  CHECK(p.waves_per_block == kDecodeMaxWavesPerBlock);
  CHECK((p.num_splits() * 10 + p.waves_per_block - 1) / p.waves_per_block <= kDecodeCUs);
  {
    // one 64-key step shorter would not fit
    int64_t k = 0;
    for (int i = 0; i < 64; ++i) k += (pl[i] + 128 + p.split_tokens - 65) / (p.split_tokens - 64);
    CHECK(k * 10 > st.resident_waves());
  }
  // With room for every 1024-key split's wave the split stays at 1024 keys.
  st.set_resident_waves(int64_t(1) << 20);
  CHECK(st.plan_decode(64, ids.data()).split_tokens == kLongSplitKeys);
  st.set_resident_waves(0);  // back to the built-in figure
  CHECK(st.resident_waves() == kDefaultResidentWaves);
  // A batch that fits one round gets the shortest 64-multiple splits that
  // keep it within kDecodeWaves waves: 8 x 4288 keys x 10 heads -> 384-key
  // splits, 12 per request (960 waves, 240 blocks).
  {
    rswa_config r2 = base_cfg();
    r2.max_positions = 32768;
    r2.max_requests = 8;
    r2.window = 128;
    r2.num_slots = 8 * 4288;
    r2.max_prefill_tokens = 1 << 20;
    HostState s8(resolved(r2));
    std::vector<int32_t> i8(8), p8(8, 4160);
    std::vector<int64_t> b8(8);
    for (int i = 0; i < 8; ++i) {
      i8[i] = i;
      b8[i] = (int64_t)i * 4288;
    }
    register_all(s8, 8, i8.data(), p8.data(), b8.data());
    DecodePlan q = s8.plan_decode(8, i8.data());
    check_tiling(q, 8, p8.data(), b8.data(), 128, rswa_key0);
    CHECK(q.num_splits() * 10 <= kDecodeCUs * kDecodeWavesPerBlock);
    CHECK(q.split_tokens == 384 && q.split_off[1] == 12);
    CHECK(q.waves_per_block == kDecodeWavesPerBlock);  // 960 waves: 240 blocks of four
  }
  // Forced split size: fixed-length splits, the last one shorter; a
  // too-small max_splits is reported.
  rc.decode_split_tokens = 64;
  rc.max_splits = 100;
  Config c2 = resolved(rc);
  HostState st2(c2);
  register_all(st2, 64, ids.data(), pl.data(), base.data());
  std::string err;
  CHECK(st2.check_set_batch(64, ids.data(), &err) == RSWA_E_CAPACITY);
  DecodePlan p2 = st2.plan_decode(64, ids.data());
  check_tiling(p2, 64, pl.data(), base.data(), 128, rswa_key0);
  CHECK(p2.split_tokens == 64);
  for (int i = 0; i < 64; ++i) CHECK(p2.split_off[i + 1] - p2.split_off[i] == (pl[i] + 128 + 63) / 64);
  rc.decode_split_tokens = 0;
  Config c3 = resolved(rc);
  HostState st3(c3);
  register_all(st3, 64, ids.data(), pl.data(), base.data());
  CHECK(st3.check_set_batch(64, ids.data(), &err) == RSWA_OK);
  CHECK(st3.plan_decode(64, ids.data()).num_splits() <= 100);
  // Standard-window baseline: splits tile P - W + 1 .. P + W - 1 only.
  rc.attention = RSWA_ATTENTION_SWA;
  rc.decode_split_tokens = 64;
  rc.max_splits = 0;
  Config c4 = resolved(rc);
  HostState st4(c4);
  register_all(st4, 64, ids.data(), pl.data(), base.data());
  CHECK(st4.check_set_batch(64, ids.data(), &err) == RSWA_OK);
  DecodePlan p4 = st4.plan_decode(64, ids.data());
  check_tiling(p4, 64, pl.data(), base.data(), 128, swa_key0);
  for (int i = 0; i < 64; ++i) {
    CHECK(st4.decode_key0(pl[i]) == pl[i] - 127);
    CHECK(p4.split_off[i + 1] - p4.split_off[i] == (2 * 128 - 1 + 63) / 64);
  }
  // a short prompt: the window reaches back to slot 0
  CHECK(st4.decode_key0(50) == 0);
  CHECK(st.decode_key0(5000) == 0);  // R-SWA: every prefill key
  rc.attention = 2;
  rswa_config bad = rc;
  Config out;
  CHECK(resolve_config(bad, &out, &err) == RSWA_E_ARG);
}

// The decode of the layer that completes a step advances t on the device.
static void test_step_completion() {
  Config c = resolved(base_cfg());  // 2 layers
  HostState st(c);
  int32_t ids[1] = {0};
  int32_t pl[1] = {10};
  int64_t base[1] = {0};
  register_all(st, 1, ids, pl, base);
  st.commit_set_batch(1, ids, st.plan_decode(1, ids));
  CHECK(!st.step_decoded());
  CHECK(!st.completes_step(0) && !st.completes_step(1));  // two layers to go
  st.commit_fused(1);
  CHECK(st.completes_step(0) && !st.completes_step(1));
  CHECK(!st.step_decoded());
  st.commit_fused(0);
  CHECK(st.step_decoded());
  st.commit_advance();
  CHECK(!st.step_decoded() && st.request(0).t == 1);
}

static void test_chunked_prefill() {
  Config c = resolved(base_cfg());
  HostState st(c);
  std::string err;
  int32_t id[1] = {2};
  int32_t pl[1] = {100};
  int64_t base[1] = {0};
  auto chunk = [&](int layer, int s0, int ln) {
    int32_t a[1] = {s0}, b[1] = {ln};
    int rc = st.check_prefill(layer, 1, id, pl, base, &err, a, b);
    if (rc == RSWA_OK) st.commit_prefill(layer, 1, id, pl, base, a, b);
    return rc;
  };
  CHECK(chunk(0, 10, 20) == RSWA_E_STATE);   // not registered: the first chunk starts at 0
  CHECK(chunk(0, 0, 101) == RSWA_E_ARG);     // past prefill_len
  CHECK(chunk(0, 0, 40) == RSWA_OK);
  CHECK(st.prefilled(2, 0) == 40 && st.request(2).plen == 100);
  CHECK(chunk(0, 50, 10) == RSWA_E_STATE);   // gap
  CHECK(chunk(1, 0, 41) == RSWA_E_STATE);    // layer 0 holds only 40 rows
  CHECK(chunk(1, 0, 40) == RSWA_OK);
  CHECK(chunk(0, 40, 60) == RSWA_OK);
  int32_t ids[1] = {2};
  CHECK(st.check_set_batch(1, ids, &err) == RSWA_E_STATE);  // layer 1 incomplete
  CHECK(chunk(1, 40, 0) == RSWA_OK);         // empty chunk is fine
  CHECK(chunk(1, 40, 60) == RSWA_OK);
  CHECK(st.fully_prefilled(2));
  CHECK(st.check_set_batch(1, ids, &err) == RSWA_OK);
  // a new layer-0 chunk at 0 re-registers and clears the other layers
  CHECK(chunk(0, 0, 30) == RSWA_OK);
  CHECK(st.prefilled(2, 0) == 30 && st.prefilled(2, 1) == 0 && !st.fully_prefilled(2));
  // plan of a chunk at offset 4096: tiles over the chunk rows only
  int32_t len[2] = {300, 64};
  int32_t off[2] = {4096, 0};
  PrefillPlan pp = st.plan_prefill(2, len, 128, off);
  int64_t blocks = 0;
  for (int64_t i = 0; i < pp.num_tiles(); ++i) blocks += pp.tiles[2 * i] >= 0;
  CHECK(blocks == (3 + 1) * 10 && pp.total_tokens == 364);
}

// Admission and retirement: first-fit ranges of P + W rows, merged on release.
static void test_admission() {
  Config c = resolved(base_cfg());
  HostState st(c);
  std::string err;
  const int64_t cap = c.row_capacity();
  CHECK(st.free_rows() == cap);
  int64_t b5 = -1, b6 = -1, b7 = -1;
  CHECK(st.check_admit(0, 100, &b5, &err) == RSWA_OK);
  st.commit_admit(0, 100, b5);
  CHECK(b5 == 0);
  CHECK(st.check_admit(1, 50, &b6, &err) == RSWA_OK);
  st.commit_admit(1, 50, b6);
  CHECK(b6 == 108);  // W = 8
  CHECK(st.free_rows() == cap - 108 - 58);
  CHECK(st.check_admit(0, 10, &b7, &err) == RSWA_E_STATE);   // already admitted
  CHECK(st.check_admit(2, (int32_t)cap, &b7, &err) == RSWA_E_POSITION);
  // prefill must use the admitted base
  int32_t id5[1] = {0};
  int32_t pl5[1] = {100};
  int64_t wrong[1] = {8};
  CHECK(st.check_prefill(0, 1, id5, pl5, wrong, &err) == RSWA_E_ARG);
  int64_t right[1] = {b5};
  CHECK(st.check_prefill(0, 1, id5, pl5, right, &err) == RSWA_OK);
  st.commit_prefill(0, 1, id5, pl5, right);
  int32_t both[2] = {0, 1};
  CHECK(st.check_retire(2, both, &err) == RSWA_OK);
  st.commit_retire(1, id5);
  CHECK(st.request(0).plen == -1 && st.prefilled(0, 0) == 0);
  CHECK(st.free_rows() == cap - 58);
  CHECK(st.check_admit(2, 90, &b7, &err) == RSWA_OK);      // first fit: the freed front
  st.commit_admit(2, 90, b7);
  CHECK(b7 == 0);
  int32_t id67[2] = {1, 2};
  st.commit_retire(2, id67);
  CHECK(st.free_rows() == cap);
  int64_t whole = -1;
  CHECK(st.check_admit(3, (int32_t)std::min<int64_t>(cap - 8, c.max_positions), &whole, &err) == RSWA_OK);
  CHECK(whole == 0);  // the ranges merged back into one
  CHECK(st.check_retire(1, nullptr, &err) == RSWA_E_ARG);
}

// Seeded random batches (heads, window, batch size and prefill lengths,
// including empty prefills): the decode plan tiles every request's keys
// exactly once and keeps the split-size rules; the prefill plan launches
// every (request, query tile, head) block exactly once, each (request, head)
// group on one XCD with its longest tiles first when there are enough groups.
// The launch shape the decode plan picks for its wave count.
static void check_launch_shape(const DecodePlan &p, int64_t heads, int64_t resident) {
  const int64_t tasks = (int64_t)p.num_splits() * heads;
  const int64_t wpb = p.waves_per_block;
  const int64_t per_cu = std::min<int64_t>(kDecodeMaxWavesPerBlock, std::max<int64_t>(1, resident / kDecodeCUs));
  CHECK(wpb >= 1 && wpb <= per_cu);
  const int64_t blocks = (tasks + wpb - 1) / wpb;
  // at most one block per CU whenever a CU can hold the waves that needs,
  // with the fewest waves per block that achieve it
  if (tasks <= per_cu * kDecodeCUs) CHECK(blocks <= kDecodeCUs);
  if (wpb > 1) CHECK((tasks + wpb - 2) / (wpb - 1) > kDecodeCUs);
  if (tasks <= kDecodeCUs) CHECK(wpb == 1);
  if (tasks > kDecodeCUs * (kDecodeWavesPerBlock - 1) && tasks <= kDecodeWaves)
    CHECK(wpb == kDecodeWavesPerBlock);
}

static void test_plans_randomized() {
  uint64_t s = 0x9e3779b97f4a7c15ull;
  auto rnd = [&](int lo, int hi) {  // xorshift64, uniform enough in [lo, hi]
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return lo + (int)(s % (uint64_t)(hi - lo + 1));
  };
  const int windows[] = {1, 2, 8, 128, 300};
  int one_round = 0, long_splits = 0, by_group = 0, by_block = 0;  // cases seen per rule
  for (int it = 0; it < 300; ++it) {
    rswa_config rc = base_cfg();
    rc.num_layers = 1;
    rc.num_heads = rnd(1, 16);
    rc.window = windows[rnd(0, 4)];
    const int n = rnd(1, 64);
    rc.max_requests = n;
    rc.max_positions = 32768;
    std::vector<int32_t> ids(n), pl(n);
    std::vector<int64_t> base(n);
    int64_t rows = 0, tokens = 0;
    for (int i = 0; i < n; ++i) {
      ids[i] = i;
      pl[i] = rnd(0, 1) ? rnd(0, 300) : rnd(1, 20000);
      base[i] = rows;
      rows += pl[i] + rc.window;
      tokens += pl[i];
    }
    rc.num_slots = rows;
    rc.max_prefill_tokens = std::max<int64_t>(1, tokens);
    HostState st(resolved(rc));
    register_all(st, n, ids.data(), pl.data(), base.data());
    const int64_t heads = rc.num_heads;

    const DecodePlan p = st.plan_decode(n, ids.data());
    check_tiling(p, n, pl.data(), base.data(), rc.window, rswa_key0);
    check_launch_shape(p, heads, st.resident_waves());
    int64_t keys = 0, longest = 0;
    for (int i = 0; i < n; ++i) {
      keys += pl[i] + rc.window;
      longest = std::max<int64_t>(longest, pl[i] + rc.window);
    }
    CHECK(p.num_splits() <= st.config().max_splits);
    const int64_t sz = p.split_tokens;
    if (sz < longest) {
      // a forced split size: a multiple of 64 that fits the rule it follows
      CHECK(sz % kSplitQuantum == 0);
      if (keys * heads <= kOneRoundKeys) {
        CHECK(p.num_splits() * heads <= kDecodeWaves || p.num_splits() == st.config().max_splits);
        ++one_round;
      } else {
        CHECK(sz >= kLongSplitKeys);
        ++long_splits;
      }
    }

    for (int tile : {64, 256}) {
      const PrefillPlan pp = st.plan_prefill(n, pl.data(), tile);
      std::set<std::tuple<int, int, int>> seen;
      std::map<std::pair<int, int>, std::vector<std::pair<int64_t, int>>> where;
      for (int64_t i = 0; i < pp.num_tiles(); ++i) {
        const int b = pp.tiles[2 * i];
        if (b < 0) continue;
        const uint32_t slot = (uint32_t)pp.tiles[2 * i + 1];
        const int qt = (int)(slot >> 16), h = (int)(slot & 0xffffu);
        CHECK(b < n && h < heads && qt * tile < pl[b]);
        CHECK(seen.insert({b, qt, h}).second);
        where[{b, h}].push_back({i, qt});
      }
      int64_t expect = 0;
      for (int i = 0; i < n; ++i) expect += heads * ((pl[i] + tile - 1) / tile);
      CHECK((int64_t)seen.size() == expect);
      CHECK(pp.num_tiles() <= st.config().max_prefill_blocks());
      CHECK(pp.num_tiles() == 0 || pp.tiles[2 * (pp.num_tiles() - 1)] >= 0);  // no trailing empty slot
      CHECK(pp.num_tiles() <= 2 * expect + 64);  // padding stays bounded
      bool grouped = true;
      for (auto &kv : where)
        for (size_t k = 0; k < kv.second.size(); ++k)
          grouped = grouped && kv.second[k].first % kNumXcds == kv.second[0].first % kNumXcds;
      if (grouped && (int64_t)where.size() >= kXcdAffinityGroups) ++by_group;
      if (!grouped) ++by_block;
      if (grouped) {
        // each (request, head) on one XCD: its query tiles longest first
        for (auto &kv : where)
          for (size_t k = 0; k < kv.second.size(); ++k)
            CHECK(kv.second[k].second == (int)(kv.second.size() - 1 - k));
      } else {
        // blocks assigned one by one, longest first: along each XCD's
        // slots the work (query tiles up to the block's) never grows
        for (int x = 0; x < kNumXcds; ++x) {
          int prev = 1 << 30;
          for (int64_t i = x; i < pp.num_tiles(); i += kNumXcds) {
            if (pp.tiles[2 * i] < 0) continue;
            const int w = (int)((uint32_t)pp.tiles[2 * i + 1] >> 16) + 1;
            CHECK(w <= prev);
            prev = w;
          }
        }
      }
    }
  }
  CHECK(one_round > 0 && long_splits > 0 && by_group > 0 && by_block > 0);
  std::printf("randomized plans: %d one-round, %d long-split decode plans; %d grouped, %d per-block prefill plans\n",
              one_round, long_splits, by_group, by_block);
}

int main() {
  test_config();
  test_layout();
  test_prefill_order_and_errors();
  test_prefill_xcd_plan();
  test_step_machine_and_ring();
  test_fused_step();
  test_prefill_tile_index_limit();
  test_decode_plan();
  test_plans_randomized();
  test_step_completion();
  test_chunked_prefill();
  test_admission();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host state: all checks passed\n");
  return 0;
}
