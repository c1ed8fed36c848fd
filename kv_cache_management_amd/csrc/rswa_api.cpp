// C ABI of the R-SWA library (declared in include/rswa.h): host validation
// through HostState, workspace carving, uploads through a pinned staging
// ring, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "host_state.hpp"
#include "kernels.hpp"
#include "rswa.h"

using rswa::Config;
using rswa::HostState;
using rswa::Layout;

namespace {

thread_local std::string g_last_error;
constexpr int kStages = 4;

int set_global_error(int code, const std::string &msg) {
  g_last_error = msg;
  return code;
}

// True while `s` is being captured into a graph.  A failed query (e.g. the
// legacy stream during another stream's global capture) counts as capturing:
// the calls that refuse capture then refuse, and launches fail on their own.
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return st != hipStreamCaptureStatusNone;
}

}  // namespace

struct rswa_cache {
  Config cfg;
  Layout lay;
  HostState st;
  void *k_pool = nullptr;
  void *v_pool = nullptr;
  char *ws = nullptr;
  float qscale = 0.f;
  std::string err;
  char *staging[kStages] = {};
  hipEvent_t staged[kStages] = {};
  bool staged_live[kStages] = {};
  int next_stage = 0;
  size_t stage_bytes = 0;

  explicit rswa_cache(const Config &c) : cfg(c), lay(rswa::make_layout(c)), st(c) {}

  int fail(int code, const std::string &msg) {
    err = msg;
    return code;
  }
  int hip_fail(hipError_t e, const char *what) {
    return fail(RSWA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
  }

  // Copy `bytes` of host data to device `dst` in stream order, through the
  // next pinned staging slot (waiting only if that slot's previous copy is
  // still pending).
  hipError_t upload(void *dst, const void *src, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const int k = next_stage;
    next_stage = (next_stage + 1) % kStages;
    if (staged_live[k]) {
      hipError_t e = hipEventSynchronize(staged[k]);
      if (e != hipSuccess) return e;
    }
    std::memcpy(staging[k], src, bytes);
    hipError_t e = hipMemcpyAsync(dst, staging[k], bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    e = hipEventRecord(staged[k], s);
    staged_live[k] = (e == hipSuccess);
    return e;
  }

  rswa::PoolArgs pool() const {
    return {k_pool, v_pool, cfg.num_slots * cfg.num_heads * cfg.head_dim, nullptr};
  }
  rswa::StateArgs state() const {
    return {(int32_t *)(ws + lay.req_p), (int32_t *)(ws + lay.req_t), (int64_t *)(ws + lay.req_base)};
  }
  const float2 *rope() const { return (const float2 *)(ws + lay.rope); }

  const int32_t *slot_table = nullptr;
  // Device address of the fixed scratch array on this handle's GPU
  // (rswa_decode_step_fused_noalloc), resolved at init; null if that failed.
  void *noalloc_scratch = nullptr;
  std::string noalloc_err;

  // Kernel timing (rswa_profile_*): event pairs per kernel kind, reused.
  bool prof = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_ev[RSWA_NUM_KERNELS];
  size_t prof_used[RSWA_NUM_KERNELS] = {};

  // Records the opening event of a timed launch; returns the pair index or -1.
  int prof_begin(int kernel, hipStream_t s) {
    if (!prof) return -1;
    auto &v = prof_ev[kernel];
    if (prof_used[kernel] == v.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return -1;
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return -1;
      }
      v.emplace_back(a, b);
    }
    const int i = (int)prof_used[kernel]++;
    (void)hipEventRecord(v[i].first, s);
    return i;
  }
  void prof_end(int kernel, int i, hipStream_t s) {
    if (i >= 0) (void)hipEventRecord(prof_ev[kernel][i].second, s);
  }
};

namespace {

template <typename F>
int guarded(rswa_cache *c, F &&f) {
  try {
    return f();
  } catch (const std::bad_alloc &) {
    return c ? c->fail(RSWA_E_CAPACITY, "host allocation failed")
             : set_global_error(RSWA_E_CAPACITY, "host allocation failed");
  } catch (...) {
    return c ? c->fail(RSWA_E_ARG, "internal error") : set_global_error(RSWA_E_ARG, "internal error");
  }
}

// Append `count` values of T at byte offset `off` of blob.
template <typename T>
void put(std::vector<char> &blob, size_t off, const T *src, size_t count) {
  if (count) std::memcpy(blob.data() + off, src, sizeof(T) * count);
}

}  // namespace

extern "C" {

int rswa_abi_version(void) { return RSWA_ABI_VERSION; }

const char *rswa_status_string(int status) {
  switch (status) {
    case RSWA_OK: return "RSWA_OK";
    case RSWA_E_ARG: return "RSWA_E_ARG";
    case RSWA_E_UNSUPPORTED: return "RSWA_E_UNSUPPORTED";
    case RSWA_E_POSITION: return "RSWA_E_POSITION";
    case RSWA_E_CAPACITY: return "RSWA_E_CAPACITY";
    case RSWA_E_STATE: return "RSWA_E_STATE";
    case RSWA_E_HIP: return "RSWA_E_HIP";
    default: return "RSWA_E_UNKNOWN";
  }
}

const char *rswa_last_error(const rswa_cache *c) {
  return c ? c->err.c_str() : g_last_error.c_str();
}

size_t rswa_workspace_bytes(const rswa_config *cfg) {
  if (!cfg) {
    set_global_error(RSWA_E_ARG, "null config");
    return 0;
  }
  Config c;
  std::string err;
  if (rswa::resolve_config(*cfg, &c, &err) != RSWA_OK) {
    set_global_error(RSWA_E_ARG, err);
    return 0;
  }
  return rswa::make_layout(c).total;
}

int rswa_cache_init(const rswa_config *cfg, void *k_pool, void *v_pool, void *workspace,
                    size_t workspace_bytes, void *stream, rswa_cache **out) {
  return guarded(nullptr, [&]() -> int {
    if (!out) return set_global_error(RSWA_E_ARG, "null output handle pointer");
    *out = nullptr;
    if (!cfg) return set_global_error(RSWA_E_ARG, "null config");
    Config c;
    std::string err;
    int rc = rswa::resolve_config(*cfg, &c, &err);
    if (rc != RSWA_OK) return set_global_error(rc, err);
    if (!k_pool || !v_pool || !workspace) return set_global_error(RSWA_E_ARG, "null pool or workspace");
    if (((uintptr_t)k_pool | (uintptr_t)v_pool) % 16)
      return set_global_error(RSWA_E_ARG, "pools must be 16-byte aligned");
    if ((uintptr_t)workspace % rswa::kAlign)
      return set_global_error(RSWA_E_ARG, "workspace must be 256-byte aligned");
    Layout lay = rswa::make_layout(c);
    if (workspace_bytes < lay.total)
      return set_global_error(RSWA_E_CAPACITY, "workspace has " + std::to_string(workspace_bytes) +
                                                   " bytes, needs " + std::to_string(lay.total));
    hipStream_t s = (hipStream_t)stream;

    // Slot table: every entry must name a pool row.
    if (c.has_table) {
      std::vector<int32_t> tab(c.slot_table_len);
      hipError_t e = hipStreamSynchronize(s);
      if (e == hipSuccess)
        e = hipMemcpy(tab.data(), cfg->slot_table, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost);
      if (e != hipSuccess)
        return set_global_error(RSWA_E_HIP, std::string("reading slot table: ") + hipGetErrorString(e));
      for (size_t i = 0; i < tab.size(); ++i)
        if (tab[i] < 0 || tab[i] >= c.num_slots)
          return set_global_error(RSWA_E_ARG, "slot_table[" + std::to_string(i) + "] = " +
                                                  std::to_string(tab[i]) + " is not a pool row");
    }

    // RoPE table, computed in fp64 and stored fp32: angle p * base^(-2i/D).
    const int half = c.head_dim / 2;
    std::vector<float> rope((size_t)c.max_positions * half * 2);
    std::vector<double> freq(half);
    for (int i = 0; i < half; ++i) freq[i] = std::pow(c.rope_base, -2.0 * i / c.head_dim);
    for (int64_t p = 0; p < c.max_positions; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * freq[i];
        rope[(p * half + i) * 2] = (float)std::cos(ang);
        rope[(p * half + i) * 2 + 1] = (float)std::sin(ang);
      }

    rswa_cache *h = new rswa_cache(c);
    h->k_pool = k_pool;
    h->v_pool = v_pool;
    h->ws = (char *)workspace;
    h->slot_table = cfg->slot_table;
    h->qscale = (float)(c.softmax_scale * 1.4426950408889634);  // scale * log2(e)
    h->stage_bytes = std::max(rswa::BatchBlob::capacity(c), rswa::PrefillBlob::capacity(c));
    auto cleanup = [&](hipError_t e, const char *what) {
      std::string msg = std::string(what) + ": " + hipGetErrorString(e);
      rswa_cache_destroy(h);
      return set_global_error(RSWA_E_HIP, msg);
    };
    for (int k = 0; k < kStages; ++k) {
      hipError_t e = hipHostMalloc((void **)&h->staging[k], h->stage_bytes, hipHostMallocDefault);
      if (e != hipSuccess) return cleanup(e, "hipHostMalloc");
      e = hipEventCreateWithFlags(&h->staged[k], hipEventDisableTiming);
      if (e != hipSuccess) return cleanup(e, "hipEventCreate");
    }
    hipError_t e = hipMemcpyAsync(h->ws + lay.rope, rope.data(), sizeof(float) * rope.size(),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->ws + lay.req_p, 0xff, sizeof(int32_t) * c.max_requests, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->ws + lay.req_t, 0, sizeof(int32_t) * c.max_requests, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->ws + lay.req_base, 0, sizeof(int64_t) * c.max_requests, s);
    // Merge and step counters start at zero; every decode launch leaves them so.
    if (e == hipSuccess)
      e = hipMemsetAsync(h->ws + lay.merge_cnt, 0, sizeof(int32_t) * (size_t)c.max_requests * c.num_heads, s);
    if (e == hipSuccess) e = hipMemsetAsync(h->ws + lay.step_cnt, 0, sizeof(int32_t) * c.max_requests, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return cleanup(e, "uploading the RoPE table");
    // How many decode waves fit on the device at once bounds the split
    // count the planner picks (a failed query keeps the built-in figure).
    int64_t resident = 0;
    if (rswa::decode_resident_waves(c.dtype, c.head_dim, &resident) == hipSuccess && resident > 0)
      h->st.set_resident_waves(resident);
    else
      (void)hipGetLastError();
    // Resolved here, once per device, for rswa_decode_step_fused_noalloc; a
    // failure only disables that entry point.
    e = rswa::noalloc_scratch_address(&h->noalloc_scratch);
    if (e != hipSuccess) {
      h->noalloc_scratch = nullptr;
      h->noalloc_err = std::string("hipGetSymbolAddress of the fixed scratch: ") + hipGetErrorString(e);
    }
    *out = h;
    return RSWA_OK;
  });
}

int rswa_cache_destroy(rswa_cache *c) {
  if (!c) return RSWA_OK;
  for (auto &v : c->prof_ev)
    for (auto &pr : v) {
      (void)hipEventSynchronize(pr.second);
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  for (int k = 0; k < kStages; ++k) {
    if (c->staged[k]) {
      if (c->staged_live[k]) (void)hipEventSynchronize(c->staged[k]);
      (void)hipEventDestroy(c->staged[k]);
    }
    if (c->staging[k]) (void)hipHostFree(c->staging[k]);
  }
  delete c;
  return RSWA_OK;
}

}  // extern "C"

namespace {

int prefill_impl(rswa_cache *c, int32_t layer, int32_t n, const int32_t *req_ids,
                 const int32_t *prefill_len, const int64_t *slot_base, const int32_t *chunk_start,
                 const int32_t *chunk_len, const void *q, const void *k, const void *v, void *out,
                 void *stream) {
  std::string err;
  int rc = c->st.check_prefill(layer, n, req_ids, prefill_len, slot_base, &err, chunk_start, chunk_len);
  if (rc != RSWA_OK) return c->fail(rc, err);
  if (capturing((hipStream_t)stream))
    return c->fail(RSWA_E_STATE, "prefill uploads its plan and cannot be captured into a graph");
  const Config &cf = c->cfg;
  const int tile = rswa::prefill_tile_rows(cf.dtype, cf.head_dim);
  std::vector<int32_t> qoff(n, 0), rows(prefill_len, prefill_len + n);
  if (chunk_start) {
    qoff.assign(chunk_start, chunk_start + n);
    rows.assign(chunk_len, chunk_len + n);
  }
  rswa::PrefillPlan plan = c->st.plan_prefill(n, rows.data(), tile, qoff.data());
  if (plan.total_tokens > 0 && (!q || !k || !v || !out))
    return c->fail(RSWA_E_ARG, "null q/k/v/out with prefill tokens");
  if (plan.num_tiles() > cf.max_prefill_blocks())
    return c->fail(RSWA_E_CAPACITY, "too many prefill blocks");
  hipStream_t s = (hipStream_t)stream;

  rswa::PrefillBlob pb = rswa::PrefillBlob::make(n, plan.num_tiles());
  std::vector<char> blob(pb.bytes, 0);
  put(blob, pb.req, req_ids, n);
  put(blob, pb.plen, rows.data(), n);
  put(blob, pb.qoff, qoff.data(), n);
  put(blob, pb.ptot, prefill_len, n);
  put(blob, pb.cu, plan.cu.data(), n + 1);
  put(blob, pb.base, slot_base, n);
  put(blob, pb.tiles, plan.tiles.data(), plan.tiles.size());
  char *dev = c->ws + c->lay.prefill;
  hipError_t e = c->upload(dev, blob.data(), pb.bytes, s);
  if (e != hipSuccess) return c->hip_fail(e, "prefill metadata upload");

  rswa::PrefillArgs a{};
  a.pool = c->pool();
  a.pool.table = c->slot_table;
  a.st = c->state();
  a.req = (const int32_t *)(dev + pb.req);
  a.plen = (const int32_t *)(dev + pb.plen);
  a.qoff = (const int32_t *)(dev + pb.qoff);
  a.ptot = (const int32_t *)(dev + pb.ptot);
  a.cu = (const int64_t *)(dev + pb.cu);
  a.base = (const int64_t *)(dev + pb.base);
  a.tiles = (const int32_t *)(dev + pb.tiles);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.rope = c->rope();
  a.qscale = c->qscale;
  a.layer_bytes = (uint32_t)std::min<int64_t>(
      cf.num_slots * cf.num_heads * cf.head_dim * cf.elem_bytes(), UINT32_MAX);
  a.n = n;
  a.heads = cf.num_heads;
  a.layer = layer;
  a.num_tiles = (int32_t)plan.num_tiles();
  a.tile = tile;
  a.total_tokens = plan.total_tokens;
  if (layer == 0) {
    e = rswa::launch_prefill_register(a, s);
    if (e != hipSuccess) return c->hip_fail(e, "prefill register launch");
  }
  e = rswa::launch_prefill_cache_write(a, cf.dtype, cf.head_dim, s);
  if (e != hipSuccess) return c->hip_fail(e, "prefill cache write launch");
  const int pi = c->prof_begin(RSWA_KERNEL_PREFILL_ATTENTION, s);
  e = rswa::launch_prefill_attention(a, cf.dtype, cf.head_dim, s);
  c->prof_end(RSWA_KERNEL_PREFILL_ATTENTION, pi, s);
  if (e != hipSuccess) return c->hip_fail(e, "prefill attention launch");
  c->st.commit_prefill(layer, n, req_ids, prefill_len, slot_base, chunk_start, chunk_len);
  return RSWA_OK;
}

}  // namespace

extern "C" {

int rswa_prefill(rswa_cache *c, int32_t layer, int32_t n, const int32_t *req_ids,
                 const int32_t *prefill_len, const int64_t *slot_base, const void *q, const void *k,
                 const void *v, void *out, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    return prefill_impl(c, layer, n, req_ids, prefill_len, slot_base, nullptr, nullptr, q, k, v, out,
                        stream);
  });
}

int rswa_prefill_chunk(rswa_cache *c, int32_t layer, int32_t n, const int32_t *req_ids,
                       const int32_t *prefill_len, const int64_t *slot_base,
                       const int32_t *chunk_start, const int32_t *chunk_len, const void *q,
                       const void *k, const void *v, void *out, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    if (n > 0 && (!chunk_start || !chunk_len)) return c->fail(RSWA_E_ARG, "null chunk_start / chunk_len");
    return prefill_impl(c, layer, n, req_ids, prefill_len, slot_base, chunk_start, chunk_len, q, k, v,
                        out, stream);
  });
}

int rswa_admit(rswa_cache *c, int32_t req_id, int32_t prefill_len, int64_t *slot_base) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    if (!slot_base) return c->fail(RSWA_E_ARG, "null slot_base");
    std::string err;
    int64_t base = 0;
    int rc = c->st.check_admit(req_id, prefill_len, &base, &err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    c->st.commit_admit(req_id, prefill_len, base);
    *slot_base = base;
    return RSWA_OK;
  });
}

int rswa_retire(rswa_cache *c, int32_t n, const int32_t *req_ids) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    std::string err;
    int rc = c->st.check_retire(n, req_ids, &err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    c->st.commit_retire(n, req_ids);
    return RSWA_OK;
  });
}

int rswa_free_rows(const rswa_cache *c, int64_t *rows) {
  if (!c || !rows) return set_global_error(RSWA_E_ARG, "null handle or output");
  *rows = c->st.free_rows();
  return RSWA_OK;
}

int rswa_set_batch(rswa_cache *c, int32_t n, const int32_t *req_ids, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    std::string err;
    int rc = c->st.check_set_batch(n, req_ids, &err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    if (capturing((hipStream_t)stream))
      return c->fail(RSWA_E_STATE, "rswa_set_batch uploads its plan and cannot be captured into a graph");
    rswa::DecodePlan plan;
    if (n > 0) {
      plan = c->st.plan_decode(n, req_ids);
      rswa::BatchBlob bb = rswa::BatchBlob::make(n, plan.num_splits());
      std::vector<char> blob(bb.bytes, 0);
      put(blob, bb.req, req_ids, n);
      put(blob, bb.split_off, plan.split_off.data(), n + 1);
      put(blob, bb.splits, plan.splits.data(), plan.splits.size());
      hipError_t e = c->upload(c->ws + c->lay.batch, blob.data(), bb.bytes, (hipStream_t)stream);
      if (e != hipSuccess) return c->hip_fail(e, "batch upload");
    }
    c->st.commit_set_batch(n, req_ids, std::move(plan));
    return RSWA_OK;
  });
}

int rswa_ring_write(rswa_cache *c, int32_t layer, const void *k_new, const void *v_new,
                    void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    std::string err;
    int rc = c->st.check_ring_write(layer, &err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    if (!k_new || !v_new) return c->fail(RSWA_E_ARG, "null k_new / v_new");
    rswa::BatchBlob bb = rswa::BatchBlob::make((int)c->st.batch().size(), c->st.plan().num_splits());
    rswa::RingWriteArgs a{};
    a.pool = c->pool();
    a.pool.table = c->slot_table;
    a.st = c->state();
    a.batch_req = (const int32_t *)(c->ws + c->lay.batch + bb.req);
    a.k_new = k_new;
    a.v_new = v_new;
    a.rope = c->rope();
    a.n = (int32_t)c->st.batch().size();
    a.heads = c->cfg.num_heads;
    a.window = c->cfg.window;
    a.layer = layer;
    hipError_t e = rswa::launch_ring_write(a, c->cfg.dtype, c->cfg.head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return c->hip_fail(e, "ring write launch");
    c->st.commit_ring_write(layer);
    if (capturing((hipStream_t)stream)) c->st.note_capture();
    return RSWA_OK;
  });
}

}  // extern "C"

namespace {

// Split-KV partials of `tasks` (split, head) items in the fixed scratch:
// float [tasks][head_dim], then float2 [tasks] at a 256-byte boundary.
size_t noalloc_ml_offset(int64_t tasks, int head_dim) {
  return rswa::align_up((size_t)tasks * head_dim * sizeof(float));
}

int decode_impl(rswa_cache *c, int32_t layer, const void *q, const void *k_new, const void *v_new,
                void *out, void *stream, bool noalloc = false) {
  const bool fused = k_new != nullptr || v_new != nullptr;
  std::string err;
  int rc = fused ? c->st.check_fused(layer, &err) : c->st.check_decode(layer, &err);
  if (rc != RSWA_OK) return c->fail(rc, err);
  if (!q || !out) return c->fail(RSWA_E_ARG, "null q / out");
  if (fused && (!k_new || !v_new)) return c->fail(RSWA_E_ARG, "null k_new / v_new");
  const rswa::DecodePlan &plan = c->st.plan();
  const int n = (int)c->st.batch().size();
  const int64_t tasks = (int64_t)plan.num_splits() * c->cfg.num_heads;
  if (noalloc) {
    if (!c->noalloc_scratch) return c->fail(RSWA_E_HIP, c->noalloc_err);
    const size_t need = noalloc_ml_offset(tasks, c->cfg.head_dim) + (size_t)tasks * sizeof(float2);
    if (need > (size_t)RSWA_NOALLOC_SCRATCH_BYTES)
      return c->fail(RSWA_E_CAPACITY, "the batch's " + std::to_string(tasks) +
                                          " split-KV partials need " + std::to_string(need) +
                                          " bytes; the fixed scratch holds " +
                                          std::to_string((size_t)RSWA_NOALLOC_SCRATCH_BYTES));
  }
  rswa::BatchBlob bb = rswa::BatchBlob::make(n, plan.num_splits());
  const char *dev = c->ws + c->lay.batch;
  rswa::DecodeArgs a{};
  a.pool = c->pool();
  a.pool.table = c->slot_table;
  a.st = c->state();
  a.splits = (const rswa::SplitDesc *)(dev + bb.splits);
  a.split_off = (const int32_t *)(dev + bb.split_off);
  a.merge_cnt = (int32_t *)(c->ws + c->lay.merge_cnt);
  a.step_cnt = (int32_t *)(c->ws + c->lay.step_cnt);
  // The decode that completes the step's layers also advances t on the device.
  a.advance = c->st.completes_step(layer) ? 1 : 0;
  a.q = q;
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  if (noalloc) {
    a.part_o = (float *)c->noalloc_scratch;
    a.part_ml = (float2 *)((char *)c->noalloc_scratch + noalloc_ml_offset(tasks, c->cfg.head_dim));
  } else {
    a.part_o = (float *)(c->ws + c->lay.part_o);
    a.part_ml = (float2 *)(c->ws + c->lay.part_ml);
  }
  a.rope = c->rope();
  a.qscale = c->qscale;
  a.layer_bytes = (uint32_t)std::min<int64_t>(
      c->cfg.num_slots * c->cfg.num_heads * c->cfg.head_dim * c->cfg.elem_bytes(), UINT32_MAX);
  a.n = n;
  a.heads = c->cfg.num_heads;
  a.window = c->cfg.window;
  a.layer = layer;
  a.num_splits = plan.num_splits();
  a.wpb = plan.waves_per_block;
  a.attention = c->cfg.attention;
  hipStream_t s = (hipStream_t)stream;
  const int pi = noalloc ? -1 : c->prof_begin(RSWA_KERNEL_DECODE_SPLIT, s);
  hipError_t e = rswa::launch_decode(a, c->cfg.dtype, c->cfg.head_dim, s);
  c->prof_end(RSWA_KERNEL_DECODE_SPLIT, pi, s);
  if (e != hipSuccess) return c->hip_fail(e, "split-KV decode launch");
  if (fused) c->st.commit_fused(layer);
  else c->st.commit_decode(layer);
  if (capturing(s)) c->st.note_capture();
  return RSWA_OK;
}

}  // namespace

extern "C" {

int rswa_decode_step(rswa_cache *c, int32_t layer, const void *q, void *out, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int { return decode_impl(c, layer, q, nullptr, nullptr, out, stream); });
}

int rswa_decode_step_fused(rswa_cache *c, int32_t layer, const void *q, const void *k_new,
                           const void *v_new, void *out, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  if (!k_new || !v_new) return c->fail(RSWA_E_ARG, "null k_new / v_new");
  return guarded(c, [&]() -> int { return decode_impl(c, layer, q, k_new, v_new, out, stream); });
}

int rswa_decode_step_fused_noalloc(rswa_cache *c, int32_t layer, const void *q, const void *k_new,
                                   const void *v_new, void *out, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  if (!k_new || !v_new) return c->fail(RSWA_E_ARG, "null k_new / v_new");
  return guarded(c, [&]() -> int {
    return decode_impl(c, layer, q, k_new, v_new, out, stream, /*noalloc=*/true);
  });
}

int rswa_advance(rswa_cache *c, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    (void)stream;  // the step's last decode kernel already advanced t on the device
    std::string err;
    int rc = c->st.check_advance(&err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    c->st.commit_advance();
    return RSWA_OK;
  });
}

int rswa_note_steps(rswa_cache *c, int32_t steps) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    std::string err;
    int rc = c->st.check_note_steps(steps, &err);
    if (rc != RSWA_OK) return c->fail(rc, err);
    c->st.commit_note_steps(steps);
    return RSWA_OK;
  });
}

int rswa_get_state(rswa_cache *c, int32_t n, const int32_t *req_ids, int32_t *ring_pos,
                   int32_t *cache_len, int32_t *next_pos, void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  return guarded(c, [&]() -> int {
    const Config &cf = c->cfg;
    if (n < 0 || (n > 0 && !req_ids)) return c->fail(RSWA_E_ARG, "bad n / req_ids");
    if (capturing((hipStream_t)stream))
      return c->fail(RSWA_E_STATE, "rswa_get_state synchronizes and cannot be captured into a graph");
    for (int i = 0; i < n; ++i) {
      if (req_ids[i] < 0 || req_ids[i] >= cf.max_requests)
        return c->fail(RSWA_E_ARG, "request id out of range");
      if (c->st.request(req_ids[i]).plen < 0)
        return c->fail(RSWA_E_STATE, "request " + std::to_string(req_ids[i]) + " not registered");
    }
    std::vector<int32_t> dp(cf.max_requests), dt(cf.max_requests);
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess)
      e = hipMemcpy(dp.data(), c->ws + c->lay.req_p, sizeof(int32_t) * dp.size(), hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(dt.data(), c->ws + c->lay.req_t, sizeof(int32_t) * dt.size(), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return c->hip_fail(e, "reading device state");
    // Between the step's last decode and rswa_advance the device copy of t
    // of the batch's requests is already one ahead.
    const bool ahead = c->st.step_decoded();
    std::vector<uint8_t> in_batch(cf.max_requests, 0);
    for (int32_t id : c->st.batch()) in_batch[id] = 1;
    for (int i = 0; i < n; ++i) {
      const rswa::RequestState &r = c->st.request(req_ids[i]);
      const int32_t p = dp[req_ids[i]];
      const int32_t t = dt[req_ids[i]] - ((ahead && in_batch[req_ids[i]]) ? 1 : 0);
      if (p != r.plen || t != r.t)
        return c->fail(RSWA_E_STATE, "device state of request " + std::to_string(req_ids[i]) +
                                         " (P=" + std::to_string(p) + ", t=" + std::to_string(t) +
                                         ") differs from the host's (P=" + std::to_string(r.plen) +
                                         ", t=" + std::to_string(r.t) + ")");
      if (ring_pos) ring_pos[i] = HostState::ring_pos(t, cf.window);
      if (cache_len) cache_len[i] = HostState::cache_len(p, t, cf.window);
      if (next_pos) next_pos[i] = HostState::next_pos(p, t);
    }
    return RSWA_OK;
  });
}

int rswa_decode_plan(const rswa_cache *c, int32_t *split_tokens, int32_t *num_splits) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  if (split_tokens) *split_tokens = c->st.plan().split_tokens;
  if (num_splits) *num_splits = c->st.plan().num_splits();
  return RSWA_OK;
}

int rswa_profile_enable(rswa_cache *c, int enable) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  c->prof = enable != 0;
  return RSWA_OK;
}

int rswa_profile_read(rswa_cache *c, int32_t kernel, double *total_ms, int64_t *launches,
                      void *stream) {
  if (!c) return set_global_error(RSWA_E_ARG, "null handle");
  if (kernel < 0 || kernel >= RSWA_NUM_KERNELS) return c->fail(RSWA_E_ARG, "unknown kernel id");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return c->hip_fail(e, "profile read");
  double sum = 0;
  auto &v = c->prof_ev[kernel];
  for (size_t i = 0; i < c->prof_used[kernel]; ++i) {
    float ms = 0;
    e = hipEventElapsedTime(&ms, v[i].first, v[i].second);
    if (e != hipSuccess) return c->hip_fail(e, "hipEventElapsedTime");
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int64_t)c->prof_used[kernel];
  c->prof_used[kernel] = 0;
  return RSWA_OK;
}

}  // extern "C"
