// Split-KV flash-decode for R-SWA on gfx950, with the cross-split merge (and
// the step's advance) in the same launch.
//
// After the ring write of the current step, a request's cache holds
// L = P + min(t + 1, W) valid logical slots: the frozen prefill and the
// newest generated tokens (page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径
// 复盘", www.gtnt.cn/news/146005, section 2.1: attention runs over the whole
// cache after the in-place ring write).  Attention is invariant to the order
// of the slots, so decode reads logical slots 0 .. L-1 in slot order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"
#include "rswa.h"

// Tuning knobs (defaults are the measured best on MI355X): cache-policy bits
// of the key/value loads (2 = non-temporal: the cache is streamed once per
// step and re-reading it from L2 never pays), and loads per lane per chunk.
#ifndef RSWA_DECODE_LOAD_AUX
#define RSWA_DECODE_LOAD_AUX 2
#endif
#ifndef RSWA_DECODE_MIN_BLOCKS
#define RSWA_DECODE_MIN_BLOCKS 1
#endif
#ifndef RSWA_DECODE_NI
#define RSWA_DECODE_NI 8
#endif

namespace rswa {
namespace {

using namespace dev;

// Partner lane distance for the reduce-scatter stage that splits on bit b of
// the row-group lane index (see decode_split_kernel).
template <int B>
struct ScatterPartner {
  static constexpr int value = B == 4 ? 16 : B == 3 ? 15 : B == 2 ? 7 : B == 1 ? 2 : 1;
};

// Reduce-scatter of partial sums across the LPR lanes of a row group, one
// bit of the row-lane index c per stage, from bit B down to bit 0.  The first
// log2(NI) stages halve the live values: the stage on bit b keeps the half
// selected by bit b of c and adds the partner's copy of that half.  The
// remaining stages (NI < LPR) add the partner's single value.  Afterwards
// v[0] of lane c holds the full sum of index c >> (log2(LPR) - log2(NI)).
template <int NI, int B>
__device__ __forceinline__ void reduce_scatter_stage(float *v, int c) {
  constexpr int M = NI / 2;
  if constexpr (M >= 1) {
    const bool up = (c >> B) & 1;
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const float keep = up ? v[k + M] : v[k];
      const float send = up ? v[k] : v[k + M];
      v[k] = keep + lane_xor<ScatterPartner<B>::value>(send);
    }
  } else {
    v[0] += lane_xor<ScatterPartner<B>::value>(v[0]);
  }
  if constexpr (B > 0) reduce_scatter_stage<(M >= 1 ? M : 1), B - 1>(v, c);
}

template <int N> struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <> struct Log2<1> { static constexpr int value = 0; };

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Cache-policy bits of the partials' stores and loads: sc1, the agent
// coherence the compiler gives agent-scope atomic stores and loads.  Partials
// are written by waves on any XCD and read back by the wave that merges
// them, so they must not sit in one XCD's L2 only.
constexpr int kCoherent = 16;

// ---------------------------------------------------------------------------
// One wavefront per (split work item, head), four independent wavefronts per
// block.  Split ks covers keys [k0, k1) of its request (SplitDesc); a step
// attends to the part below L = P + min(t + 1, W) (with the standard window,
// from lo = P + t + 1 - W on).
//
// A head's key row is D * sizeof(T) bytes = LPR lanes x 16 bytes, so one
// 16-byte buffer load per lane covers TPI = 64 / LPR rows, and NI loads cover
// a chunk of CH = NI * TPI keys.  Lane (g, c) = (lane / LPR, lane % LPR)
// multiplies its 16-byte slice of key i * TPI + g with the matching query
// slice; the reduce-scatter then leaves lane (g, c) with the score of key
// (c >> SH) * TPI + g, SH = log2(LPR / NI) (DUP = LPR / NI lanes hold each
// score).  Softmax is online in base 2 (the query carries scale * log2 e).
// Probabilities go through LDS so each lane can weight the value slices it
// loaded with the same row mapping.
//
// The first chunk is requested before t is read (with R-SWA a split's first
// key does not depend on t); the loads of chunk i + 1 are issued while chunk
// i is computed: next keys right after this chunk's scores, next values
// right after this chunk's value accumulation.  With the page-size-1 layout
// the slot-table entries of a chunk are fetched one chunk ahead of its
// key/value loads.  Addresses are bounded by k1 (rows the request owns);
// keys of the last chunk at or past the step's end get score -inf and zeroed
// value registers, whatever rows they read.
//
// Merge: each wave stores its partial (running max m in log2 units, sum l,
// vector o; an empty split stores (-inf, 0) and zeros) with agent-coherent
// stores, waits until they complete, and adds one to its (entry, head)
// counter.  The wave that brings the counter to the entry's split count
// resets it and merges every split's partial, read back with agent-coherent
// loads: M = max m_s, out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s.  No
// wave waits on another.  When the launch ends the step, the wave that merges
// an entry's last head also sets t = t + 1 for it: by then every wave of
// that entry has read t.
// ---------------------------------------------------------------------------
template <typename T, int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(64 * kDecodeMaxWavesPerBlock, RSWA_DECODE_MIN_BLOCKS) void decode_split_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per key row
  constexpr int TPI = 64 / LPR;         // key rows per load instruction
  constexpr int NI = LPR < RSWA_DECODE_NI ? LPR : RSWA_DECODE_NI;  // loads per chunk
  constexpr int CH = NI * TPI;          // keys per chunk
  constexpr int DUP = LPR / NI;         // lanes holding each score
  constexpr int SH = Log2<DUP>::value;
  static_assert(CH <= 64, "chunk keys must fit one table load");
  __shared__ float lds_p[kDecodeMaxWavesPerBlock][64];
  __shared__ int32_t lds_row[kDecodeMaxWavesPerBlock][64];
  __shared__ uint4 lds_new[FUSED ? kDecodeMaxWavesPerBlock : 1][2][LPR];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int task = blockIdx.x * (int)(blockDim.x >> 6) + wid;  // blocks of 1 .. 12 waves
  if (task >= a.num_splits * a.heads) return;
  const int ks = task / a.heads;
  const int h = task % a.heads;
  const SplitDesc sd = a.splits[ks];
  const int b = sd.b;
  const int r = sd.r;
  const int p_len = sd.p;
  const int64_t base = sd.base;
  const int k1 = sd.k1;  // address bound: the request owns rows below P + W >= k1
  const bool swa = a.attention == RSWA_ATTENTION_SWA;
  const int g = lane / LPR;
  const int c = lane % LPR;

  const uint32_t row_bytes = (uint32_t)(a.heads * D * sizeof(T));
  const uint32_t lane_off = (uint32_t)((h * D + c * EPL) * sizeof(T));
  const size_t layer_off = (size_t)a.layer * a.pool.layer_stride * sizeof(T);
  __amdgpu_buffer_rsrc_t rk, rv, rt;
  if constexpr (PAGED) {
    rk = make_rsrc((const char *)a.pool.k + layer_off, a.layer_bytes);
    rv = make_rsrc((const char *)a.pool.v + layer_off, a.layer_bytes);
    rt = make_rsrc(a.pool.table + base, (uint32_t)k1 * 4u);
  } else {
    const size_t req_off = layer_off + (size_t)base * row_bytes;
    rk = make_rsrc((const char *)a.pool.k + req_off, (uint32_t)k1 * row_bytes);
    rv = make_rsrc((const char *)a.pool.v + req_off, (uint32_t)k1 * row_bytes);
  }
  // Table entry of chunk key `lane` (clamped to the split's last row).
  auto table_entry = [&](int c0) -> uint32_t {
    return buf_load4(rt, (uint32_t)min(c0 + min(lane, CH - 1), k1 - 1) * 4u);
  };
  // Stores a chunk's table entries so that lane (g, c) later finds the row of
  // key i * TPI + g at [g * NI + i].
  auto stash_rows = [&](uint32_t tab) {
    if (lane < CH) lds_row[wid][(lane % TPI) * NI + lane / TPI] = (int32_t)tab;
    __builtin_amdgcn_wave_barrier();
  };
  // Byte offset of key c0 + i * TPI + g for this lane.
  auto row_offset = [&](int c0, int i) -> uint32_t {
    if constexpr (PAGED)
      return (uint32_t)lds_row[wid][g * NI + i] * row_bytes + lane_off;
    else
      return (uint32_t)(c0 + i * TPI + g) * row_bytes + lane_off;
  };

  uint4 kr[NI], vr[NI];
  uint32_t tab_next = 0;
  auto issue_first = [&](int c0) {
    if constexpr (PAGED) stash_rows(table_entry(c0));
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rk, row_offset(c0, i));
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rv, row_offset(c0, i));
    if (PAGED && c0 + CH < k1) tab_next = table_entry(c0 + CH);
  };
  if (!swa) issue_first(sd.k0);

  const int t = a.st.t[r];
  const int L = p_len + min(t + 1, a.window);
  // Keys lo .. L-1 are visible: all of them for R-SWA; with the standard
  // window only logical positions P + t + 1 - W .. P + t.
  const int lo = swa ? min(p_len, max(0, p_len + t + 1 - a.window)) : 0;
  const int start = max(sd.k0, lo);
  const int end = min(k1, L);
  const bool nonempty = start < end;
  if (swa && nonempty) issue_first(start);

  float m_run = -INFINITY;
  float l_tot = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  if (nonempty) {
    // Query rotated at position P + t, pre-scaled by scale * log2(e).
    const int pos = p_len + t;
    const T *qp = (const T *)a.q + ((int64_t)b * a.heads + h) * D;
    const float2 *cs = a.rope + (int64_t)pos * (D / 2);
    float qh[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = c * EPL + e;
      const float x = to_f(qp[d]);
      const float y = d < D / 2 ? -to_f(qp[d + D / 2]) : to_f(qp[d - D / 2]);
      const float2 cc = cs[d % (D / 2)];
      qh[e] = (x * cc.x + y * cc.y) * a.qscale;
    }

    // Fused ring write: the wave whose split holds this step's ring slot
    // rotates k_new at position P + t, stores the new key/value row for its
    // head, and uses the new row in place of the stale one it loaded.
    const int slot_new = p_len + t % a.window;
    const bool writes = FUSED && slot_new >= start && slot_new < end;
    // This lane's 16-byte slices of the new rotated key row and value row.
    auto new_row = [&](uint4 &kn_pk, uint4 &vn_pk) {
      const T *kp = (const T *)a.k_new + ((int64_t)b * a.heads + h) * D;
      const T *vp = (const T *)a.v_new + ((int64_t)b * a.heads + h) * D;
      T kn[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = c * EPL + e;
        const float2 cc = cs[d % (D / 2)];
        if (d < D / 2) {
          const float x1 = to_f(kp[d]), x2 = to_f(kp[d + D / 2]);
          kn[e] = from_f<T>(rope_lo(x1, x2, cc));
        } else {
          const float x2 = to_f(kp[d]), x1 = to_f(kp[d - D / 2]);
          kn[e] = from_f<T>(rope_hi(x1, x2, cc));
        }
      }
      kn_pk = __builtin_bit_cast(uint4, kn);
      vn_pk = *(const uint4 *)(vp + c * EPL);
    };
    // The new row goes to the pool and, for this wave's later use, to LDS.
    if (writes) {
      if (g == 0) {
        uint4 kn_pk, vn_pk;
        new_row(kn_pk, vn_pk);
        lds_new[wid][0][c] = kn_pk;
        lds_new[wid][1][c] = vn_pk;
        const int64_t row = PAGED ? (int64_t)a.pool.table[base + slot_new] : base + slot_new;
        const size_t off = layer_off + (size_t)row * row_bytes + lane_off;
        *(uint4 *)((char *)a.pool.k + off) = kn_pk;
        *(uint4 *)((char *)a.pool.v + off) = vn_pk;
      }
      __builtin_amdgcn_wave_barrier();
    }
    // Replaces the stale loaded copy of the new slot (key c0 + i * TPI + g)
    // in the chunk that holds it.
    auto patch = [&](uint4 *regs, int c0, int which) {
      if (writes && slot_new >= c0 && slot_new < c0 + CH) {
        const int rel = slot_new - c0;
        if (g == rel % TPI) {
          const uint4 fresh = lds_new[wid][which][c];
#pragma unroll
          for (int i = 0; i < NI; ++i)
            if (i == rel / TPI) regs[i] = fresh;
        }
      }
    };

    float l_run = 0.f;
    int c0 = start;
    for (;;) {
      const bool more = c0 + CH < end;
      patch(kr, c0, 0);
      float sc[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float kf[EPL];
        Vec16<T>::unpack(kr[i], kf);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qh[e], kf[e], acc);
        sc[i] = acc;
      }
      reduce_scatter_stage<NI, Log2<LPR>::value - 1>(sc, c);
      float score = sc[0];  // key c0 + (c >> SH) * TPI + g
      if (c0 + (c >> SH) * TPI + g >= end) score = -INFINITY;
      const float m_new = fmaxf(m_run, wave_max(score));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float p = __builtin_amdgcn_exp2f(score - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= alpha;
      m_run = m_new;
      lds_p[wid][lane] = p;
      if (more) {
        if constexpr (PAGED) stash_rows(tab_next);
#pragma unroll
        for (int i = 0; i < NI; ++i) kr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rk, row_offset(c0 + CH, i));
        if (PAGED && c0 + 2 * CH < end) tab_next = table_entry(c0 + 2 * CH);
      }
      __builtin_amdgcn_wave_barrier();
      patch(vr, c0, 1);
      // Keys at or past the end (the tail of the last chunk) have weight 0;
      // zeroed values keep 0 * v finite whatever row they read.
      if (!more) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (c0 + i * TPI + g >= end) vr[i] = make_uint4(0, 0, 0, 0);
      }
      // Key i * TPI + g is scored by lanes g * LPR + (i << SH) ...
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pi = lds_p[wid][g * LPR + (i << SH)];
        float vf[EPL];
        Vec16<T>::unpack(vr[i], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = fmaf(pi, vf[e], o[e]);
      }
      __builtin_amdgcn_wave_barrier();
      if (!more) break;
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rv, row_offset(c0 + CH, i));
      c0 += CH;
    }
    // Each score was accumulated by DUP lanes.
    l_tot = wave_sum(l_run) * (1.0f / DUP);
#pragma unroll
    for (int msk = LPR; msk < 64; msk <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], msk);
    }
  }

  // ---- this (split, head)'s partial, then the merge by the last one -------
  if (g == 0) {
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part_o + (int64_t)task * D, D * 4);
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 v = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp,
                                             (uint32_t)((c * EPL + e) * 4), 0, kCoherent);
    }
  }
  if (lane == 0) {
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.part_ml + task, 8);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(m_run, l_tot)), rm, 0,
                                          0, kCoherent);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0);  // the partial has reached the coherence point
  int done = 0;
  if (lane == 0)
    done = __hip_atomic_fetch_add(a.merge_cnt + b * a.heads + h, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  done = __builtin_amdgcn_readfirstlane(done);
  const int first = a.split_off[b];
  const int count = a.split_off[b + 1] - first;
  if (done != count - 1) return;

  // Last split of (entry b, head h): merge all count partials.  Lane
  // (q, j) = (lane / CPS, lane % CPS) reads 16-byte chunk j of split slot q
  // (SPS split slots per load instruction), MB loads in flight per batch, and
  // weights it by 2^(m - M) fetched from the lane that read that split's
  // (m, l); the SPS slot sums then meet across lanes.
  if (lane == 0)
    __hip_atomic_store(a.merge_cnt + b * a.heads + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int CPS = D / 4;       // 16-byte chunks per split vector
  constexpr int SPS = 64 / CPS;    // splits per load instruction
  constexpr int MB = 16;           // loads in flight per lane
  constexpr int BATCH = SPS * MB;  // splits per batch
  const int q = lane / CPS;
  const int j = lane % CPS;
  const __amdgpu_buffer_rsrc_t rml =
      make_rsrc(a.part_ml + (int64_t)first * a.heads + h, (uint32_t)count * (uint32_t)a.heads * 8u);
  auto load_ml = [&](int k) -> float2 {
    if (k >= count) return make_float2(-INFINITY, 0.f);
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                                          rml, (uint32_t)k * (uint32_t)a.heads * 8u, 0, kCoherent));
  };
  // Chunk j of split k's vector.
  auto load_o = [&](int k) -> float4 {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.part_o + ((int64_t)(first + k) * a.heads + h) * D, D * 4);
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)j * 16u, 0, kCoherent));
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  // Batch of splits k0 .. k0 + BATCH - 1 (clamped; extra slots get weight 0)
  // whose weights wk sit in lanes k - kw of the current (m, l) window.
  auto batch = [&](int k0, int kw, float wk, const float4 *ov) {
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int k = k0 + u * SPS + q;
      const float w = __shfl(wk, min(k, count - 1) - kw);
      const float wu = k < count ? w : 0.f;
      acc.x = fmaf(wu, ov[u].x, acc.x);
      acc.y = fmaf(wu, ov[u].y, acc.y);
      acc.z = fmaf(wu, ov[u].z, acc.z);
      acc.w = fmaf(wu, ov[u].w, acc.w);
    }
  };
  auto issue = [&](int k0, float4 *ov) {
#pragma unroll
    for (int u = 0; u < MB; ++u) ov[u] = load_o(min(k0 + u * SPS + q, count - 1));
  };
  if (count <= 64 && count <= BATCH) {
    // One batch: the (m, l) pairs and the vectors are requested together.
    float4 ov[MB];
    const float2 v = load_ml(lane);
    issue(0, ov);
    const float mx = wave_max(v.y > 0.f ? v.x : -INFINITY);
    const float wk = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
    den = wk * v.y;
    batch(0, 0, wk, ov);
  } else {
    float mx = -INFINITY;
    for (int k0 = 0; k0 < count; k0 += 64) {
      const float2 v = load_ml(k0 + lane);
      if (v.y > 0.f) mx = fmaxf(mx, v.x);
    }
    mx = wave_max(mx);
    for (int kw = 0; kw < count; kw += 64) {
      const float2 v = load_ml(kw + lane);
      const float wk = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
      den = fmaf(wk, v.y, den);
      const int kend = min(count, kw + 64);
      for (int k0 = kw; k0 < kend; k0 += BATCH) {
        float4 ov[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) ov[u] = load_o(min(k0 + u * SPS + q, kend - 1));
#pragma unroll
        for (int u = 0; u < MB; ++u) {
          const int k = k0 + u * SPS + q;
          const float w = __shfl(wk, min(k, kend - 1) - kw);
          const float wu = k < kend ? w : 0.f;
          acc.x = fmaf(wu, ov[u].x, acc.x);
          acc.y = fmaf(wu, ov[u].y, acc.y);
          acc.z = fmaf(wu, ov[u].z, acc.z);
          acc.w = fmaf(wu, ov[u].w, acc.w);
        }
      }
    }
  }
#pragma unroll
  for (int msk = CPS; msk < 64; msk <<= 1) {
    acc.x += __shfl_xor(acc.x, msk);
    acc.y += __shfl_xor(acc.y, msk);
    acc.z += __shfl_xor(acc.z, msk);
    acc.w += __shfl_xor(acc.w, msk);
  }
  const float inv = 1.f / wave_sum(den);
  if (q == 0) {
    struct alignas(4 * sizeof(T)) Out4 { T v[4]; };
    const Out4 res = {{from_f<T>(acc.x * inv), from_f<T>(acc.y * inv), from_f<T>(acc.z * inv),
                       from_f<T>(acc.w * inv)}};
    *(Out4 *)((T *)a.out + ((int64_t)b * a.heads + h) * D + 4 * j) = res;
  }

  // End of the step: the entry's last merged head advances its t.
  if (a.advance) {
    int heads_done = 0;
    if (lane == 0)
      heads_done = __hip_atomic_fetch_add(a.step_cnt + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    heads_done = __builtin_amdgcn_readfirstlane(heads_done);
    if (heads_done == a.heads - 1 && lane == 0) {
      __hip_atomic_store(a.step_cnt + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.st.t[r] = t + 1;
    }
  }
}

template <typename F>
hipError_t dispatch(int dtype, int head_dim, F &&f) {
  if (dtype == RSWA_DTYPE_BF16 && head_dim == 128) return f(bf16{}, std::integral_constant<int, 128>{});
  if (dtype == RSWA_DTYPE_BF16 && head_dim == 64) return f(bf16{}, std::integral_constant<int, 64>{});
  if (dtype == RSWA_DTYPE_F32 && head_dim == 128) return f(float{}, std::integral_constant<int, 128>{});
  if (dtype == RSWA_DTYPE_F32 && head_dim == 64) return f(float{}, std::integral_constant<int, 64>{});
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    const int64_t tasks = (int64_t)a.num_splits * a.heads;
    if (a.wpb < 1 || a.wpb > kDecodeMaxWavesPerBlock) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((tasks + a.wpb - 1) / a.wpb));
    const bool fused = a.k_new != nullptr;
    if (a.pool.table && fused)
      hipLaunchKernelGGL((decode_split_kernel<T, D, true, true>), grid, dim3(64 * a.wpb), 0, s, a);
    else if (a.pool.table)
      hipLaunchKernelGGL((decode_split_kernel<T, D, true, false>), grid, dim3(64 * a.wpb), 0, s, a);
    else if (fused)
      hipLaunchKernelGGL((decode_split_kernel<T, D, false, true>), grid, dim3(64 * a.wpb), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, D, false, false>), grid, dim3(64 * a.wpb), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t decode_resident_waves(int dtype, int head_dim, int64_t *waves) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    const void *k[4] = {(const void *)decode_split_kernel<T, D, true, true>,
                        (const void *)decode_split_kernel<T, D, true, false>,
                        (const void *)decode_split_kernel<T, D, false, true>,
                        (const void *)decode_split_kernel<T, D, false, false>};
    int fewest = 1 << 30;
    for (const void *f : k) {
      int blocks = 0;
      const hipError_t r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, 64, 0);
      if (r != hipSuccess) return r;
      fewest = std::min(fewest, blocks);
    }
    *waves = (int64_t)fewest * cus;  // single-wave blocks: waves per CU
    return hipSuccess;
  });
}

}  // namespace rswa
