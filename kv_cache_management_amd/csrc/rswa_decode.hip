// Split-KV flash-decode for R-SWA on gfx950, and the cross-split combine.
//
// After the ring write of the current step, a request's cache holds
// L = P + min(t + 1, W) valid logical slots: the frozen prefill and the
// newest generated tokens (page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径
// 复盘", www.gtnt.cn/news/146005, section 2.1: attention runs over the whole
// cache after the in-place ring write).  Attention is invariant to the order
// of the slots, so decode reads logical slots 0 .. L-1 in slot order.
#include <hip/hip_runtime.h>

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

// ---------------------------------------------------------------------------
// One wavefront per (split work item, head), four independent wavefronts per
// block.  A split covers keys [s * split_tokens, min((s+1) * split_tokens, L)).
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
// The loads of chunk i + 1 are issued while chunk i is computed: next keys
// right after this chunk's scores, next values right after this chunk's
// value accumulation.  With the page-size-1 layout the slot-table entries of
// a chunk are fetched one chunk ahead of its key/value loads.
//
// Contiguous layout: the buffer resource starts at the request's first row
// and ends at the split's last key, so the ragged tail of the last chunk
// reads zeros without touching memory.  Paged layout: the resource spans the
// layer; tail keys reuse the last valid key's row, get probability 0 and
// have their value registers zeroed.
// ---------------------------------------------------------------------------
template <typename T, int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(256, RSWA_DECODE_MIN_BLOCKS) void decode_split_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per key row
  constexpr int TPI = 64 / LPR;         // key rows per load instruction
  constexpr int NI = LPR < RSWA_DECODE_NI ? LPR : RSWA_DECODE_NI;  // loads per chunk
  constexpr int CH = NI * TPI;          // keys per chunk
  constexpr int DUP = LPR / NI;         // lanes holding each score
  constexpr int SH = Log2<DUP>::value;
  static_assert(CH <= 64, "chunk keys must fit one table load");
  __shared__ float lds_p[4][64];
  __shared__ int32_t lds_row[4][64];
  __shared__ uint4 lds_new[FUSED ? 4 : 1][2][LPR];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int task = blockIdx.x * 4 + wid;
  if (task >= a.num_splits * a.heads) return;
  const int ks = task / a.heads;
  const int h = task % a.heads;
  const int b = a.split_map[2 * ks];
  const int s = a.split_map[2 * ks + 1];
  const int r = a.batch_req[b];
  const int p_len = a.st.plen[r];
  const int t = a.st.t[r];
  const int64_t base = a.st.base[r];
  const int L = p_len + min(t + 1, a.window);
  // Keys lo .. L-1 are visible: all of them for R-SWA; with the standard
  // window only logical positions P + t + 1 - W .. P + t.  Splits tile the
  // range from key0, the lowest lo any step of this request can have.
  const bool swa = a.attention == RSWA_ATTENTION_SWA;
  const int key0 = swa ? max(0, p_len - a.window + 1) : 0;
  const int lo = swa ? min(p_len, max(0, p_len + t + 1 - a.window)) : 0;
  const int split0 = key0 + s * a.split_tokens;
  const int start = max(split0, lo);
  const int end = min(split0 + a.split_tokens, L);
  float2 *ml = a.part_ml + (int64_t)ks * a.heads + h;
  if (start >= end) {
    if (lane == 0) *ml = make_float2(-INFINITY, 0.f);
    return;
  }
  const int g = lane / LPR;
  const int c = lane % LPR;

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

  const uint32_t row_bytes = (uint32_t)(a.heads * D * sizeof(T));
  const uint32_t lane_off = (uint32_t)((h * D + c * EPL) * sizeof(T));
  const size_t layer_off = (size_t)a.layer * a.pool.layer_stride * sizeof(T);
  __amdgpu_buffer_rsrc_t rk, rv, rt;
  if constexpr (PAGED) {
    rk = make_rsrc((const char *)a.pool.k + layer_off, a.layer_bytes);
    rv = make_rsrc((const char *)a.pool.v + layer_off, a.layer_bytes);
    rt = make_rsrc(a.pool.table + base, (uint32_t)end * 4u);
  } else {
    const size_t req_off = layer_off + (size_t)base * row_bytes;
    rk = make_rsrc((const char *)a.pool.k + req_off, (uint32_t)end * row_bytes);
    rv = make_rsrc((const char *)a.pool.v + req_off, (uint32_t)end * row_bytes);
  }
  // Table entry of chunk key `lane` (clamped to the split's last key).
  auto table_entry = [&](int c0) -> uint32_t {
    return buf_load4(rt, (uint32_t)min(c0 + min(lane, CH - 1), end - 1) * 4u);
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

  // Fused ring write: the wave whose split holds this step's ring slot
  // rotates k_new at position P + t, stores the new key/value row for its
  // head, and uses the new row in place of the stale one it loads.
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
  // Replaces the stale loaded copy of the new slot (key c0 + i * TPI + g) in
  // the chunk that holds it.
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

  float m_run = -INFINITY;
  float l_run = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  int c0 = start;
  uint4 kr[NI], vr[NI];
  uint32_t tab_next = 0;
  if constexpr (PAGED) stash_rows(table_entry(c0));
#pragma unroll
  for (int i = 0; i < NI; ++i) kr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rk, row_offset(c0, i));
#pragma unroll
  for (int i = 0; i < NI; ++i) vr[i] = buf_load16<RSWA_DECODE_LOAD_AUX>(rv, row_offset(c0, i));
  if (PAGED && c0 + CH < end) tab_next = table_entry(c0 + CH);

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
    // Paged tail: keys past the split's end loaded the row of its last key
    // (possibly the row this wave has just written); their weight is 0, and
    // zeroed values keep 0 * v finite whatever that row held.
    if constexpr (PAGED) {
      if (!more) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          if (c0 + i * TPI + g >= end) vr[i] = make_uint4(0, 0, 0, 0);
      }
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
  const float l_tot = wave_sum(l_run) * (1.0f / DUP);
#pragma unroll
  for (int msk = LPR; msk < 64; msk <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], msk);
  }
  if (g == 0) {
    float *po = a.part_o + ((int64_t)ks * a.heads + h) * D + c * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) *(float4 *)(po + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
  }
  if (lane == 0) *ml = make_float2(m_run, l_tot);
}

// Cross-split combine: one block of four wavefronts per (batch entry, head).
// M = max_s m_s; out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Wave w accumulates splits w, w + 4, ... (lanes over the head dimension,
// four splits' loads in flight); the four partial sums meet in LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int J = D / 64;
  constexpr int U = 4;
  __shared__ float red_max[4];
  __shared__ float red_acc[4][D];
  __shared__ float red_den[4];
  const int b = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int k0 = a.split_off[b];
  const int k1 = a.split_off[b + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  float mx = -INFINITY;
  for (int k = k0 + tid; k < k1; k += 256) mx = fmaxf(mx, a.part_ml[(int64_t)k * a.heads + h].x);
  mx = wave_max(mx);
  if (lane == 0) red_max[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
  float den = 0.f;
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.f;
  for (int kb = k0 + w; kb < k1; kb += 4 * U) {
    float2 m_l[U];
    float pv[U][J];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + 4 * u;
      if (k < k1) {
        m_l[u] = a.part_ml[(int64_t)k * a.heads + h];
        const float *po = a.part_o + ((int64_t)k * a.heads + h) * D + lane;
#pragma unroll
        for (int j = 0; j < J; ++j) pv[u][j] = po[64 * j];
      } else {
        m_l[u] = make_float2(-INFINITY, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // splits past the cache end carry (-inf, 0) and get weight 0
      if (m_l[u].y > 0.f) {
        const float wgt = __builtin_amdgcn_exp2f(m_l[u].x - mx);
        den = fmaf(wgt, m_l[u].y, den);
#pragma unroll
        for (int j = 0; j < J; ++j) acc[j] = fmaf(wgt, pv[u][j], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) red_acc[w][lane + 64 * j] = acc[j];
  if (lane == 0) red_den[w] = den;
  __syncthreads();
  if (w != 0) return;
  const float inv = 1.f / (red_den[0] + red_den[1] + red_den[2] + red_den[3]);
  T *out = (T *)a.out + ((int64_t)b * a.heads + h) * D;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int d = lane + 64 * j;
    out[d] = from_f<T>((red_acc[0][d] + red_acc[1][d] + red_acc[2][d] + red_acc[3][d]) * inv);
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

hipError_t launch_decode_split(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    const int64_t tasks = (int64_t)a.num_splits * a.heads;
    const dim3 grid((unsigned)((tasks + 3) / 4));
    const bool fused = a.k_new != nullptr;
    if (a.pool.table && fused)
      hipLaunchKernelGGL((decode_split_kernel<T, D, true, true>), grid, dim3(256), 0, s, a);
    else if (a.pool.table)
      hipLaunchKernelGGL((decode_split_kernel<T, D, true, false>), grid, dim3(256), 0, s, a);
    else if (fused)
      hipLaunchKernelGGL((decode_split_kernel<T, D, false, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, D, false, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_decode_combine(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.n * a.heads), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace rswa
