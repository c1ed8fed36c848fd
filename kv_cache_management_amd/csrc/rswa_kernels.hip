// gfx950 kernels of the R-SWA hot path, except the MFMA prefill attention:
// ring write (RoPE at the absolute position, in-place slot overwrite),
// split-KV flash-decode over the frozen prefill plus the ring, the
// cross-split combine, the step advance, and prefill registration / cache
// write / a VALU causal attention used for fp32 and as a reference path.
//
// The cache policy is that of page "开源5天Star破万之后：百度Unlimited-OCR的爆火
// 路径复盘" (www.gtnt.cn/news/146005), section 2.1: prefill rows are kept
// whole, the ring slot after the prefill is overwritten in place at
// prefill_len + ring_pos, and attention runs over the whole cache.  RoPE is
// not on the pages: rotate-half over the head dimension at the absolute
// position, with cos/sin read from a table the host computes in fp64.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.hpp"
#include "rswa.h"

namespace rswa {
namespace {

using bf16 = __bf16;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// A 16-byte vector of T unpacked to fp32.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ int64_t pool_row(const int32_t *table, int64_t base, int64_t i) {
  return table ? (int64_t)table[base + i] : base + i;
}

// ---------------------------------------------------------------------------
// Ring write: one block of 64 threads per (batch entry, head).
// slot = P + (t mod W), position = P + t; K row = RoPE(k_new, P + t), V row =
// v_new.  Thread i handles the rotation pair (i, i + D/2).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void ring_write_kernel(RingWriteArgs a) {
  const int b = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int r = a.batch_req[b];
  const int p_len = a.st.plen[r];
  const int t = a.st.t[r];
  const int pos = p_len + t;
  const int slot = p_len + t % a.window;
  const int64_t row = pool_row(a.pool.table, a.st.base[r], slot);
  const int64_t dst = (int64_t)a.layer * a.pool.layer_stride + (row * a.heads + h) * D;
  const int64_t src = ((int64_t)b * a.heads + h) * D;
  const T *kn = (const T *)a.k_new + src;
  const T *vn = (const T *)a.v_new + src;
  T *K = (T *)a.pool.k + dst;
  T *V = (T *)a.pool.v + dst;
  const float2 *cs = a.rope + (int64_t)pos * (D / 2);
  for (int i = threadIdx.x; i < D / 2; i += 64) {
    const float2 c = cs[i];
    const float x1 = to_f(kn[i]);
    const float x2 = to_f(kn[i + D / 2]);
    K[i] = from_f<T>(x1 * c.x - x2 * c.y);
    K[i + D / 2] = from_f<T>(x2 * c.x + x1 * c.y);
    V[i] = vn[i];
    V[i + D / 2] = vn[i + D / 2];
  }
}

// Advance: every active request has one more generated token cached.
__global__ __launch_bounds__(256) void advance_kernel(AdvanceArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b < a.n) a.st.t[a.batch_req[b]] += 1;
}

// ---------------------------------------------------------------------------
// Split-KV decode.  One wavefront per (split work item, head); four
// independent wavefronts per block.  A split covers keys
// [s * split_tokens, min((s+1) * split_tokens, L)) of logical slots
// 0 .. L-1, L = P + min(t + 1, W).
//
// Keys are streamed 64 at a time.  A head's key row is D * sizeof(T) bytes =
// LPR lanes x 16 bytes, so one 16-byte load per lane covers TPI = 64 / LPR
// rows and NI = LPR loads cover the 64-key chunk.  Lane (g, c) = (lane / LPR,
// lane % LPR) multiplies its 16-byte slice of row i * TPI + g with the
// matching query slice; a reduce-scatter over the LPR lanes of a row group
// then leaves lane (g, c) with the full score of key c * TPI + g.  Softmax
// runs online in base 2 (the query carries scale * log2 e).  The
// probabilities go through LDS so each lane can weight the value slices it
// loaded with the same row mapping.  Per split the wave writes its running
// max, sum and unnormalised output vector.
// ---------------------------------------------------------------------------
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int EPL = Vec16<T>::N;  // elements per 16-byte load
  constexpr int LPR = D / EPL;      // lanes per key row
  constexpr int TPI = 64 / LPR;     // key rows per load instruction
  constexpr int NI = LPR;           // load instructions per 64-key chunk
  static_assert(TPI * NI == 64, "chunk must be 64 keys");
  __shared__ float lds_p[4][64];
  __shared__ int32_t lds_row[4][64];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
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
  const int start = s * a.split_tokens;
  float2 *ml = a.part_ml + (int64_t)ks * a.heads + h;
  if (start >= L) {
    if (lane == 0) *ml = make_float2(-INFINITY, 0.f);
    return;
  }
  const int end = min(start + a.split_tokens, L);
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

  const int64_t row_stride = (int64_t)a.heads * D;
  const T *Kl = (const T *)a.pool.k + (int64_t)a.layer * a.pool.layer_stride + h * D + c * EPL;
  const T *Vl = (const T *)a.pool.v + (int64_t)a.layer * a.pool.layer_stride + h * D + c * EPL;

  float m_run = -INFINITY;
  float l_run = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;

  for (int c0 = start; c0 < end; c0 += 64) {
    int64_t rows[NI];
    if (PAGED) {
      // Row of chunk key `lane`, stored so that lane (g, c) finds the rows of
      // keys i * TPI + g (i = 0 .. NI-1) contiguously at [g * NI + i].
      const int jj = min(c0 + lane, end - 1);
      lds_row[wid][(lane % TPI) * NI + lane / TPI] = a.pool.table[base + jj];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < NI; ++i) rows[i] = lds_row[wid][g * NI + i];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) rows[i] = base + min(c0 + i * TPI + g, end - 1);
    }
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = *(const uint4 *)(Kl + rows[i] * row_stride);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = *(const uint4 *)(Vl + rows[i] * row_stride);

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
    // Reduce-scatter across the LPR lanes of the row group: after the stage
    // with mask m each lane keeps the half of the live values selected by
    // bit m of c and adds its partner's copy of that half.
#pragma unroll
    for (int m = NI / 2; m >= 1; m >>= 1) {
      const bool up = (c & m) != 0;
#pragma unroll
      for (int k = 0; k < m; ++k) {
        const float keep = up ? sc[k + m] : sc[k];
        const float send = up ? sc[k] : sc[k + m];
        sc[k] = keep + __shfl_xor(send, m);
      }
    }
    float score = sc[0];  // key c0 + c * TPI + g
    if (c0 + c * TPI + g >= end) score = -INFINITY;
    const float m_new = fmaxf(m_run, wave_max(score));
    const float alpha = exp2f(m_run - m_new);
    const float p = exp2f(score - m_new);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= alpha;
    m_run = m_new;

    // Key i * TPI + g is owned by lane g * LPR + i.
    lds_p[wid][lane] = p;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pi = lds_p[wid][g * LPR + i];
      float vf[EPL];
      Vec16<T>::unpack(vr[i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pi, vf[e], o[e]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  const float l_tot = wave_sum(l_run);
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

// Cross-split combine: one wavefront per (batch entry, head).
// M = max_s m_s; out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  const int b = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int k0 = a.split_off[b];
  const int k1 = a.split_off[b + 1];
  const int lane = threadIdx.x;
  float mx = -INFINITY;
  for (int k = k0; k < k1; ++k) mx = fmaxf(mx, a.part_ml[(int64_t)k * a.heads + h].x);
  float den = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) acc[j] = 0.f;
  for (int k = k0; k < k1; ++k) {
    const float2 m_l = a.part_ml[(int64_t)k * a.heads + h];
    if (m_l.y == 0.f) continue;  // split past the cache end: no keys
    const float w = exp2f(m_l.x - mx);
    den += w * m_l.y;
    const float *po = a.part_o + ((int64_t)k * a.heads + h) * D;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) acc[j] = fmaf(w, po[lane + 64 * j], acc[j]);
  }
  T *out = (T *)a.out + ((int64_t)b * a.heads + h) * D;
  const float inv = 1.f / den;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) out[lane + 64 * j] = from_f<T>(acc[j] * inv);
}

// ---------------------------------------------------------------------------
// Prefill: registration (layer 0) and the cache write K = RoPE(k, j), V = v.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_register_kernel(PrefillArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.n) return;
  const int r = a.req[b];
  a.st.plen[r] = a.plen[b];
  a.st.t[r] = 0;
  a.st.base[r] = a.base[b];
}

// Batch entry holding packed token `tok`: the largest b with cu[b] <= tok.
__device__ __forceinline__ int find_request(const int64_t *cu, int n, int64_t tok) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One block per packed prefill token; threads cover (head, rotation pair).
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_cache_write_kernel(PrefillArgs a) {
  const int64_t tok = blockIdx.x;
  const int b = find_request(a.cu, a.n, tok);
  const int j = (int)(tok - a.cu[b]);
  const int64_t row = pool_row(a.pool.table, a.base[b], j);
  const int64_t dst0 = (int64_t)a.layer * a.pool.layer_stride + row * a.heads * D;
  const int64_t src0 = tok * a.heads * D;
  const float2 *cs = a.rope + (int64_t)j * (D / 2);
  for (int idx = threadIdx.x; idx < a.heads * (D / 2); idx += 256) {
    const int h = idx / (D / 2);
    const int i = idx % (D / 2);
    const int64_t src = src0 + h * D;
    const int64_t dst = dst0 + h * D;
    const T *k = (const T *)a.k + src;
    const T *v = (const T *)a.v + src;
    T *K = (T *)a.pool.k + dst;
    T *V = (T *)a.pool.v + dst;
    const float2 c = cs[i];
    const float x1 = to_f(k[i]);
    const float x2 = to_f(k[i + D / 2]);
    K[i] = from_f<T>(x1 * c.x - x2 * c.y);
    K[i + D / 2] = from_f<T>(x2 * c.x + x1 * c.y);
    V[i] = v[i];
    V[i + D / 2] = v[i + D / 2];
  }
}

// ---------------------------------------------------------------------------
// Causal prefill attention on the VALU (fp32 path and cross-check path).
// One block of 64 threads per (query tile of 64 rows, head); thread = query
// row.  Keys (already rotated, read from the pool) and values are staged 32
// at a time in LDS; softmax is online in base 2.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void prefill_attn_valu_kernel(PrefillArgs a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int item = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int b = a.tiles[2 * item];
  const int qt = a.tiles[2 * item + 1];
  const int p_len = a.plen[b];
  const int64_t base = a.base[b];
  const int64_t cu = a.cu[b];
  const int i = qt * 64 + threadIdx.x;
  const bool active = i < p_len;
  const int64_t layer0 = (int64_t)a.layer * a.pool.layer_stride;

  float qh[D];
  float o[D];
  if (active) {
    const T *qp = (const T *)a.q + ((cu + i) * a.heads + h) * D;
    const float2 *cs = a.rope + (int64_t)i * (D / 2);
    for (int d = 0; d < D / 2; ++d) {
      const float2 c = cs[d];
      const float x1 = to_f(qp[d]);
      const float x2 = to_f(qp[d + D / 2]);
      qh[d] = (x1 * c.x - x2 * c.y) * a.qscale;
      qh[d + D / 2] = (x2 * c.x + x1 * c.y) * a.qscale;
    }
  }
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int kend = min(p_len, (qt + 1) * 64);
  for (int k0 = 0; k0 < kend; k0 += KT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < KT * D; idx += 64) {
      const int kk = idx / D;
      const int d = idx % D;
      const int j = k0 + kk;
      if (j < p_len) {
        const int64_t off = layer0 + (pool_row(a.pool.table, base, j) * a.heads + h) * D + d;
        ks[kk][d] = to_f(((const T *)a.pool.k)[off]);
        vs[kk][d] = to_f(((const T *)a.pool.v)[off]);
      }
    }
    __syncthreads();
    if (active) {
      const int jn = min(KT, i - k0 + 1);
      for (int kk = 0; kk < jn; ++kk) {
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(qh[d], ks[kk][d], s);
        const float m_new = fmaxf(m_run, s);
        const float alpha = exp2f(m_run - m_new);
        const float p = exp2f(s - m_new);
        l_run = l_run * alpha + p;
        for (int d = 0; d < D; ++d) o[d] = fmaf(p, vs[kk][d], o[d] * alpha);
        m_run = m_new;
      }
    }
  }
  if (active) {
    T *op = (T *)a.out + ((cu + i) * a.heads + h) * D;
    const float inv = 1.f / l_run;
    for (int d = 0; d < D; ++d) op[d] = from_f<T>(o[d] * inv);
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

hipError_t launch_ring_write(const RingWriteArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((ring_write_kernel<T, D>), dim3(a.n * a.heads), dim3(64), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_advance(const AdvanceArgs &a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(advance_kernel, dim3((a.n + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    const int64_t tasks = (int64_t)a.num_splits * a.heads;
    const dim3 grid((unsigned)((tasks + 3) / 4));
    if (a.pool.table)
      hipLaunchKernelGGL((decode_split_kernel<T, D, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<T, D, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_decode_combine(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.n * a.heads), dim3(64), 0, s, a);
    return hipGetLastError();
  });
}

hipError_t launch_prefill_register(const PrefillArgs &a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_register_kernel, dim3((a.n + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_cache_write(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.total_tokens == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((prefill_cache_write_kernel<T, D>), dim3((unsigned)a.total_tokens), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

int prefill_tile_rows(int dtype, int head_dim) { return 64; }

hipError_t launch_prefill_attention(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.num_tiles == 0) return hipSuccess;
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((prefill_attn_valu_kernel<T, D>), dim3(a.num_tiles * a.heads), dim3(64), 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace rswa
