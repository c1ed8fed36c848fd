// gfx950 kernels of the R-SWA hot path other than decode attention and the
// MFMA prefill attention: ring write (RoPE at the absolute position, in-place
// slot overwrite), prefill registration and cache write, and a VALU causal
// prefill attention used for fp32 and as a reference path.  (The step
// advance, t += 1, runs inside the decode kernel of the step's last layer.)
//
// The cache policy is that of page "开源5天Star破万之后：百度Unlimited-OCR的爆火
// 路径复盘" (www.gtnt.cn/news/146005), section 2.1: prefill rows are kept
// whole, the ring slot after the prefill is overwritten in place at
// prefill_len + ring_pos, and attention runs over the whole cache.  RoPE is
// not on the pages: rotate-half over the head dimension at the absolute
// position, with cos/sin read from a table the host computes in fp64.
#include <hip/hip_runtime.h>

#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"
#include "rswa.h"

namespace rswa {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// Ring write: TPP = (D/2) / EPL threads per (batch entry, head), 64 threads
// per block.  slot = P + (t mod W), position = P + t; K row = RoPE(k_new,
// P + t), V row = v_new.  Thread c moves 16-byte pieces: elements
// [c*EPL, c*EPL + EPL) of the lower half and the same offsets of the upper
// half (their rotation partners) of k and v.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void ring_write_kernel(RingWriteArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int TPP = (D / 2) / EPL;
  const int64_t gid = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int64_t pair = gid / TPP;
  if (pair >= (int64_t)a.n * a.heads) return;
  const int c = (int)(gid % TPP);
  const int b = (int)(pair / a.heads);
  const int h = (int)(pair % a.heads);
  const int r = a.batch_req[b];
  const int p_len = a.st.plen[r];
  const int t = a.st.t[r];
  const int pos = p_len + t;
  const int slot = p_len + t % a.window;
  const int64_t row = pool_row(a.pool.table, a.st.base[r], slot);
  const int64_t dst = (int64_t)a.layer * a.pool.layer_stride + (row * a.heads + h) * D + c * EPL;
  const int64_t src = ((int64_t)b * a.heads + h) * D + c * EPL;
  const uint4 k1 = *(const uint4 *)((const T *)a.k_new + src);
  const uint4 k2 = *(const uint4 *)((const T *)a.k_new + src + D / 2);
  const uint4 v1 = *(const uint4 *)((const T *)a.v_new + src);
  const uint4 v2 = *(const uint4 *)((const T *)a.v_new + src + D / 2);
  float x1[EPL], x2[EPL];
  Vec16<T>::unpack(k1, x1);
  Vec16<T>::unpack(k2, x2);
  const float2 *cs = a.rope + (int64_t)pos * (D / 2) + c * EPL;
  T r1[EPL], r2[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float2 cc = cs[e];
    r1[e] = from_f<T>(rope_lo(x1[e], x2[e], cc));
    r2[e] = from_f<T>(rope_hi(x1[e], x2[e], cc));
  }
  T *K = (T *)a.pool.k + dst;
  T *V = (T *)a.pool.v + dst;
  *(uint4 *)K = __builtin_bit_cast(uint4, r1);
  *(uint4 *)(K + D / 2) = __builtin_bit_cast(uint4, r2);
  *(uint4 *)V = v1;
  *(uint4 *)(V + D / 2) = v2;
}

// ---------------------------------------------------------------------------
// Prefill: registration (layer 0) and the cache write K = RoPE(k, j), V = v.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_register_kernel(PrefillArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.n) return;
  if (a.qoff[b] != 0) return;  // a later chunk: the request is registered
  const int r = a.req[b];
  a.st.plen[r] = a.ptot[b];
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

// Cache write of the prefill: TPP threads per (token, head); thread c moves
// 16-byte pieces: elements [c*EPL, c*EPL + EPL) of the lower half and the
// same offsets of the upper half (its rotation partners) of k and v.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_cache_write_kernel(PrefillArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int TPP = (D / 2) / EPL;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = gid / TPP;
  if (pair >= a.total_tokens * a.heads) return;
  const int c = (int)(gid % TPP);
  const int64_t tok = pair / a.heads;
  const int h = (int)(pair % a.heads);
  const int b = find_request(a.cu, a.n, tok);
  const int j = a.qoff[b] + (int)(tok - a.cu[b]);  // logical slot = position
  const int64_t row = pool_row(a.pool.table, a.base[b], j);
  const int64_t src = (tok * a.heads + h) * D + c * EPL;
  const int64_t dst = (int64_t)a.layer * a.pool.layer_stride + (row * a.heads + h) * D + c * EPL;
  const uint4 k1 = *(const uint4 *)((const T *)a.k + src);
  const uint4 k2 = *(const uint4 *)((const T *)a.k + src + D / 2);
  const uint4 v1 = *(const uint4 *)((const T *)a.v + src);
  const uint4 v2 = *(const uint4 *)((const T *)a.v + src + D / 2);
  float x1[EPL], x2[EPL];
  Vec16<T>::unpack(k1, x1);
  Vec16<T>::unpack(k2, x2);
  const float2 *cs = a.rope + (int64_t)j * (D / 2) + c * EPL;
  T r1[EPL], r2[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float2 cc = cs[e];
    r1[e] = from_f<T>(rope_lo(x1[e], x2[e], cc));
    r2[e] = from_f<T>(rope_hi(x1[e], x2[e], cc));
  }
  T *K = (T *)a.pool.k + dst;
  T *V = (T *)a.pool.v + dst;
  *(uint4 *)K = __builtin_bit_cast(uint4, *(const T(*)[EPL])r1);
  *(uint4 *)(K + D / 2) = __builtin_bit_cast(uint4, *(const T(*)[EPL])r2);
  *(uint4 *)V = v1;
  *(uint4 *)(V + D / 2) = v2;
}

// ---------------------------------------------------------------------------
// Causal prefill attention on the VALU (the fp32 path).  One block of 256
// threads per (query tile of 64 rows, head); LPQ = 4 lanes per query row,
// each holding E = D / 4 elements of the rotated query and of the output
// (element j * E + e in lane j of the row), so no thread keeps a whole head
// vector.  Keys (already rotated, read from the pool) and values are staged
// KT at a time in LDS, element j * E + e of a row at position e * LPQ + j so
// the four lanes of a row read four consecutive words.  A key's score is the
// lanes' partial dot products summed over the row's four lanes; softmax is
// online in base 2.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_attn_valu_kernel(PrefillArgs a) {
  constexpr int KT = 32;
  constexpr int LPQ = 4;
  constexpr int E = D / LPQ;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int b = a.tiles[2 * blockIdx.x];
  if (b < 0) return;  // empty launch slot
  const uint32_t slot = (uint32_t)a.tiles[2 * blockIdx.x + 1];  // qt << 16 | head, unsigned
  const int qt = (int)(slot >> 16);
  const int h = (int)(slot & 0xffffu);
  const int c_len = a.plen[b];   // rows of this chunk
  const int q_off = a.qoff[b];   // position of its first row
  const int64_t base = a.base[b];
  const int64_t cu = a.cu[b];
  const int tid = threadIdx.x;
  const int j = tid % LPQ;                 // this lane's element slice
  const int li = qt * 64 + tid / LPQ;      // row in the chunk
  const int i = q_off + li;                // its position
  const bool active = li < c_len;
  const int64_t layer0 = (int64_t)a.layer * a.pool.layer_stride;

  // Rotated query slice: element d = j * E + e pairs with d +- D/2.
  float qh[E];
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qh[e] = 0.f;
    o[e] = 0.f;
  }
  if (active) {
    const T *qp = (const T *)a.q + ((cu + li) * a.heads + h) * D;
    const float2 *cs = a.rope + (int64_t)i * (D / 2);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = j * E + e;
      const float2 c = cs[d % (D / 2)];
      const float x = to_f(qp[d]);
      const float y = d < D / 2 ? -to_f(qp[d + D / 2]) : to_f(qp[d - D / 2]);
      qh[e] = (x * c.x + y * c.y) * a.qscale;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int kend = q_off + min(c_len, (qt + 1) * 64);
  const int last = q_off + min(c_len, (qt + 1) * 64) - 1;  // the tile's last row position
  for (int k0 = 0; k0 < kend; k0 += KT) {
    __syncthreads();
    for (int idx = tid; idx < KT * D; idx += 256) {
      const int kk = idx / D;
      const int d = idx % D;
      const int jj = k0 + kk;
      if (jj < kend) {
        const int64_t off = layer0 + (pool_row(a.pool.table, base, jj) * a.heads + h) * D + d;
        ks[kk][(d % E) * LPQ + d / E] = to_f(((const T *)a.pool.k)[off]);
        vs[kk][(d % E) * LPQ + d / E] = to_f(((const T *)a.pool.v)[off]);
      }
    }
    __syncthreads();
    const int nk = min(KT, min(kend, last + 1) - k0);  // keys of this tile any row may see
    for (int kk = 0; kk < nk; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(qh[e], ks[kk][e * LPQ + j], part);
      part += __shfl_xor(part, 1);  // sum over the row's four lanes
      const float s = part + __shfl_xor(part, 2);
      if (active && k0 + kk <= i) {
        const float m_new = fmaxf(m_run, s);
        const float alpha = exp2f(m_run - m_new);
        const float p = exp2f(s - m_new);
        l_run = l_run * alpha + p;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(p, vs[kk][e * LPQ + j], o[e] * alpha);
        m_run = m_new;
      }
    }
  }
  if (active) {
    T *op = (T *)a.out + ((cu + li) * a.heads + h) * D;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int e = 0; e < E; ++e) op[j * E + e] = from_f<T>(o[e] * inv);
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
    constexpr int TPP = (D / 2) / (16 / (int)sizeof(T));
    const int64_t threads = (int64_t)a.n * a.heads * TPP;
    hipLaunchKernelGGL((ring_write_kernel<T, D>), dim3((unsigned)((threads + 63) / 64)), dim3(64), 0, s, a);
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
    constexpr int TPP = (D / 2) / (16 / (int)sizeof(T));
    const int64_t threads = a.total_tokens * a.heads * TPP;
    hipLaunchKernelGGL((prefill_cache_write_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

int prefill_tile_rows(int dtype, int head_dim) {
  return prefill_mfma_supported(dtype, head_dim) ? prefill_mfma_rows() : 64;
}

hipError_t launch_prefill_attention(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (a.num_tiles == 0) return hipSuccess;
  if (prefill_mfma_supported(dtype, head_dim)) return launch_prefill_mfma(a, head_dim, s);
  return dispatch(dtype, head_dim, [&](auto tv, auto dv) {
    using T = decltype(tv);
    constexpr int D = decltype(dv)::value;
    hipLaunchKernelGGL((prefill_attn_valu_kernel<T, D>), dim3(a.num_tiles), dim3(256), 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace rswa
