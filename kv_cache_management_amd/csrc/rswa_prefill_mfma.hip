// Causal prefill attention on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// The prefill segment keeps complete attention and loses no token (page
// "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘", www.gtnt.cn/news/146005,
// section 2.1); the page's eager path computes it with a full-matrix softmax
// (section 三).  Here it is a flash-attention forward: one block per (query
// tile of kBM rows, head, request), kWaves wavefronts of 32 query rows each, key
// tiles of 64 streamed through LDS (K and V tiles double-buffered apart, one
// barrier per tile), online softmax in base 2.  Tiles go from the pool to LDS
// without passing through registers (buffer loads with the LDS destination),
// into an unpadded layout whose 16-byte chunks are XOR-swizzled per row.  The
// loop is software-pipelined one tile deep: while the probabilities of tile k
// run on the VALU, the scores of tile k + 1 run on the matrix cores, and P.V
// of tile k runs beside the row max of tile k + 1.
//
// Per wavefront and key tile:
//   S^T (64 keys x 32 queries) = K (64 x D) . Q^T (D x 32): A = K rows from
//     LDS, B = the wave's rotated queries held in registers.  In the result
//     layout each lane owns one query column, so row max / sum are in-lane
//     plus one exchange with lane ^ 32.
//   O^T (D x 32) += V^T (D x 64) . P^T (64 x 32): B = the probabilities,
//     straight from the S^T registers (converted to bf16), A = V^T, read
//     from the V tile with the transposing LDS read
//     (ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
//     j mod 4 of the 64-bit rows addressed by lanes 4e + j/4, e = 0..3, so
//     one read turns a 4-key x 16-dim block into 4 keys per lane).  The key
//     order inside each 16-key MFMA step follows the S^T register layout.
//   The running max is raised (and the output rescaled) only when a row's
//   max grows by more than 8 in log2 units, so probabilities stay <= 2^8;
//   the final division by the row sum, taken against the same max, is exact.
// Keys come from the pool (already rotated by the cache write); queries are
// rotated on load at their absolute positions.  Probabilities are rounded to
// bf16 for the P.V product; accumulation is fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "rswa.h"

namespace rswa {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 4 x bf16 from the transposing LDS read.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16 *p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(const void *)p);
  return __builtin_bit_cast(bf16x4, v);
}

// Wavefronts per block, 32 query rows each.
#ifndef RSWA_PREFILL_WAVES
#define RSWA_PREFILL_WAVES 8
#endif
constexpr int kWaves = RSWA_PREFILL_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per block
constexpr int kBN = 64;           // keys per tile

// Blocks per CU the register budget is sized for: two wavefronts per SIMD.
constexpr int kMinBlocks = 8 / kWaves;

// 16-byte chunk position of chunk c in LDS row r: c ^ swz(r).  K rows are
// read 16 at a time at one chunk index, V rows 8 at a time at 4 chunks by
// the transposing read; the XOR patterns keep both conflict-free without
// padding, so a tile is one contiguous block the loads can write directly.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

typedef __attribute__((address_space(3))) void lds_void;

// Barrier that also publishes this wave's writes to LDS.  The workgroup
// fence of __syncthreads does not wait for loads whose destination is LDS,
// so each wave first waits until its own have landed, and its LDS stores
// too (vmcnt = lgkmcnt = 0; gfx9 s_waitcnt fields: vmcnt [15:14,3:0],
// expcnt [6:4], lgkmcnt [11:8]).
__device__ __forceinline__ void lds_publish_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes bytes
// 16 i .. 16 i + 15 after the wave-uniform address `lds`; completion is
// counted by vmcnt.  (Kept out of the kernel's lambdas: called directly from
// one, the builtin makes the host pass drop the kernel's launch stub.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, bf16 *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, 0, 0, 0);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads, kMinBlocks) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  constexpr int KLD = kBN * CPR / kThreads;  // chunks per thread per tile
  constexpr int TILE = kBN * D;              // elements per tile buffer
  static_assert(KLD >= 1 && kBN * CPR % kThreads == 0, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) bf16 lk0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 lk1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 lv0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 lv1[TILE];

  const int b = a.tiles[2 * blockIdx.x];
  if (b < 0) return;  // empty launch slot
  const uint32_t slot = (uint32_t)a.tiles[2 * blockIdx.x + 1];  // qt << 16 | head, unsigned
  const int qt = (int)(slot >> 16);
  const int h = (int)(slot & 0xffffu);
  const int c_len = a.plen[b];   // query rows of this call (a chunk of the prefill)
  const int q_off = a.qoff[b];   // position of the chunk's first row
  const int64_t base = a.base[b];
  const int64_t cu = a.cu[b];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;
  const int li = qt * kBM + w * 32 + (lane & 31);  // this lane's query row in the chunk
  const int q0 = q_off + qt * kBM + w * 32;        // position of this wave's first row
  const int qi = q0 + (lane & 31);                 // position of this lane's row
  const int row_stride = a.heads * D;
  const int32_t *table = a.pool.table;

  // Keys past the end of the pool rows are masked, but their V rows still
  // enter the P.V product with weight 0: start from finite (zero) tiles.
  {
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (int i = tid; i < TILE / 8; i += kThreads) {
      ((uint4 *)lk0)[i] = z;
      ((uint4 *)lk1)[i] = z;
      ((uint4 *)lv0)[i] = z;
      ((uint4 *)lv1)[i] = z;
    }
  }

  // ---- queries: B operand fragments, rotated at their positions ----------
  // (loaded once the first key/value tiles are requested, so both latencies
  // overlap)
  bf16x8 qf[KS];
  auto load_queries = [&]() {
    float qv[KS][8];
    const bool qok = li < c_len;
    const bf16 *qp = (const bf16 *)a.q + ((cu + (qok ? li : 0)) * a.heads + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = qok ? *(const uint4 *)(qp + 16 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      Vec16<bf16>::unpack(u, qv[ks]);
    }
    const float2 *cs = a.rope + (int64_t)(qok ? qi : 0) * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 c = cs[16 * ks + 8 * g + e];
        const float x1 = qv[ks][e];
        const float x2 = qv[ks + KS / 2][e];
        qf[ks][e] = (bf16)(x1 * c.x - x2 * c.y);
        qf[ks + KS / 2][e] = (bf16)(x2 * c.x + x1 * c.y);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float qscale = a.qscale;

  // Keys 0 .. kend-1 are in the pool: earlier chunks plus this one's rows.
  const int kend = q_off + min(c_len, qt * kBM + kBM);
  const int ntile = (kend + kBN - 1) / kBN;

  // ---- tile loads: pool -> LDS directly (16 bytes per lane) --------------
  // Thread-chunk idx = tid + kThreads * it of a tile lands at byte 16 * idx
  // of the tile buffer (row idx / CPR, position idx % CPR) and holds chunk
  // position ^ swz(row) of that key row.  32-bit buffer offsets: contiguous
  // rows use a resource over this request's first kend rows (keys past kend
  // read zero); paged rows use a resource over the layer and an offset past
  // its end for keys past kend.
  const uint32_t row_bytes = (uint32_t)row_stride * 2u;
  const size_t layer_off = (size_t)a.layer * a.pool.layer_stride * 2;
  __amdgpu_buffer_rsrc_t rk, rv;
  if constexpr (PAGED) {
    rk = make_rsrc((const char *)a.pool.k + layer_off, a.layer_bytes);
    rv = make_rsrc((const char *)a.pool.v + layer_off, a.layer_bytes);
  } else {
    const size_t req_off = layer_off + (size_t)base * row_bytes;
    rk = make_rsrc((const char *)a.pool.k + req_off, (uint32_t)kend * row_bytes);
    rv = make_rsrc((const char *)a.pool.v + req_off, (uint32_t)kend * row_bytes);
  }
  uint32_t col_off[KLD];
#pragma unroll
  for (int it = 0; it < KLD; ++it) {
    const int idx = tid + kThreads * it;
    col_off[it] = (uint32_t)(h * D * 2 + (((idx % CPR) ^ swz<D>(idx / CPR)) * 16));
  }
  // Paged layout: pool rows of a tile's keys, fetched from the slot table a
  // step ahead of the loads that use them (-1 past kend).
  int32_t rows_k[KLD], rows_v[KLD];
  auto fetch_rows = [&](int32_t *rows, int k0) {
    if constexpr (PAGED) {
#pragma unroll
      for (int it = 0; it < KLD; ++it) {
        // Clamped index: an unconditional load keeps the loop body one
        // basic block.
        const int j = k0 + (tid + kThreads * it) / CPR;
        const int32_t row = table[base + min(j, kend - 1)];
        rows[it] = j < kend ? row : -1;
      }
    }
  };
  auto tile_off = [&](const int32_t *rows, int k0, int it) -> uint32_t {
    if constexpr (PAGED)
      return rows[it] >= 0 ? (uint32_t)rows[it] * row_bytes + col_off[it] : a.layer_bytes;
    else
      return (uint32_t)(k0 + (tid + kThreads * it) / CPR) * row_bytes + col_off[it];
  };
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, bf16 *buf, int k0, const int32_t *rows) {
#pragma unroll
    for (int it = 0; it < KLD; ++it)
      lds_load16(rs, buf + (w * 64 + kThreads * it) * 8, tile_off(rows, k0, it));
  };
  auto shift_rows = [&]() {
#pragma unroll
    for (int it = 0; it < KLD; ++it) rows_v[it] = rows_k[it];
  };
  // Read addresses (bytes inside a tile buffer).  K: the lane reads row
  // 32 j + (lane & 31), chunk 2 ks + g, at position (g ^ swz(row)) ^ 2 ks.
  // V (transposing read): rows 4 g + (tp >> 2) + 8 hi + 16 hh + 32 j, chunk
  // 4 d + 2 ((lane >> 4) & 1) + ((tp & 3) >> 1), 8-byte half tp & 1, at
  // position (its chunk for d = 0 ^ swz(its row for hi = 0)) ^ (4 d + 2 hi).
  // Rows are 2 D bytes, so the per-read chunk index enters by XOR on the
  // low address bits and j, hh go into the instruction offset.
  const int lrow = lane & 31;
  const int tp = lane & 15;
  const int vrow = 4 * g + (tp >> 2);
  const uint32_t ka0 = (uint32_t)(lrow * D * 2 + ((g ^ swz<D>(lrow)) * 16));
  const uint32_t va0 = (uint32_t)(vrow * D * 2 + 8 * (tp & 1) +
                                  (((2 * ((lane >> 4) & 1) + ((tp & 3) >> 1)) ^ swz<D>(vrow)) * 16));
  // S^T = K . Q^T for the key tile in K buffer `kb`, two 32-key blocks.
  auto scores = [&](const bf16 *kb, f32x16 *s) {
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 ka = *(const bf16x8 *)((const char *)kb + (ka0 ^ (32u * ks)) + 64 * j * D);
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? zero : s[j], 0, 0, 0);
      }
  };
  // Row max of the scores of tile k0 (lane's query column), after the causal
  // mask on tiles that reach this wave's diagonal.
  auto mask_max = [&](f32x16 *s, int k0, bool may_mask) -> float {
    if (may_mask && k0 + kBN - 1 > q0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > qi) s[j][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // Raises the running max when a row's max grows by more than 8 (log2
  // units), rescaling its sum and output.
  auto rescale = [&](float mx) {
    const float m_cand = mx * qscale;
    const bool grow = m_cand > m_run + 8.f;
    if (__any(grow)) {
      const float m_new = grow ? m_cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      m_run = m_new;
    }
  };
  // Probabilities of the 8 keys (j, hh) of each query column as the bf16
  // B operand.  The row sum adds the bf16-rounded weights, the same ones the
  // PV product uses, so the output is an exact convex combination of V rows
  // up to fp32 accumulation (v_dot2 against (1, 1) adds a rounded pair).
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  auto probs = [&](const f32x16 *s, int j, int hh, float &lsum) -> bf16x8 {
    f32x8 pv;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pv[e] = __builtin_amdgcn_exp2f(fmaf(s[j][8 * hh + e], qscale, -m_run));
    const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), ones, lsum, false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), ones, lsum, false);
    return pb;
  };
  // O^T += V^T . P^T over the 16 keys (j, hh) of the V tile `vb`.
  auto pv_block = [&](const bf16 *vb, int j, int hh, bf16x8 pb) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const char *p0 = (const char *)vb + (32 * j + 16 * hh) * D * 2;
      const bf16x4 lo = lds_read_tr4((const bf16 *)(p0 + (va0 ^ (64u * d))));
      const bf16x4 hi = lds_read_tr4((const bf16 *)(p0 + 16 * D + (va0 ^ (64u * d + 32u))));
      o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[d], 0, 0, 0);
    }
  };

  // Pipeline.  K(k) lives in lk(k & 1), V(k) in lv(k & 1).  At the top of
  // step k (after the barrier, whose wait also completes every load the
  // step before issued) the LDS holds K(k+1) and V(k); the registers hold
  // the masked scores and row max of tile k.  Step k issues the loads of
  // K(k+2) into lk[k & 1] and V(k+1) into lv[(k+1) & 1] (both last read in
  // step k-1), then scores of tile k+1 beside the probabilities of tile k,
  // then P.V of tile k beside the row max of tile k+1.  A wave takes part
  // in tile k only if k * kBN <= its last query row.
  const int last_q = q0 + 31;
  auto tile_step = [&](auto steady_c, auto par_c, int k, f32x16 *sc, f32x16 *sn, float mx_cur, float &mx_nxt) {
    constexpr bool kSteady = decltype(steady_c)::value;
    constexpr int kPar = decltype(par_c)::value;
    bf16 *kcur = kPar ? lk1 : lk0;   // K(k): free, receives K(k+2)
    bf16 *knxt = kPar ? lk0 : lk1;   // K(k+1)
    bf16 *vcur = kPar ? lv1 : lv0;   // V(k)
    bf16 *vnxt = kPar ? lv0 : lv1;   // free, receives V(k+1)
    lds_publish_barrier();
    if (kSteady || k + 2 < ntile) dma(rk, kcur, (k + 2) * kBN, rows_k);
    if (kSteady || k + 1 < ntile) dma(rv, vnxt, (k + 1) * kBN, rows_v);
    shift_rows();
    fetch_rows(rows_k, (k + 3) * kBN);
    const bool act = kSteady || k * kBN <= last_q;
    const bool act_n = kSteady || (k + 1 < ntile && (k + 1) * kBN <= last_q);
    if (act) rescale(mx_cur);
    if (act_n) scores(knxt, sn);
    float lsum = 0.f;
    bf16x8 p00, p01, p10, p11;
    if (act) {
      p00 = probs(sc, 0, 0, lsum);
      p01 = probs(sc, 0, 1, lsum);
      p10 = probs(sc, 1, 0, lsum);
      pv_block(vcur, 0, 0, p00);
      pv_block(vcur, 0, 1, p01);
      pv_block(vcur, 1, 0, p10);
      p11 = probs(sc, 1, 1, lsum);
      pv_block(vcur, 1, 1, p11);
      l_run += lsum;
    }
    if (act_n) mx_nxt = mask_max(sn, (k + 1) * kBN, !kSteady);
  };

  // Prologue: K(0), V(0), K(1) loaded; rows of tiles 1 (V) and 2 (K) fetched.
  f32x16 sA[2], sB[2];
  float mxA = -INFINITY, mxB = -INFINITY;
  fetch_rows(rows_k, 0);
  fetch_rows(rows_v, kBN);
  lds_publish_barrier();  // zero fill done before any load writes the tiles
  dma(rk, lk0, 0, rows_k);
  dma(rv, lv0, 0, rows_k);
  dma(rk, lk1, kBN, rows_v);
  fetch_rows(rows_k, 2 * kBN);
  load_queries();
  lds_publish_barrier();

  // A wave with no valid query row (the tail of a chunk's last query tile)
  // only takes its share of the loads, behind the same barriers.
  if (qt * kBM + w * 32 >= c_len) {
    auto load_step = [&](auto par_c, int k) {
      constexpr int kPar = decltype(par_c)::value;
      lds_publish_barrier();
      if (k + 2 < ntile) dma(rk, kPar ? lk1 : lk0, (k + 2) * kBN, rows_k);
      if (k + 1 < ntile) dma(rv, kPar ? lv0 : lv1, (k + 1) * kBN, rows_v);
      shift_rows();
      fetch_rows(rows_k, (k + 3) * kBN);
    };
    for (int kt = 0; kt < ntile; kt += 2) {
      load_step(std::integral_constant<int, 0>{}, kt);
      if (kt + 1 < ntile) load_step(std::integral_constant<int, 1>{}, kt + 1);
    }
    return;
  }

  scores(lk0, sA);
  mxA = mask_max(sA, 0, true);

  // Steady state (pairs of steps): tiles k and k + 1 lie wholly below the
  // block's first query row (no mask, every wave takes part) and tile k + 2
  // exists.  The two steps of a pair swap the score registers and buffers.
  const int steady = max(0, min(ntile - 2, (q_off + qt * kBM) / kBN - 1)) & ~1;
  int kt = 0;
  for (; kt < steady; kt += 2) {
    tile_step(std::true_type{}, std::integral_constant<int, 0>{}, kt, sA, sB, mxA, mxB);
    tile_step(std::true_type{}, std::integral_constant<int, 1>{}, kt + 1, sB, sA, mxB, mxA);
  }
  for (; kt < ntile; kt += 2) {
    tile_step(std::false_type{}, std::integral_constant<int, 0>{}, kt, sA, sB, mxA, mxB);
    if (kt + 1 < ntile)
      tile_step(std::false_type{}, std::integral_constant<int, 1>{}, kt + 1, sB, sA, mxB, mxA);
  }

  if (li >= c_len) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  bf16 *op = (bf16 *)a.out + ((cu + li) * a.heads + h) * D;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[d][4 * q4 + e] * inv);
      *(bf16x4 *)(op + 32 * d + 8 * q4 + 4 * g) = v;
    }
}


}  // namespace

bool prefill_mfma_supported(int dtype, int head_dim) {
  return dtype == RSWA_DTYPE_BF16 && (head_dim == 64 || head_dim == 128);
}

int prefill_mfma_rows() { return kBM; }

hipError_t launch_prefill_mfma(const PrefillArgs &a, int head_dim, hipStream_t s) {
  if (a.num_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_tiles);
  const bool paged = a.pool.table != nullptr;
  if (head_dim == 128 && paged)
    hipLaunchKernelGGL((prefill_mfma_kernel<128, true>), grid, dim3(kThreads), 0, s, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((prefill_mfma_kernel<128, false>), grid, dim3(kThreads), 0, s, a);
  else if (head_dim == 64 && paged)
    hipLaunchKernelGGL((prefill_mfma_kernel<64, true>), grid, dim3(kThreads), 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((prefill_mfma_kernel<64, false>), grid, dim3(kThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rswa
