// Device helpers shared by the gfx950 kernels: element conversion, 16-byte
// vector unpacking, wavefront reductions, buffer-resource loads and DPP lane
// exchanges.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "rswa.h"

namespace rswa {
namespace dev {

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

// RoPE rotate-half of the pair (x1, x2) = (x_i, x_{i+D/2}) by the angle
// whose (cos, sin) is cs: (x1 cos - x2 sin, x2 cos + x1 sin).  Each half is
// one product plus one fused multiply-add, written out so that every kernel
// that writes a key row rounds it identically.
__device__ __forceinline__ float rope_lo(float x1, float x2, float2 cs) {
  return fmaf(x1, cs.x, -(x2 * cs.y));
}
__device__ __forceinline__ float rope_hi(float x1, float x2, float2 cs) {
  return fmaf(x2, cs.x, x1 * cs.y);
}

__device__ __forceinline__ int64_t pool_row(const int32_t *table, int64_t base, int64_t i) {
  return table ? (int64_t)table[base + i] : base + i;
}

// Raw buffer resource over [p, p + bytes): loads at offsets past `bytes`
// return zero and touch no memory.  Word 3 is the gfx9-family raw-buffer
// format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <int AUX = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

// DPP lane exchanges inside 16-lane rows (gfx9 DPP controls).
enum : int {
  kDppQuadXor1 = 0xB1,        // quad_perm [1,0,3,2]: lane ^ 1
  kDppQuadXor2 = 0x4E,        // quad_perm [2,3,0,1]: lane ^ 2
  kDppRowHalfMirror = 0x141,  // lane ^ 7 within each group of 8
  kDppRowMirror = 0x140,      // lane ^ 15 within each row of 16
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of `x` held by lane ^ m, for the partner patterns the reduce-scatter
// uses: m = 15, 7, 2, 1 through DPP inside a 16-lane row; others via
// ds_bpermute.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  if constexpr (M == 1) return dpp<kDppQuadXor1>(x);
  else if constexpr (M == 2) return dpp<kDppQuadXor2>(x);
  else if constexpr (M == 7) return dpp<kDppRowHalfMirror>(x);
  else if constexpr (M == 15) return dpp<kDppRowMirror>(x);
  else return __shfl_xor(x, M);
}

}  // namespace dev
}  // namespace rswa
