// Measurement helpers, not part of the attention path:
//   - a plain streaming read of device memory, giving the HBM read rate that
//     this GPU reaches with the same load instruction the decode kernel uses
//     (16-byte non-temporal buffer loads): one wavefront per SIMD, all of
//     them sweeping the buffer together in 8 KB slabs, the pattern that
//     reads fastest here (one contiguous chunk per wavefront, 2048 chunks in
//     flight, read ~6 % slower);
//   - a matrix-core loop with the prefill kernel's instruction
//     (v_mfma_f32_32x32x16_bf16) on operands taken from a caller buffer, two
//     wavefronts per SIMD, nothing else: the bf16 MFMA rate this GPU
//     sustains for a given operand distribution (with random operands the
//     matrix cores draw more power and the clock settles lower than with
//     zeros or repeated values).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "device_common.hpp"
#include "rswa.h"

namespace rswa {
namespace {

using namespace dev;

constexpr int kReadThreads = 256;  // four wavefronts: one per SIMD of the CU
constexpr int kUnroll = 8;         // 16-byte loads in flight per lane
constexpr uint32_t kSlab = 64u * 16u * kUnroll;  // bytes of one wavefront pass

// Wavefront w reads slabs w, w + W, w + 2W, ... (W wavefronts in the grid),
// so at any moment the grid reads one contiguous stretch of the buffer.
// Loads past the end are cut off by the slab's resource bound.  Each
// wavefront writes the wrapping 32-bit sum of the words it read, so for a
// size that is a multiple of 16 bytes the sink words sum to the buffer's
// word sum: every byte is read exactly once.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const char *buf, uint64_t bytes,
                                                                   uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = (uint64_t)blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6);
  const uint64_t stride = (uint64_t)gridDim.x * (kReadThreads / 64) * kSlab;
  uint32_t acc = 0;
  for (uint64_t s0 = wave * kSlab; s0 < bytes; s0 += stride) {
    const uint64_t left = bytes - s0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + s0, left < kSlab ? (uint32_t)left : kSlab);
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = buf_load16<2>(r, (uint32_t)(u * 64 + lane) * 16u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (int o = 32; o > 0; o >>= 1) acc += (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) sink[wave] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaBlocks = 512;   // 2048 wavefronts: two per SIMD on 256 CUs
constexpr int kMfmaThreads = 256;

// Each lane takes two A and two B fragments (8 bf16 each) from the operand
// buffer and runs four independent accumulation chains; the chains' sum,
// one float per block, keeps the loop live.
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const bf16x8 *ops, int32_t iters,
                                                                float *sink) {
  const int t = blockIdx.x * kMfmaThreads + threadIdx.x;
  const int n = RSWA_MEASURE_MFMA_FRAGMENTS;
  const bf16x8 a0 = ops[(4 * t) % n], a1 = ops[(4 * t + 1) % n];
  const bf16x8 b0 = ops[(4 * t + 2) % n], b1 = ops[(4 * t + 3) % n];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace
}  // namespace rswa

extern "C" int rswa_measure_read(const void *buf, uint64_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0) return RSWA_E_ARG;
  if (bytes >= (1ull << 44)) return RSWA_E_UNSUPPORTED;
  // One block (one wavefront per SIMD) per CU, one sink word per wavefront.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return RSWA_E_HIP;
  const int blocks = std::min(cus, RSWA_MEASURE_SINK_WORDS / (rswa::kReadThreads / 64));
  hipLaunchKernelGGL(rswa::stream_read_kernel, dim3(blocks), dim3(rswa::kReadThreads), 0,
                     (hipStream_t)stream, (const char *)buf, bytes, sink);
  return hipGetLastError() == hipSuccess ? RSWA_OK : RSWA_E_HIP;
}

extern "C" int rswa_measure_mfma(const void *operands, int32_t iters, float *sink, void *stream) {
  if (!operands || !sink || iters < 1) return RSWA_E_ARG;
  hipLaunchKernelGGL(rswa::mfma_loop_kernel, dim3(rswa::kMfmaBlocks), dim3(rswa::kMfmaThreads), 0,
                     (hipStream_t)stream, (const rswa::bf16x8 *)operands, iters, sink);
  return hipGetLastError() == hipSuccess ? RSWA_OK : RSWA_E_HIP;
}
