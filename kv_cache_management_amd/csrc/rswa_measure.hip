// Measurement helper: a plain streaming read of device memory, giving the
// HBM read rate that this GPU reaches with the same load instruction the
// decode kernel uses (16-byte non-temporal buffer loads, large contiguous
// chunk per wavefront).  Not part of the attention path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "rswa.h"

namespace rswa {
namespace {

using namespace dev;

constexpr int kReadBlocks = 4096;
constexpr int kReadThreads = 256;
constexpr int kUnroll = 8;

// Block b reads the b-th of kReadBlocks equal contiguous chunks (the tail
// past `bytes` reads zero through the buffer resource bound).  Each wave
// streams its own quarter of the chunk with kUnroll 16-byte loads in flight
// per lane.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const char *buf, uint64_t bytes,
                                                                   uint64_t chunk, uint32_t *sink) {
  const uint64_t b0 = (uint64_t)blockIdx.x * chunk;
  if (b0 >= bytes) {
    if (threadIdx.x == 0) sink[blockIdx.x] = 0;
    return;
  }
  const uint64_t len = bytes - b0 < chunk ? bytes - b0 : chunk;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf + b0, (uint32_t)len);
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint32_t wchunk = (uint32_t)(chunk / 4);
  uint32_t acc = 0;
  for (uint32_t off = (uint32_t)w * wchunk; off < (uint32_t)(w + 1) * wchunk;
       off += 64u * 16u * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = buf_load16<2>(r, off + (uint32_t)(u * 64 + lane) * 16u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // Keep the loads live: one word per block.
  acc = (uint32_t)__shfl_xor((int)acc, 1) ^ acc;
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace
}  // namespace rswa

extern "C" int rswa_measure_read(const void *buf, uint64_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0) return RSWA_E_ARG;
  // Equal chunks, a multiple of one wave pass (64 lanes x 16 B x kUnroll)
  // per wave, each below 4 GiB for the 32-bit buffer offsets.
  const uint64_t quantum = 4ull * 64 * 16 * rswa::kUnroll;
  uint64_t chunk = (bytes + rswa::kReadBlocks - 1) / rswa::kReadBlocks;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  if (chunk >= (1ull << 32)) return RSWA_E_UNSUPPORTED;
  hipLaunchKernelGGL(rswa::stream_read_kernel, dim3(rswa::kReadBlocks), dim3(rswa::kReadThreads), 0,
                     (hipStream_t)stream, (const char *)buf, bytes, chunk, sink);
  return hipGetLastError() == hipSuccess ? RSWA_OK : RSWA_E_HIP;
}
