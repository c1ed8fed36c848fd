// Launch interface between the C-ABI host layer and the gfx950 kernels.
// Each launch_* enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "host_state.hpp"

namespace rswa {

// Where a request's logical slot i lives: pool row table[base + i] when
// table != nullptr, else row base + i.  Row r of layer l starts at element
// l * layer_stride + r * heads * head_dim.
struct PoolArgs {
  void *k;
  void *v;
  int64_t layer_stride;   // elements per layer: num_slots * heads * head_dim
  const int32_t *table;   // nullable
};

struct StateArgs {
  int32_t *plen;          // [max_requests]
  int32_t *t;             // [max_requests]
  int64_t *base;          // [max_requests]
};

struct RingWriteArgs {
  PoolArgs pool;
  StateArgs st;
  const int32_t *batch_req;   // [n]
  const void *k_new;          // [n][H][D]
  const void *v_new;
  const float2 *rope;         // [max_positions][D/2]
  int32_t n, heads, window, layer;
};

struct DecodeArgs {
  PoolArgs pool;
  StateArgs st;
  const SplitDesc *splits;    // [num_splits]
  const int32_t *split_off;   // [n + 1] first split of each batch entry
  const void *q;              // [n][H][D]
  void *out;                  // [n][H][D]
  const void *k_new;          // [n][H][D] or null: ring write fused into the split kernel
  const void *v_new;
  float *part_o;              // [num_splits][H][D]
  float2 *part_ml;            // [num_splits][H]  (running max in log2 units, sum)
  int32_t *merge_cnt;         // [n][H] zero between launches
  int32_t *step_cnt;          // [n] zero between launches
  const float2 *rope;
  float qscale;               // softmax_scale * log2(e)
  uint32_t layer_bytes;       // bytes of one layer of a pool (< 2^32)
  int32_t n, heads, window, layer, num_splits;
  int32_t attention;          // RSWA_ATTENTION_RSWA or RSWA_ATTENTION_SWA
  int32_t advance;            // nonzero: this launch ends the step (t += 1 per entry)
  int32_t wpb;                // waves per block, 1 .. kDecodeMaxWavesPerBlock
};

struct PrefillArgs {
  PoolArgs pool;
  StateArgs st;
  const int32_t *req;         // [n]
  const int32_t *plen;        // [n] rows of this call (chunk length)
  const int32_t *qoff;        // [n] position (logical slot) of the chunk's first row
  const int32_t *ptot;        // [n] the request's whole prefill_len
  const int64_t *cu;          // [n + 1] packed token offsets
  const int64_t *base;        // [n]
  const int32_t *tiles;       // [2 * num_tiles] launch slots (b, qt << 16 | head as uint32); b < 0 empty
  const void *q;              // [total][H][D]
  const void *k;
  const void *v;
  void *out;
  const float2 *rope;
  float qscale;
  uint32_t layer_bytes;       // bytes of one layer of a pool (< 2^32 - 64 with a slot table)
  int32_t n, heads, layer, num_tiles, tile;
  int64_t total_tokens;
};

// dtype: RSWA_DTYPE_BF16 or RSWA_DTYPE_F32; head_dim 64 or 128.
hipError_t launch_ring_write(const RingWriteArgs &a, int dtype, int head_dim, hipStream_t s);
// Split-KV decode attention with the cross-split merge in the same launch
// (and, with DecodeArgs::advance, the step's t += 1).
hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, hipStream_t s);
// Decode waves the current device keeps resident at once for (dtype,
// head_dim): the fewest over the kernel's layout / fused variants.
hipError_t decode_resident_waves(int dtype, int head_dim, int64_t *waves);
hipError_t launch_prefill_register(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_cache_write(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s);
// bf16 MFMA causal prefill attention (query tiles of prefill_mfma_rows() rows).
bool prefill_mfma_supported(int dtype, int head_dim);
// Query rows per block of the MFMA prefill kernel.
int prefill_mfma_rows();
hipError_t launch_prefill_mfma(const PrefillArgs &a, int head_dim, hipStream_t s);
// Query-tile height the prefill attention kernel for (dtype, head_dim) uses.
int prefill_tile_rows(int dtype, int head_dim);
hipError_t launch_prefill_attention(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s);

// Device address, on the current device, of the fixed scratch array that
// rswa_decode_step_fused_noalloc keeps its split-KV partials in
// (RSWA_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned).
hipError_t noalloc_scratch_address(void **out);

}  // namespace rswa
