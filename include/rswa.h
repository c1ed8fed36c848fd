/*
 * rswa.h -- C ABI of the R-SWA (Reference Sliding Window Attention) library
 * for AMD MI355X (gfx950).
 *
 * The method [page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘",
 * www.gtnt.cn/news/146005, section 2.1 "环形滑窗注意力"]: the prefill tokens of
 * a request (a document's image tokens plus its prompt) keep complete
 * attention and are never evicted; decode keys/values are appended until the
 * cache holds prefill_len + W entries; from then on each new token overwrites
 * in place the ring slot prefill_len + ring_pos, ring_pos advancing by one
 * modulo W, and attention runs over the whole cache, whose size therefore
 * stays prefill_len + W however long the output grows.
 *
 * Positional encoding is not given on the pages.  This library rotates keys
 * and queries with rotate-half RoPE (frequencies base^(-2i/D)) at the token's
 * absolute position -- prefill token j at j, decode step s at
 * prefill_len + s -- and stores keys already rotated.  ring_pos starts at 0
 * on the first decode step, and the current token's key/value is written
 * before its attention, so the ring window includes the current token.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All device pointers are HIP device memory owned by the caller.  The
 *   library never allocates or frees device memory.  It allocates only the
 *   host-side handle and a small pinned host staging area, both released by
 *   rswa_cache_destroy.  Its only device memory of its own is the fixed
 *   scratch array of rswa_decode_step_fused_noalloc (a static device array of
 *   RSWA_NOALLOC_SCRATCH_BYTES, present on each GPU the library is loaded on
 *   until the process ends).
 * - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *   enqueued asynchronously on it; only rswa_cache_init and rswa_get_state
 *   block.  Use one stream per handle.
 * - Element type of every tensor is the config's dtype (bf16 or fp32).
 * - Layouts (row-major, last index fastest):
 *     pools         [num_layers][num_slots][num_heads][head_dim]
 *     prefill q/k/v/out  [sum of prefill_len][num_heads][head_dim], packed
 *                   in the order of req_ids
 *     decode q/k/v/out   [n][num_heads][head_dim] in rswa_set_batch order
 *   q and k are passed unrotated; the library applies RoPE.
 * - Logical slot i (0 <= i < prefill_len + W) of a request lives at pool
 *   row slot_base + i, or at pool row slot_table[slot_base + i] when the
 *   config has a slot table (page-size-1 layout).
 * - Every entry point validates on the host before launching anything.  A
 *   call that returns an error launched nothing and changed no state;
 *   rswa_last_error gives the reason.  No C++ exception crosses the ABI.
 * - A handle is not thread-safe.
 */
#ifndef RSWA_H
#define RSWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSWA_ABI_VERSION 1

/* Status codes. */
enum {
  RSWA_OK = 0,
  RSWA_E_ARG = -1,         /* bad argument or config value */
  RSWA_E_UNSUPPORTED = -2, /* head_dim / dtype combination not built */
  RSWA_E_POSITION = -3,    /* a position would reach max_positions */
  RSWA_E_CAPACITY = -4,    /* pool, slot table, workspace or batch too small */
  RSWA_E_STATE = -5,       /* call out of order (see each entry point) */
  RSWA_E_HIP = -6          /* a HIP runtime call failed */
};

enum { RSWA_DTYPE_BF16 = 0, RSWA_DTYPE_F32 = 1 };

/* Which keys a decode step attends to.
 *   RSWA_ATTENTION_RSWA: the method [page section 2.1]: every prefill key
 *     plus the newest min(t + 1, W) generated keys.
 *   RSWA_ATTENTION_SWA: the baseline the same section contrasts it with, a
 *     standard sliding window that also cuts the prefill keys: only the
 *     newest W logical positions, P + t + 1 - W .. P + t, prefill and
 *     generated alike.  The cache layout, prefill and ring writes are the
 *     same; prefill attention stays causal.
 * A growing full cache is RSWA_ATTENTION_RSWA with W at least the number of
 * decode steps (the ring never wraps). */
enum { RSWA_ATTENTION_RSWA = 0, RSWA_ATTENTION_SWA = 1 };

typedef struct rswa_config {
  int32_t num_layers;     /* >= 1 */
  int32_t num_heads;      /* >= 1; key/value heads = query heads */
  int32_t head_dim;       /* 64 or 128 */
  int32_t window;         /* W >= 1: generated tokens kept in the ring */
  int32_t max_positions;  /* positions 0 .. max_positions-1; 0 means 32768 */
  int32_t max_requests;   /* request ids are 0 .. max_requests-1 */
  int64_t num_slots;      /* pool rows per layer */
  int32_t dtype;          /* RSWA_DTYPE_BF16 or RSWA_DTYPE_F32 */
  int32_t max_splits;     /* split-KV partial slots in the workspace;
                             0 means max(16384, 4 * max_requests) */
  int64_t max_prefill_tokens; /* largest sum of prefill_len in one
                                 rswa_prefill call; 0 means 262144 */
  int32_t decode_split_tokens; /* keys per split-KV work item, a multiple
                                  of 64; 0 means chosen per batch */
  int32_t attention;      /* RSWA_ATTENTION_RSWA (0) or the baseline
                             RSWA_ATTENTION_SWA (1), see below */
  double rope_base;       /* > 0; 0 means 10000 */
  double softmax_scale;   /* <= 0 means 1/sqrt(head_dim) */
  const int32_t *slot_table; /* device int32[slot_table_len] of pool rows,
                                or NULL for contiguous rows.  Read once at
                                init (entries must lie in [0, num_slots))
                                and then by kernels; must not change while
                                the handle lives. */
  int64_t slot_table_len;
} rswa_config;

typedef struct rswa_cache rswa_cache;

/* ABI version of the loaded library (RSWA_ABI_VERSION). */
int rswa_abi_version(void);

/* Bytes of device workspace rswa_cache_init needs for cfg (0 if cfg is
 * invalid; rswa_last_error(NULL) then says why).  The workspace holds the
 * RoPE table (computed in fp64 on the host, stored fp32), per-request device
 * state, batch tables and split-KV partials. */
size_t rswa_workspace_bytes(const rswa_config *cfg);

/* Create a handle over caller-owned pools and workspace (256-byte aligned).
 * k_pool / v_pool: device [num_layers][num_slots][num_heads][head_dim].
 * Blocks: uploads the RoPE table and validates the slot table.
 * Pool contents are not touched.  On success *out receives the handle. */
int rswa_cache_init(const rswa_config *cfg, void *k_pool, void *v_pool,
                    void *workspace, size_t workspace_bytes, void *stream,
                    rswa_cache **out);

/* Release the handle (host memory only).  Waits for the handle's pending
 * staging copies.  NULL is accepted. */
int rswa_cache_destroy(rswa_cache *c);

/* Prefill one layer for n requests [section 2.1: complete attention over the
 * prefill, nothing evicted; section 三 of the same page: the eager path does
 * this with a full-matrix softmax].
 * req_ids, prefill_len, slot_base: host arrays of n entries.  Layer 0
 * (re)registers each request: prefill_len P >= 0, slot_base, and zero
 * generated tokens; layers 1 .. num_layers-1 must then follow in order with
 * the same values.  Needs P + W rows from slot_base (pool or table), and
 * P <= max_positions.
 * Writes pool rows of logical slots 0 .. P-1 of `layer`: K = RoPE(k, j),
 * V = v.  Writes out[j] = causal attention of RoPE(q_j, j) over keys 0..j
 * (scale softmax_scale).  q, k, v, out: device, packed as above. */
int rswa_prefill(rswa_cache *c, int32_t layer, int32_t n, const int32_t *req_ids,
                 const int32_t *prefill_len, const int64_t *slot_base,
                 const void *q, const void *k, const void *v, void *out,
                 void *stream);

/* Prefill by chunks: the same as rswa_prefill for rows chunk_start[i] ..
 * chunk_start[i] + chunk_len[i] - 1 of each request's prefill (host arrays
 * of n), so a long prompt can be fed in pieces between decode steps of
 * other requests [section 三 of the page names multi-request memory
 * scheduling as open work].  q, k, v, out are packed over the chunks
 * ([sum chunk_len][H][D] in req_ids order).  The chunk's keys/values go to
 * logical slots chunk_start .. ; its queries are rotated at those positions
 * and attend causally to every prefill key written so far in this layer
 * plus their own chunk.  Layer 0 with chunk_start 0 registers the request
 * (prefill_len, slot_base, zero generated tokens); every other chunk must
 * repeat those values, start where its layer stopped, and (for layer > 0)
 * end at or before the rows layer - 1 already holds.  A request joins a
 * decode batch once every layer holds all its prefill_len rows.
 * Errors: as rswa_prefill, and RSWA_E_ARG for a chunk outside prefill_len,
 * RSWA_E_STATE for a chunk out of order. */
int rswa_prefill_chunk(rswa_cache *c, int32_t layer, int32_t n, const int32_t *req_ids,
                       const int32_t *prefill_len, const int64_t *slot_base,
                       const int32_t *chunk_start, const int32_t *chunk_len, const void *q,
                       const void *k, const void *v, void *out, void *stream);

/* Admission and retirement of requests over the pool's rows (host only, no
 * device work).  rswa_admit reserves prefill_len + W consecutive rows of the
 * pool (or slot-table) index space, first fit, for request req_id, which
 * must be neither registered nor admitted, and returns their first index in
 * *slot_base; that request's prefill calls must then pass this slot_base.
 * RSWA_E_CAPACITY when no free range is long enough.  rswa_retire
 * unregisters n requests (host array; none may be in the active decode
 * batch, RSWA_E_STATE) and returns their reserved rows, merged with free
 * neighbours; their ids can be prefilled or admitted again.  Requests
 * placed by the caller's own slot_base are only unregistered.
 * rswa_free_rows reports the rows not reserved by rswa_admit. */
int rswa_admit(rswa_cache *c, int32_t req_id, int32_t prefill_len, int64_t *slot_base);
int rswa_retire(rswa_cache *c, int32_t n, const int32_t *req_ids);
int rswa_free_rows(const rswa_cache *c, int64_t *rows);

/* Select the active decode batch (host array of n distinct ids, each
 * prefilled in every layer) [section 2.1: each request decodes over its own
 * cache -- its whole prefill plus its own W-slot ring -- so a batch is a set
 * of independent requests, each with its own prefill_len and ring_pos].
 * Plans the split-KV work for it.  Must not be called in the middle of a
 * step (after a ring write, before advance: RSWA_E_STATE), nor on a stream
 * that is being captured into a graph (RSWA_E_STATE: it uploads the plan).
 * It invalidates graphs captured before it (see rswa_note_steps). */
int rswa_set_batch(rswa_cache *c, int32_t n, const int32_t *req_ids, void *stream);

/* Ring write for `layer` [section 2.1: in-place overwrite of the ring slot].
 * For active request b with P prefill tokens and t generated tokens so far:
 * slot = P + (t mod W), position = P + t; K[slot] = RoPE(k_new[b], P + t),
 * V[slot] = v_new[b].  Fails with RSWA_E_POSITION if P + t >= max_positions
 * for any active request.  Once per layer per step, before rswa_decode_step
 * of that layer. */
int rswa_ring_write(rswa_cache *c, int32_t layer, const void *k_new,
                    const void *v_new, void *stream);

/* Decode attention for `layer` [section 2.1: attention over the whole cache
 * after the write].  For active request b: out[b] = softmax attention of
 * RoPE(q[b], P + t) over logical slots 0 .. L-1 with L = P + min(t + 1, W):
 * the whole prefill and the newest min(t + 1, W) generated tokens (with
 * RSWA_ATTENTION_SWA only slots max(0, P + t + 1 - W) .. L-1).  Split-KV:
 * partial (max, sum, vector) per split in the workspace, then a combine.
 * q, out: device [n][H][D] in batch order.  Needs this step's
 * rswa_ring_write(layer) first (RSWA_E_STATE otherwise). */
int rswa_decode_step(rswa_cache *c, int32_t layer, const void *q, void *out,
                     void *stream);

/* rswa_ring_write followed by rswa_decode_step for `layer`, in fewer launches:
 * the split-KV kernel itself performs the in-place slot write (the wave
 * whose split holds slot P + (t mod W) writes the rotated key and the value
 * for its head and attends with them).  Same inputs, results, state rules
 * and errors as the two calls (RSWA_E_POSITION, RSWA_E_STATE if this layer
 * was already written or decoded in this step); the pool holds the new row
 * once this call's kernels have run. */
int rswa_decode_step_fused(rswa_cache *c, int32_t layer, const void *q, const void *k_new,
                           const void *v_new, void *out, void *stream);

/* rswa_decode_step_fused for callers that cannot allocate device memory or
 * call hipMalloc (code under graph capture, tight serving loops, harnesses
 * that forbid it): the same kernels, inputs, outputs, state rules and
 * errors, but the split-KV partials go to a fixed device array inside the
 * library instead of the handle's workspace, and no allocating call is made
 * (kernel timing by rswa_profile_* is skipped for this call).  The array
 * holds RSWA_NOALLOC_SCRATCH_BYTES per GPU, from the library's first
 * rswa_cache_init on that GPU until the process ends.  A batch whose
 * partials need more -- num_splits * num_heads * (head_dim * 4 + 8) bytes
 * plus alignment, see rswa_decode_plan -- is refused with RSWA_E_CAPACITY
 * before anything launches.  Every handle on one GPU shares the array:
 * calls that overlap in time on one GPU (on different streams, or from
 * different threads) race and must be ordered by the caller. */
#define RSWA_NOALLOC_SCRATCH_BYTES (16u << 20)
int rswa_decode_step_fused_noalloc(rswa_cache *c, int32_t layer, const void *q,
                                   const void *k_new, const void *v_new, void *out,
                                   void *stream);

/* End the step: t += 1 for every active request [section 2.1: after each
 * generated token the ring position advances by one modulo W,
 * ring_pos = t mod W, and the cache grows by one entry until it holds
 * prefill_len + W].  Needs rswa_decode_step of every layer in this step
 * (RSWA_E_STATE otherwise). */
int rswa_advance(rswa_cache *c, void *stream);

/* Graph replay of whole decode steps, for callers that capture the
 * per-step calls to cut launch latency (page section 三 names a faster
 * ring implementation as open work).  The decode, ring-write and advance
 * kernels read and advance each request's generated count in device
 * memory, so a captured graph of k whole steps (every layer's
 * rswa_ring_write + rswa_decode_step or rswa_decode_step_fused, then
 * rswa_advance) replays correctly on its own; only the host view that the
 * calls validate against has to be told.  The calls made while capturing
 * count as enqueuing those k steps once (they advance the host view);
 * before each further replay call rswa_note_steps(c, k): it checks that
 * no step is half done (RSWA_E_STATE) and that every active request stays
 * below max_positions for k more steps (RSWA_E_POSITION), then advances
 * the host view by k.  Capture only whole steps of one batch, with kernel
 * timing off; rswa_set_batch, rswa_prefill, rswa_prefill_chunk and
 * rswa_get_state refuse a capturing stream (RSWA_E_STATE).  A graph holds
 * the batch's size, split plan and tables as they were at capture, so
 * rswa_note_steps also fails with RSWA_E_STATE unless decode work was
 * captured after the last rswa_set_batch.  The graph reads the same input
 * and output buffers on every replay; refill them between replays. */
int rswa_note_steps(rswa_cache *c, int32_t steps);

/* Read the device-side state of n registered requests (host arrays of n)
 * [section 2.1: the next token goes to slot prefill_len + ring_pos with
 * ring_pos advancing modulo W, and the cache holds at most prefill_len + W
 * entries].  With t generated tokens cached: ring_pos = t mod W (slot
 * offset the next step writes), cache_len = P + min(t, W) (valid entries
 * now), next_pos = P + t (the next token's RoPE position).  Any output
 * pointer may be NULL.  Synchronizes `stream` (RSWA_E_STATE on a capturing
 * stream); fails with RSWA_E_STATE if the device copy of t differs from the
 * host's. */
int rswa_get_state(rswa_cache *c, int32_t n, const int32_t *req_ids,
                   int32_t *ring_pos, int32_t *cache_len, int32_t *next_pos,
                   void *stream);

/* Split-KV split size (keys per work item) and the number of decode work
 * items planned for the current batch; 0s before rswa_set_batch. */
int rswa_decode_plan(const rswa_cache *c, int32_t *split_tokens, int32_t *num_splits);

/* Kernel timing, for measurement.  While enabled, the library records a HIP
 * event pair on the caller's stream immediately before and after every launch
 * of the selected kernels.  rswa_profile_read synchronizes `stream`, returns
 * the summed elapsed milliseconds and the launch count of one kernel since
 * the last read, and resets that kernel's record.  Off by default; enabling
 * it costs two event records per timed launch. */
enum { RSWA_KERNEL_DECODE_SPLIT = 0, RSWA_KERNEL_PREFILL_ATTENTION = 1, RSWA_NUM_KERNELS = 2 };
int rswa_profile_enable(rswa_cache *c, int enable);
int rswa_profile_read(rswa_cache *c, int32_t kernel, double *total_ms, int64_t *launches,
                      void *stream);

/* Windowed no-repeat n-gram ban on decode logits [page section 2.3: the
 * anti-loop processor looks for repeats only inside a sliding window of
 * recent tokens and sets to -inf every token that would reproduce an n-gram
 * of `ngram` tokens found there; defaults ngram = 35, window = 128].
 * Independent of any cache handle.
 *   tokens   device int32 [n][token_stride]: row r holds request r's token
 *            sequence; only its first lengths[r] entries count (lengths
 *            outside [0, token_stride] are clamped into it).
 *   lengths  device int32 [n].
 *   logits   device [n][vocab], RSWA_DTYPE_BF16 or RSWA_DTYPE_F32, updated
 *            in place: for a sequence x_0 .. x_{L-1}, every n-gram x_i ..
 *            x_{i+ngram-1} with max(0, L - window) <= i <= L - ngram whose
 *            first ngram - 1 tokens equal the last ngram - 1 tokens of the
 *            sequence bans x_{i+ngram-1}: logits[r][x] = -inf.  Nothing is
 *            banned when L < ngram or window < ngram; tokens outside
 *            [0, vocab) are skipped.  Other logits are not touched.
 * The caller owns every buffer; asynchronous on `stream`.
 * Errors: RSWA_E_ARG (n < 0, ngram < 1, window < 1, vocab < 1, negative
 * token_stride, unknown dtype, null pointer with n > 0), RSWA_E_UNSUPPORTED
 * (window > RSWA_NGRAM_MAX_WINDOW), RSWA_E_HIP (launch failure). */
enum { RSWA_NGRAM_MAX_WINDOW = 4096 };
int rswa_ngram_ban(const int32_t *tokens, int64_t token_stride, const int32_t *lengths, int32_t n,
                   int32_t ngram, int32_t window, void *logits, int64_t vocab, int32_t dtype,
                   void *stream);

/* Measurement helper, not part of the attention path: reads `bytes` of
 * device memory at `buf` with the decode kernel's 16-byte non-temporal
 * loads, one block of 256 threads (one wavefront per SIMD) per CU, the
 * wavefronts sweeping the buffer together in 8 KB slabs, so that the
 * bytes / kernel time it reaches is the read rate the decode kernel's HBM
 * figure can be set against.  Writes to `sink` (device, at least
 * RSWA_MEASURE_SINK_WORDS uint32) one word per wavefront: the wrapping
 * 32-bit sum of the 32-bit words it read, so for a size that is a multiple
 * of 16 bytes the words written sum to the buffer's word sum; words past
 * the grid's wavefronts are left untouched.  Asynchronous on `stream`.
 * Errors: RSWA_E_ARG (null pointer or zero bytes), RSWA_E_UNSUPPORTED
 * (bytes of 16 TiB or more), RSWA_E_HIP (device query or launch failure). */
enum { RSWA_MEASURE_SINK_WORDS = 4096 };
int rswa_measure_read(const void *buf, uint64_t bytes, uint32_t *sink, void *stream);

/* Measurement helper, not part of the attention path: the bf16 matrix-core
 * rate of this GPU with the prefill kernel's instruction
 * (v_mfma_f32_32x32x16_bf16).  512 blocks of 256 threads (two wavefronts per
 * SIMD on 256 CUs); every lane loads two A and two B fragments of 8 bf16
 * from `operands` (device, RSWA_MEASURE_MFMA_FRAGMENTS x 8 bf16, read only)
 * and runs `iters` iterations of four independent 32x32x16 products, so one
 * call does RSWA_MEASURE_MFMA_FLOPS_PER_ITER * iters flops; the rate depends
 * on the operand values (power), so fill `operands` like the data being
 * priced.  Writes one float per block to `sink` (device, at least 512).
 * Asynchronous on `stream`.  Errors: RSWA_E_ARG (null pointer, iters < 1),
 * RSWA_E_HIP (launch failure). */
enum { RSWA_MEASURE_MFMA_FRAGMENTS = 65536 };
#define RSWA_MEASURE_MFMA_FLOPS_PER_ITER (2048.0 * 4.0 * 2.0 * 32.0 * 32.0 * 16.0)
int rswa_measure_mfma(const void *operands, int32_t iters, float *sink, void *stream);

/* Static name of a status code. */
const char *rswa_status_string(int status);

/* Message of the last failed call on c, or of the last failed handle-less
 * call (rswa_workspace_bytes, rswa_cache_init) when c is NULL.  Valid until
 * the next call on the same handle. */
const char *rswa_last_error(const rswa_cache *c);

#ifdef __cplusplus
}
#endif

#endif /* RSWA_H */
