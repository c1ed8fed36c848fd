// Windowed no-repeat n-gram ban on decode logits.
//
// Page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘"
// (www.gtnt.cn/news/146005), section 2.3: long decoding can fall into an
// n-gram loop, so the model's processor looks for repeats only inside a
// sliding window of recent tokens and gives -inf to every token that would
// reproduce an n-gram of ngram_size tokens found there (defaults 35 and 128).
//
// For a sequence x_0 .. x_{L-1} the window is x_{w0} .. x_{L-1},
// w0 = max(0, L - window); each n-gram x_i .. x_{i+n-1} with
// w0 <= i <= L - n whose first n - 1 tokens equal x_{L-n+1} .. x_{L-1} bans
// x_{i+n-1}.  One block per request: the window is staged in LDS, each
// thread tests candidate starts i, and a match writes -inf straight into
// the logits row (several threads may write the same -inf).  The logits are
// never read, so the cost is the window load plus a few scattered stores.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "rswa.h"

namespace rswa {
namespace {

constexpr int kNgramThreads = 128;

template <typename T>
__global__ __launch_bounds__(kNgramThreads) void ngram_ban_kernel(
    const int32_t *tokens, int64_t token_stride, const int32_t *lengths, int32_t ngram,
    int32_t window, T *logits, int64_t vocab) {
  __shared__ int32_t win[RSWA_NGRAM_MAX_WINDOW];
  const int r = blockIdx.x;
  int64_t len = lengths[r];
  len = len < 0 ? 0 : (len > token_stride ? token_stride : len);  // stay inside the row
  if (len < ngram || window < ngram) return;
  const int64_t w0 = len - window > 0 ? len - window : 0;
  const int wl = (int)(len - w0);  // tokens in the window, <= window
  const int32_t *row = tokens + (int64_t)r * token_stride + w0;
  for (int j = threadIdx.x; j < wl; j += kNgramThreads) win[j] = row[j];
  __syncthreads();
  // Window-relative: candidate starts i = 0 .. wl - ngram, prefix at
  // wl - ngram + 1 .. wl - 1.
  const int p0 = wl - ngram + 1;
  T *out = logits + (int64_t)r * vocab;
  for (int i = threadIdx.x; i <= wl - ngram; i += kNgramThreads) {
    bool match = true;
    for (int j = 0; j < ngram - 1 && match; ++j) match = win[i + j] == win[p0 + j];
    if (match) {
      const int32_t t = win[i + ngram - 1];
      if (t >= 0 && t < vocab) out[t] = (T)(-INFINITY);
    }
  }
}

}  // namespace
}  // namespace rswa

extern "C" int rswa_ngram_ban(const int32_t *tokens, int64_t token_stride, const int32_t *lengths,
                              int32_t n, int32_t ngram, int32_t window, void *logits, int64_t vocab,
                              int32_t dtype, void *stream) {
  if (n < 0 || ngram < 1 || window < 1 || vocab < 1 || token_stride < 0) return RSWA_E_ARG;
  if (dtype != RSWA_DTYPE_BF16 && dtype != RSWA_DTYPE_F32) return RSWA_E_ARG;
  if (window > RSWA_NGRAM_MAX_WINDOW) return RSWA_E_UNSUPPORTED;
  if (n == 0) return RSWA_OK;
  if (!tokens || !lengths || !logits) return RSWA_E_ARG;
  const hipStream_t s = (hipStream_t)stream;
  if (dtype == RSWA_DTYPE_BF16)
    hipLaunchKernelGGL(rswa::ngram_ban_kernel<__bf16>, dim3(n), dim3(rswa::kNgramThreads), 0, s,
                       tokens, token_stride, lengths, ngram, window, (__bf16 *)logits, vocab);
  else
    hipLaunchKernelGGL(rswa::ngram_ban_kernel<float>, dim3(n), dim3(rswa::kNgramThreads), 0, s,
                       tokens, token_stride, lengths, ngram, window, (float *)logits, vocab);
  return hipGetLastError() == hipSuccess ? RSWA_OK : RSWA_E_HIP;
}
