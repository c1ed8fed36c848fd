// Fixed device scratch of rswa_decode_step_fused_noalloc, the decode entry
// point that allocates nothing: its split-KV partials (per split and head, a
// fp32 vector of head_dim values plus the (max, sum) pair) live in this
// file-scope array instead of the handle's workspace.  Every GPU the library
// runs on holds its own copy, RSWA_NOALLOC_SCRATCH_BYTES bytes, until the
// process ends; all handles on one GPU share it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"
#include "rswa.h"

namespace rswa {
namespace {

static __device__ __align__(256) unsigned char scratch[RSWA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Device address of `scratch` on the current device, resolved once per
// device with hipGetSymbolAddress (the array's name is only a host-side
// stand-in and must never reach a kernel).
hipError_t noalloc_scratch_address(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace rswa
