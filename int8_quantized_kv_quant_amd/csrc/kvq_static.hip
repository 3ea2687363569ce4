// The library's fixed device scratch for kv_decode_attn_static, the decode
// entry point that allocates nothing: the split-K partials live in a
// file-scope device array of kStaticScratchBytes instead of a caller workspace.
//
// Host code never uses the array's name as a device address (in host code it
// names a host-side stand-in). The first call on each device, with that device
// current, asks the runtime for the array's address on that device
// (hipGetSymbolAddress) and keeps it; kernels receive that address as their
// workspace argument. Every device holds its own copy of the array until the
// process ends, and every call on a device shares it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return KVQ_OK;
}

}  // namespace kvq
