// The whole layer on a fixed device scratch buffer, for callers that cannot
// allocate (code under stream capture, tight serving loops, hosts that forbid
// device allocation).  The buffer is a file-scope device array: each GPU the
// library runs on holds its own copy from the moment the code object loads
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in for the symbol); it
// uses the device address that hipGetSymbolAddress returns, looked up once
// per device with that device current.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (different streams, or threads) race on it.  The layer writes every
// part of its workspace before reading it, so nothing has to start at zero
// and the contents a previous call left behind are never read.
#include <mutex>

#include "internal.h"

namespace k3 {
namespace {

static __device__ __align__(256) unsigned char scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lookup;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device id, set under g_lookup

// Device address of this device's scratch array (looked up on the first call
// made with the device current); nullptr with *err set on failure.
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_lookup);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace
}  // namespace k3

using namespace k3;

extern "C" k3moe_status k3moe_layer_noalloc(const k3moe_shape* shape,
                                            const k3moe_layer_weights* weights, const void* x,
                                            void* out, int32_t* diag, void* stream) {
  size_t need = 0;
  const k3moe_status st = layer_validate(shape, weights, x, out, diag, &need);
  if (st != K3MOE_OK) return st;
  if (shape->T == 0) return K3MOE_OK;
  if (need > (size_t)K3MOE_NOALLOC_SCRATCH_BYTES)
    return workspace_too_small((size_t)K3MOE_NOALLOC_SCRATCH_BYTES, need);
  hipError_t err = hipSuccess;
  void* ws = scratch_address(&err);
  if (!ws) return hip_failure(err, "k3moe_layer_noalloc: scratch address");
  return layer_run(*shape, *weights, x, out, diag, ws, static_cast<hipStream_t>(stream));
}
