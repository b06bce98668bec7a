// moe_layer_forward_noalloc: the whole layer with its intermediate buffers
// (logits, routing, permutation, h, per-pair outputs) in a library-owned
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, serving loops that must
// not call the allocator).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never uses the array's name as an address (on the host the name is only
// a stand-in for the symbol): the first call on a device looks the address up
// with hipGetSymbolAddress, with that device current, and keeps it per device.
// No kernel of the layer needs any part of the array to start at zero (every
// region is written before it is read), so it is never cleared.  Calls that
// overlap on one device share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size is a multiple of the workspace alignment");

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, null until looked up

// The address of this device's copy of `scratch`, looked up once per device.
moe_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_E_DEVICE;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_E_DEVICE;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_E_DEVICE;
    if (e != hipSuccess || !p) return MOE_E_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer* layer, const void* x, int32_t T, float* y,
                                                void* x_next_opt, int32_t* topk_ids_opt, float* topk_w_opt,
                                                void* stream) {
  // argument errors and T == 0 are answered without touching the device
  const size_t need = moe_workspace_bytes(layer, T > 0 ? T : 1);
  if (need == 0 || T <= 0)
    return moe_layer_forward(layer, x, T, y, x_next_opt, topk_ids_opt, topk_w_opt, nullptr, 0, stream);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  int dev = -1;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return MOE_E_DEVICE;
  void* ws = nullptr;
  const moe_status st = scratch_on(dev, &ws);
  if (st != MOE_OK) return st;
  return moe_layer_forward(layer, x, T, y, x_next_opt, topk_ids_opt, topk_w_opt, ws,
                           (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}
