// Range checks of caller-provided routing arrays, compiled into the debug
// library only (libmoe_debug.so, built with MOE_RANGE_CHECKS): its entry
// points that take ids, offsets, sorted pairs or pair positions from the
// caller run this check first and return MOE_E_ARG, enqueueing nothing else,
// when a value is out of range.  The check reads each array inside its own
// extent only and reports through a device word, so a bad value never becomes
// a bad address.  (The ids index the E experts picked by the gating network,
// page 2 "Layer 1: On-Demand MoE Expert Scheduling"; the permutation groups
// the pairs by expert, page 3 "The 'Doorbell' Mechanism".)
#ifdef MOE_RANGE_CHECKS
#include "moe_internal.h"

namespace moe {

static __device__ uint32_t g_range_err;

// bit 0: an id outside [0, E); bit 1: offsets not a non-decreasing run from 0
// to T K; bit 2: a sorted pair outside [0, T K); bit 3: a pair position
// outside [0, T K)
__global__ void k_check_routing(RoutingCheck c) {
  const int n = c.T * c.K;
  const int m = n > c.E + 1 ? n : c.E + 1;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < m; i += gridDim.x * blockDim.x) {
    uint32_t bad = 0;
    if (i < n) {
      if (c.ids && (uint32_t)c.ids[i] >= (uint32_t)c.E) bad |= 1u;
      if (c.sorted && (uint32_t)c.sorted[i] >= (uint32_t)n) bad |= 4u;
      if (c.pos && (uint32_t)c.pos[i] >= (uint32_t)n) bad |= 8u;
    }
    if (c.offsets && i <= c.E) {
      const int v = c.offsets[i];
      if (i == 0 ? v != 0 : (v < c.offsets[i - 1] || v > n)) bad |= 2u;
      if (i == c.E && v != n) bad |= 2u;
    }
    if (bad) atomicOr(&g_range_err, bad);
  }
}

hipError_t check_routing(const RoutingCheck& c, hipStream_t s, uint32_t* err) {
  uint32_t zero = 0;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_range_err), &zero, sizeof(zero), 0, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const int n = c.T * c.K > c.E + 1 ? c.T * c.K : c.E + 1;
  k_check_routing<<<(n + 255) / 256, 256, 0, s>>>(c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(err, HIP_SYMBOL(g_range_err), sizeof(*err), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);  // the host copies above stay valid until here
}

}  // namespace moe
#endif
