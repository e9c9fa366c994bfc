// fff_forward_static: the whole layer with the library's own fixed scratch
// region as the workspace, for callers that cannot allocate device memory.
//
// The region is a file-scope device array, so every GPU the library runs on
// holds one copy of it from the first use until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
//
// Calls on one GPU share its copy and leave their contents behind.  Nothing
// in it must start at zero: every plan writes each workspace word before
// reading it within a call, and the single-launch decode plan tags its
// cross-workgroup slots with a fresh per-call value.  Calls that overlap on
// one GPU (other streams, other host threads) race on the region.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fff.h"

static __device__ __align__(256) unsigned char scratch[FFF_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of the region (looked up once).
fff_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FFF_ERROR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FFF_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FFF_ERROR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return FFF_SUCCESS;
}

}  // namespace

extern "C" fff_status_t fff_forward_static(const fff_shape_t* shape, const fff_plan_t* plan,
                                           const void* x, const void* W_node, const void* b_node,
                                           const void* V_node, const void* W_out, void* y,
                                           int32_t* path_out, hipStream_t stream,
                                           const fff_stage_events_t* events) {
  // Host-side checks first: a shape or plan the library rejects, or one
  // whose workspace exceeds the region, returns before any HIP call.
  size_t need = 0;
  fff_status_t st = fff_workspace_size(shape, plan, &need);
  if (st != FFF_SUCCESS) return st;
  if (need > FFF_STATIC_SCRATCH_BYTES) return FFF_ERROR_WORKSPACE;
  if (shape->T == 0) return FFF_SUCCESS;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != FFF_SUCCESS) return st;
  return fff_forward(shape, plan, x, W_node, b_node, V_node, W_out, y, path_out, ws,
                     FFF_STATIC_SCRATCH_BYTES, stream, events);
}
