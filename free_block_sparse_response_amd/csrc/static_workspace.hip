// sparsepr_plan_static: sparsepr_plan with the plan's device state in a library-owned
// static device array instead of a caller workspace, for callers that cannot allocate
// device memory. Declaration, limit and sharing rules are documented in include/sparsepr.h.
#include <mutex>

#include "../../include/sparsepr.h"
#include "common.h"

namespace {

// The plan state of every handle planned by sparsepr_plan_static on one GPU. Each GPU the
// library runs on holds its own copy for the life of the process. Host code must never
// pass this name to a kernel or a copy (on the host it is only a stand-in symbol): it
// uses the device address hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[SPARSEPR_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once per device
// (with that device current) and kept.
sparsepr_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPARSEPR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SPARSEPR_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess || !g_ptr[dev]) return SPARSEPR_ERR_HIP;
  *out = g_ptr[dev];
  return SPARSEPR_OK;
}

}  // namespace

extern "C" sparsepr_status sparsepr_plan_static(sparsepr_plan_t plan, const void* q, const void* k, void* stream) {
  if (!plan || !q || !k) return SPARSEPR_ERR_INVALID_ARG;
  if (sparsepr_workspace_bytes(plan) > (size_t)SPARSEPR_STATIC_WORKSPACE_BYTES) return SPARSEPR_ERR_TOO_LARGE;
  void* ws = nullptr;
  const sparsepr_status st = scratch_address(&ws);
  if (st != SPARSEPR_OK) return st;
  // the same planner; every buffer it reads is written first in this call (status words,
  // padding of the permuted keys and values included), so nothing needs clearing here
  return sparsepr_plan(plan, q, k, ws, (size_t)SPARSEPR_STATIC_WORKSPACE_BYTES, stream);
}
