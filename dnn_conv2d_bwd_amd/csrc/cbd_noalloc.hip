// cbd_noalloc.hip -- cbd_run_noalloc: cbd_run_ws with a workspace that the
// library holds itself, in a device array of fixed size, for callers that
// cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "cbd_internal.h"

namespace {

// The workspace of cbd_run_noalloc: one copy on each GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: only the address hipGetSymbolAddress returns
// for the current device is ever passed on.
static __device__ __align__(256) unsigned char scratch[CBD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of each GPU's copy (null: not looked up yet)

// Device address of the current device's copy, looked up on the first call
// on that device (with it current) and kept.
cbd_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    cbd::set_error(std::string("hipGetDevice failed: ") + hipGetErrorName(e));
    return CBD_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    cbd::set_error("cbd_run_noalloc supports device ordinals below 64");
    return CBD_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      cbd::set_error(std::string("hipGetSymbolAddress of the static workspace failed: ") +
                     hipGetErrorName(e));
      return CBD_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CBD_OK;
}

}  // namespace

extern "C" cbd_status cbd_run_noalloc(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                                      void* stream) {
  if (!plan || !dy || !w || !dx) {
    cbd::set_error("NULL plan or tensor pointer");
    return CBD_ERR_INVALID_ARG;
  }
  const uint64_t cap = CBD_NOALLOC_SCRATCH_BYTES;
  const uint64_t need = (uint64_t)plan->info.workspace_bytes;
  if (need > cap) {
    cbd::set_error("the plan needs " + std::to_string(need) + " bytes of workspace; cbd_run_noalloc holds " +
                   std::to_string(cap) + " (use cbd_run_ws, or a smaller ksplit)");
    return CBD_ERR_UNSUPPORTED;
  }
  const bool use = need > 0 || (plan->split_alt && (uint64_t)plan->split_alt->info.workspace_bytes <= cap);
  void* ws = nullptr;
  if (use) {
    const cbd_status st = scratch_address(&ws);
    if (st != CBD_OK) return st;
  }
  return cbd::run_with_workspace(plan, dy, w, dx, ws, use ? cap : 0, stream);
}
