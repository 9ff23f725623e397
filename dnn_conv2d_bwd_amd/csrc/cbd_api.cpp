// cbd_api.cpp -- cbd_run and the status / error helpers of the C ABI.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "cbd_internal.h"

namespace {
thread_local std::string g_last_error;

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}
}  // namespace

namespace cbd {
void set_error(const std::string& msg) { g_last_error = msg; }
}  // namespace cbd

extern "C" const char* cbd_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* cbd_status_string(cbd_status s) {
  switch (s) {
    case CBD_OK: return "CBD_OK";
    case CBD_ERR_INVALID_ARG: return "CBD_ERR_INVALID_ARG";
    case CBD_ERR_UNSUPPORTED: return "CBD_ERR_UNSUPPORTED";
    case CBD_ERR_HIP: return "CBD_ERR_HIP";
    case CBD_ERR_NO_MEMORY: return "CBD_ERR_NO_MEMORY";
  }
  return "CBD_ERR_UNKNOWN";
}

extern "C" cbd_status cbd_run(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                              void* stream) {
  if (!plan || !dy || !w || !dx) {
    cbd::set_error("NULL plan or tensor pointer");
    return CBD_ERR_INVALID_ARG;
  }
  if (((uintptr_t)dy | (uintptr_t)w | (uintptr_t)dx) & 15u) {
    cbd::set_error("tensor pointers must be 16-byte aligned");
    return CBD_ERR_UNSUPPORTED;
  }
  const cbd::GemmArgs& tmpl = plan->gemm;
  if (overlap(dx, tmpl.dx_bytes, dy, tmpl.dy_bytes) || overlap(dx, tmpl.dx_bytes, w, tmpl.w_bytes)) {
    cbd::set_error("dx overlaps dy or w");
    return CBD_ERR_INVALID_ARG;
  }
  const cbd_plan_info_t& info = plan->info;
  if (info.grid_main > 0) {
    cbd::GemmArgs a = tmpl;
    a.dy = dy;
    a.w = w;
    a.dx = dx;
    int err = 0;
    switch (info.kernel) {
      case CBD_KERNEL_NHWC_BF16: err = cbd::launch_nhwc_bf16(a, info.grid_main, stream); break;
      case CBD_KERNEL_GROUPED:
        err = a.grp_mfma      ? cbd::launch_grouped_mfma(a, info.grid_main, stream)
              : a.grp_rows > 0  ? cbd::launch_grouped_pipe(a, plan->prob.dtype, info.grid_main, stream)
              : a.grp_lds > 0 ? cbd::launch_grouped_rows(a, plan->prob.dtype, info.grid_main, stream)
                              : cbd::launch_grouped(a, plan->prob.dtype, info.grid_main, stream);
        break;
      default: err = cbd::launch_generic(a, plan->prob.layout, plan->prob.dtype, info.grid_main, stream); break;
    }
    if (err) {
      cbd::set_error(std::string("main kernel launch failed: ") + cbd::hip_error_name(err));
      return CBD_ERR_HIP;
    }
  }
  if (info.grid_zero > 0) {
    cbd::ZeroArgs z = plan->zero;
    z.dx = dx;
    const int err = cbd::launch_zero_fill(z, info.grid_zero, stream);
    if (err) {
      cbd::set_error(std::string("zero-fill launch failed: ") + cbd::hip_error_name(err));
      return CBD_ERR_HIP;
    }
  }
  cbd::set_error("");
  return CBD_OK;
}
