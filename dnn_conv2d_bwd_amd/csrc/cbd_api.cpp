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

namespace {

cbd_status run_impl(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                    void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!plan || !dy || !w || !dx) {
    cbd::set_error("NULL plan or tensor pointer");
    return CBD_ERR_INVALID_ARG;
  }
  const uint64_t need = (uint64_t)plan->info.workspace_bytes;
  if (need > 0) {
    if (!workspace) {
      cbd::set_error("the plan splits K and needs a workspace (cbd_run_ws)");
      return CBD_ERR_INVALID_ARG;
    }
    if (workspace_bytes < need) {
      cbd::set_error("workspace smaller than cbd_plan_workspace_size");
      return CBD_ERR_INVALID_ARG;
    }
    if ((uintptr_t)workspace & 255u) {
      cbd::set_error("workspace must be 256-byte aligned");
      return CBD_ERR_UNSUPPORTED;
    }
    if (overlap(workspace, need, dx, plan->gemm.dx_bytes) ||
        overlap(workspace, need, dy, plan->gemm.dy_bytes) ||
        overlap(workspace, need, w, plan->gemm.w_bytes)) {
      cbd::set_error("workspace overlaps a tensor");
      return CBD_ERR_INVALID_ARG;
    }
  }
  {
    const cbd_plan_info_t& in = plan->info;
    if (((uintptr_t)dy & (uintptr_t)(in.align_dy - 1)) || ((uintptr_t)w & (uintptr_t)(in.align_w - 1)) ||
        ((uintptr_t)dx & (uintptr_t)(in.align_dx - 1))) {
      cbd::set_error("a tensor pointer is not aligned as the plan requires (dy " + std::to_string(in.align_dy) +
                     ", w " + std::to_string(in.align_w) + ", dx " + std::to_string(in.align_dx) + " bytes)");
      return CBD_ERR_UNSUPPORTED;
    }
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
    a.ws = need > 0 ? workspace : nullptr;
    auto launch_main = [&](const cbd::GemmArgs& args, int64_t grid) -> int {
      switch (info.kernel) {
        case CBD_KERNEL_NHWC_BF16: return cbd::launch_nhwc_bf16(args, grid, stream);
        case CBD_KERNEL_NCHW_ROWS: return cbd::launch_nchw_rows(args, plan->prob.dtype, grid, stream);
        case CBD_KERNEL_GROUPED:
          return args.grp_wide      ? cbd::launch_grouped_wide(args, grid, stream)
                 : args.grp_mfma    ? cbd::launch_grouped_mfma(args, grid, stream)
                 : args.grp_rows > 0 ? cbd::launch_grouped_pipe(args, plan->prob.dtype, grid, stream)
                 : args.grp_lds > 0  ? cbd::launch_grouped_rows(args, plan->prob.dtype, grid, stream)
                                     : cbd::launch_grouped(args, plan->prob.dtype, grid, stream);
        default: return cbd::launch_generic(args, plan->prob.layout, plan->prob.dtype, grid, stream);
      }
    };
    int err = 0;
    if (plan->per_class) {
      // One launch per class (an ablation of the single launch): the class
      // alone in the descriptor table, its tiles numbered from 0.
      for (size_t i = 0; i < plan->subs.size() && !err; i++) {
        cbd::GemmArgs c = a;
        c.sub[0] = a.sub[i];
        c.sub[0].tile_begin = 0;
        c.class_begin[0] = 0;
        if (info.kernel == CBD_KERNEL_GENERIC && a.tile_n > 0) {  // the class's divisor reciprocals at index 0
          const cbd::SubDesc& d = a.sub[i];
          const int64_t npix = int64_t(d.pos_h) * d.pos_w;
          c.mag_npix[0] = cbd::recip32(npix);
          c.mag_posw[0] = cbd::recip32(d.pos_w);
          c.mag_pergroup[0] = cbd::recip32(int64_t(a.tiles_m) * ((int64_t(a.N) * npix + a.tile_n - 1) / a.tile_n));
        }
        c.num_sub = 1;
        c.total_tiles = (int32_t)plan->subs[i].tiles;
        err = launch_main(c, plan->subs[i].tiles);
      }
    } else {
      err = launch_main(a, info.grid_main);
    }
    if (err) {
      cbd::set_error(std::string("main kernel launch failed: ") + cbd::hip_error_name(err));
      return CBD_ERR_HIP;
    }
    if (a.ksplit > 1) {
      const int ferr =
          info.kernel == CBD_KERNEL_GENERIC
              ? cbd::launch_generic_finalize(a, plan->prob.layout, plan->prob.dtype, plan->grid_finalize, stream)
              : cbd::launch_splitk_finalize(a, plan->grid_finalize, stream);
      if (ferr) {
        cbd::set_error(std::string("split-K finalising launch failed: ") + cbd::hip_error_name(ferr));
        return CBD_ERR_HIP;
      }
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

}  // namespace

namespace cbd {
cbd_status run_with_workspace(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                              void* workspace, uint64_t workspace_bytes, void* stream) {
  // The planner's split configuration when the workspace holds it.
  if (plan && plan->split_alt && workspace &&
      workspace_bytes >= (uint64_t)plan->split_alt->info.workspace_bytes)
    return run_impl(plan->split_alt, dy, w, dx, workspace, workspace_bytes, stream);
  return run_impl(plan, dy, w, dx, workspace, workspace_bytes, stream);
}
}  // namespace cbd

extern "C" cbd_status cbd_run(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                              void* stream) {
  return run_impl(plan, dy, w, dx, nullptr, 0, stream);
}

extern "C" cbd_status cbd_run_ws(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                                 void* workspace, uint64_t workspace_bytes, void* stream) {
  return cbd::run_with_workspace(plan, dy, w, dx, workspace, workspace_bytes, stream);
}

extern "C" cbd_status cbd_plan_workspace_size(const cbd_plan_t* plan, uint64_t* bytes) {
  if (!plan || !bytes) {
    cbd::set_error("NULL plan or output");
    return CBD_ERR_INVALID_ARG;
  }
  *bytes = (uint64_t)(plan->info.workspace_bytes > 0 ? plan->info.workspace_bytes
                                                      : plan->info.auto_workspace_bytes);
  return CBD_OK;
}
