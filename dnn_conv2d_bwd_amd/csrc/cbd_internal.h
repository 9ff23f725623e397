// cbd_internal.h -- the plan object and the launchers behind the C ABI.
#pragma once
#include <string>
#include <vector>

#include "../../include/cbd.h"
#include "cbd_kernarg.h"

struct cbd_plan_s {
  cbd_problem prob;
  cbd_plan_info_t info;
  std::vector<cbd_subgemm_t> subs;       // in launch (LPT) order, ids 0..R-1
  std::vector<cbd_zero_region_t> zeros;
  cbd::GemmArgs gemm;                    // pointers filled per run
  cbd::ZeroArgs zero;
  int64_t grid_finalize = 0;             // split-K finalising launch (0: none)
  bool per_class = false;                // one main launch per class (ablation)
  // The planner's split-K configuration of the same problem, run by
  // cbd_run_ws when the caller's workspace holds it (null: none).
  cbd_plan_s* split_alt = nullptr;
  cbd_plan_s() = default;
  cbd_plan_s(const cbd_plan_s&) = delete;
  cbd_plan_s& operator=(const cbd_plan_s&) = delete;
  ~cbd_plan_s() { delete split_alt; }
};

namespace cbd {

// Thread-local error detail for CBD_ERR_HIP and planner rejections.
void set_error(const std::string& msg);

// cbd_run_ws: the plan's split configuration when the workspace holds it,
// else the plan itself.
cbd_status run_with_workspace(const cbd_plan_t* plan, const void* dy, const void* w, void* dx,
                              void* workspace, uint64_t workspace_bytes, void* stream);

// Launchers (defined next to their kernels).  Each returns 0 or a hipError_t.
int launch_generic(const GemmArgs& a, int layout, int dtype, int64_t grid, void* stream);
int launch_nhwc_bf16(const GemmArgs& a, int64_t grid, void* stream);
int launch_splitk_finalize(const GemmArgs& a, int64_t grid, void* stream);
int launch_generic_finalize(const GemmArgs& a, int layout, int dtype, int64_t grid, void* stream);
int launch_grouped(const GemmArgs& a, int dtype, int64_t grid, void* stream);
int launch_grouped_rows(const GemmArgs& a, int dtype, int64_t grid, void* stream);
int launch_grouped_pipe(const GemmArgs& a, int dtype, int64_t grid, void* stream);
int launch_grouped_mfma(const GemmArgs& a, int64_t grid, void* stream);
int launch_grouped_wide(const GemmArgs& a, int64_t grid, void* stream);
int launch_nchw_rows(const GemmArgs& a, int dtype, int64_t grid, void* stream);
int launch_zero_fill(const ZeroArgs& z, int64_t grid, void* stream);
const char* hip_error_name(int err);

// Tile shapes of each kernel family (the planner sizes grids with them).
constexpr int kGenericBM = 64, kGenericBN = 64, kGenericBK = 16, kGenericThreads = 256;  // tiles 64 or 32
// k-tile width of the generic family: 8 for 32x32 tiles (short K loops of
// small problems: more, shorter gather chains), 16 for larger tiles.
constexpr int generic_bk(int bm, int bn) { return bm * bn <= 32 * 32 ? 8 : kGenericBK; }
constexpr int kFastBM = 256, kFastBN = 256, kFastBK = 32, kFastThreads = 256, kFastMaxTaps = 16;
constexpr int kFastMaxKTiles = 4096;  // k tiles per tap (K/G / 32): bound of the kernel's tap division
constexpr int kGroupedThreads = 256, kGroupedMaxTaps = 9;
constexpr int kGroupedRowLds = 64 * 1024;  // one-row kernel: staged dY rows per workgroup
constexpr int kLdsPerCu = 160 * 1024;       // gfx950 LDS per compute unit (also the per-workgroup limit)
constexpr int kZeroThreads = 256, kZeroItemsPerThread = 2;
constexpr int kRowsThreads = 256;
// Row-block family staging capacity per lane: dY loads (k planes per wave
// x 64-element chunks per plane) and 16-byte W loads.
constexpr int kRowsMaxChunks = 4, kRowsMaxDyLoads = 64, kRowsMaxWLoads = 16;

}  // namespace cbd
