// kern_grouped_direct.hip -- grouped backward-data with few channels per
// group (C/G == K/G in {1, 2, 4, 8}; ResNeXt-style 32 groups of 4 is the
// motivating shape): too little reuse per group for a matrix-core tile, so
// each lane accumulates its group's C/G outputs directly.
//
// The same stride-residue classes as the GEMM families (kern_igemm_generic.hip)
// drive the work: a workgroup belongs to one class, so every lane of it walks
// the same tap list (taps cls + T*j; dY row t + beta - delta*j) with no
// divergence, and positions no tap of any class reaches are left to the
// zero-fill launch.
//
// Lane layout: lane = group (G divides 256), slot = tid / G; consecutive
// slots take consecutive positions, so a wave's dY and dX accesses cover
// whole NHWC pixel rows (G*C/G contiguous channels).  Each lane keeps its
// group's filter slice for the class's taps (<= 9) in registers as f32.
#include "cbd_device.h"
#include "cbd_internal.h"
#include "grouped_vec.h"

namespace cbd {
namespace {

using grp::Vec;
using grp::load_vec;
using grp::store_vec;

template <int DT>
__device__ inline float elem(const uint32_t* w, int i) {
  if constexpr (DT == 0) return __uint_as_float(w[i]);
  return dev::bf16_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
}

template <int DT, int CG>
__global__ __launch_bounds__(kGroupedThreads) void grouped_direct_kernel(const GemmArgs a) {
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int VB = CG * ES;  // bytes of one group's channels at one position
  constexpr int MT = kGroupedMaxTaps;

  dev::prefetch_args(a);
  const int tid = threadIdx.x;
  const int G = a.G;
  const int g = tid % G;
  const int slot = tid / G;
  const int slots = kGroupedThreads / G;

  const int t = blockIdx.x;
  const SubDesc s = a.sub[dev::find_class(a, t)];
  const int npix_img = s.pos_h * s.pos_w;
  const int npos = a.N * npix_img;
  const int p0 = (t - s.tile_begin) * slots * a.iters;

  const auto rdy = dev::rsrc(a.dy, a.dy_bytes);
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);

  const int ntaps = s.taps_h * s.taps_w;
  const int YX = a.Y * a.X;
  float wr[MT][CG][CG];  // [tap][k][c]
  int dho[MT], dwo[MT];
#pragma unroll
  for (int tp = 0; tp < MT; tp++) {
    const bool on = tp < ntaps;
    const int jh = on ? tp / s.taps_w : 0;
    const int jw = on ? tp - jh * s.taps_w : 0;
    const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
    dho[tp] = s.beta_h - a.delta_h * jh;
    dwo[tp] = s.beta_w - a.delta_w * jw;
#pragma unroll
    for (int k = 0; k < CG; k++) {
      const uint32_t off = on ? (uint32_t)(((g * CG + k) * YX + ty * a.X + tx) * CG) * ES : dev::kOOB;
      const Vec<VB> v = load_vec<VB>(rw, off);
#pragma unroll
      for (int c = 0; c < CG; c++) wr[tp][k][c] = elem<DT>(v.w, c);
    }
  }

  for (int it = 0; it < a.iters; it++) {
    const int p = p0 + slot + slots * it;
    if (p >= npos) break;
    const int n = p / npix_img;
    const int rr = p - n * npix_img;
    const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
    float acc[CG];
#pragma unroll
    for (int c = 0; c < CG; c++) acc[c] = 0.f;
#pragma unroll
    for (int tp = 0; tp < MT; tp++) {
      if (tp < ntaps) {
        const int ho = th + dho[tp], wo = tw + dwo[tp];
        const bool ok = ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
        const uint32_t off =
            ok ? (uint32_t)(((n * a.Ho + ho) * a.Wo + wo) * a.K + g * CG) * ES : dev::kOOB;
        const Vec<VB> v = load_vec<VB>(rdy, off);
#pragma unroll
        for (int k = 0; k < CG; k++) {
          const float d = elem<DT>(v.w, k);
#pragma unroll
          for (int c = 0; c < CG; c++) acc[c] = __builtin_fmaf(d, wr[tp][k][c], acc[c]);
        }
      }
    }
    const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
    Vec<VB> o;
    if constexpr (DT == 0) {
#pragma unroll
      for (int c = 0; c < CG; c++) o.w[c] = __float_as_uint(acc[c]);
    } else {
#pragma unroll
      for (int j = 0; j < Vec<VB>::W; j++) o.w[j] = 0;
#pragma unroll
      for (int c = 0; c < CG; c++) o.w[c >> 1] |= dev::bf16_rne(acc[c]) << (16 * (c & 1));
    }
    store_vec<VB>(rdx, (uint32_t)(((n * a.Hi + hi) * a.Wi + wi) * a.C + g * CG) * ES, o);
  }
}

template <int DT, int CG>
int launch_one(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_direct_kernel<DT, CG>, dim3((unsigned)grid),
                              dim3(kGroupedThreads), args, 0, (hipStream_t)stream);
}

template <int DT>
int launch_dt(const GemmArgs& a, int64_t grid, void* stream) {
  switch (a.Cg) {
    case 1: return launch_one<DT, 1>(a, grid, stream);
    case 2: return launch_one<DT, 2>(a, grid, stream);
    case 4: return launch_one<DT, 4>(a, grid, stream);
    case 8: return launch_one<DT, 8>(a, grid, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_grouped(const GemmArgs& a, int dtype, int64_t grid, void* stream) {
  return dtype == CBD_F32 ? launch_dt<0>(a, grid, stream) : launch_dt<1>(a, grid, stream);
}

}  // namespace cbd
