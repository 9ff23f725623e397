// cbd_geo.h -- geometry policies of the kernels that have shape-specialised
// instances (generic family, grouped 4x4x4-MFMA kernel).
#pragma once
#include "cbd_device.h"
#include "cbd_kernarg.h"
#include "../../include/cbd.h"

namespace cbd {

// Geometry of a launch: read from the kernel arguments (DynGeo, the
// descriptor-driven instances) or fixed at compile time (StatGeo<T>, the
// shape-specialised instances: T::k is one plan's whole geometry, so every
// index computation folds to constants and no argument is read before the
// first gather but the three tensor pointers, which arrive preloaded).
struct DynGeo {
  static constexpr bool kStatic = false;
  static constexpr int kRowPats = kRowPatsAll;  // row-load patterns compiled in (generic family)
#define CBD_DYN(f) \
  __device__ static int f(const GemmArgs& a) { return a.f; }
  CBD_DYN(N) CBD_DYN(C) CBD_DYN(K) CBD_DYN(Cg) CBD_DYN(Kg) CBD_DYN(Hi) CBD_DYN(Wi) CBD_DYN(Ho)
  CBD_DYN(Wo) CBD_DYN(Y) CBD_DYN(X) CBD_DYN(Sh) CBD_DYN(Sw) CBD_DYN(tstep_h) CBD_DYN(tstep_w)
  CBD_DYN(delta_h) CBD_DYN(delta_w) CBD_DYN(tiles_m) CBD_DYN(total_tiles) CBD_DYN(xcd_remap)
  CBD_DYN(ksplit) CBD_DYN(zblock) CBD_DYN(G) CBD_DYN(grp_rows) CBD_DYN(grp_cols)
#undef CBD_DYN
  __device__ static uint32_t dy_bytes(const GemmArgs& a) { return a.dy_bytes; }
  __device__ static uint32_t dx_bytes(const GemmArgs& a) { return a.dx_bytes; }
  __device__ static uint32_t w_bytes(const GemmArgs& a) { return a.w_bytes; }
  __device__ static SubDesc sub(const GemmArgs& a, int t) { return a.sub[dev::find_class(a, t)]; }
  __device__ static SubDesc sub_at(const GemmArgs& a, int i) { return a.sub[i]; }
  __device__ static int sub_index(const GemmArgs& a, int t) { return dev::find_class(a, t); }
  // The reciprocals of class ci's divisors (read together, right after the
  // class's descriptor), and x / d with one of them (a division for the
  // classes past the first kMagSub, whose reciprocals are not stored).
  struct Mags {
    uint32_t npix, posw, pergroup, tiles_m;
  };
  __device__ static Mags mags(const GemmArgs& a, int ci) {
    const int c = ci < kMagSub ? ci : 0;
    return Mags{a.mag_npix[c], a.mag_posw[c], a.mag_pergroup[c], a.mag_tiles_m};
  }
  __device__ static uint32_t div(int ci, uint32_t x, uint32_t d, uint32_t mag) {
    return ci < kMagSub ? dev::fdiv(x, d, mag) : x / d;
  }
};

// A descriptor-driven launch whose classes need only the row-load
// patterns in M (the others are not compiled into it, which keeps its
// register count to that of the paths it runs).
template <int M>
struct DynGeoRows : DynGeo {
  static constexpr int kRowPats = M;
};

template <class T>
struct StatGeo {
  static constexpr bool kStatic = true;
  // Row-load patterns of its classes.
  static constexpr int row_pats() {
    int m = 0;
    for (int q = 0; q < T::k.num_sub; q++)
      m |= 1 << row_pattern(T::k.sub[q].taps_h, T::k.sub[q].taps_w, T::k.sub[q].cls_w, T::k.X, T::k.tstep_w);
    return m & kRowPatsAll;
  }
  static constexpr int kRowPats = row_pats();
#define CBD_STAT(f) \
  __device__ static constexpr int f(const GemmArgs&) { return T::k.f; }
  CBD_STAT(N) CBD_STAT(C) CBD_STAT(K) CBD_STAT(Cg) CBD_STAT(Kg) CBD_STAT(Hi) CBD_STAT(Wi) CBD_STAT(Ho)
  CBD_STAT(Wo) CBD_STAT(Y) CBD_STAT(X) CBD_STAT(Sh) CBD_STAT(Sw) CBD_STAT(tstep_h) CBD_STAT(tstep_w)
  CBD_STAT(delta_h) CBD_STAT(delta_w) CBD_STAT(tiles_m) CBD_STAT(total_tiles) CBD_STAT(xcd_remap)
  CBD_STAT(zblock) CBD_STAT(G)
#undef CBD_STAT
  // (grouped row kernels: the tile fields hold rows and positions per workgroup)
  __device__ static constexpr int grp_rows(const GemmArgs&) { return T::k.bm; }
  __device__ static constexpr int grp_cols(const GemmArgs&) { return T::k.bn; }
  __device__ static constexpr int ksplit(const GemmArgs&) { return 0; }
  static constexpr uint32_t kEs = T::k.dtype == CBD_F32 ? 4 : 2;
  __device__ static constexpr uint32_t dy_bytes(const GemmArgs&) {
    return (uint32_t)(T::k.N * T::k.K * T::k.Ho * T::k.Wo) * kEs;
  }
  __device__ static constexpr uint32_t dx_bytes(const GemmArgs&) {
    return (uint32_t)(T::k.N * T::k.C * T::k.Hi * T::k.Wi) * kEs;
  }
  __device__ static constexpr uint32_t w_bytes(const GemmArgs&) {
    return (uint32_t)(T::k.K * T::k.Cg * T::k.Y * T::k.X) * kEs;
  }
  // The class of logical tile t: classes own ascending tile ranges.
  __device__ static SubDesc sub(const GemmArgs&, int t) {
    SubDesc r = T::k.sub[0];
#pragma unroll
    for (int q = 1; q < T::k.num_sub; q++)
      if (t >= T::k.sub[q].tile_begin) r = T::k.sub[q];
    return r;
  }
  __device__ static constexpr SubDesc sub_at(const GemmArgs&, int i) { return T::k.sub[i]; }
  __device__ static int sub_index(const GemmArgs&, int t) {
    int r = 0;
#pragma unroll
    for (int q = 1; q < T::k.num_sub; q++)
      if (t >= T::k.sub[q].tile_begin) r = q;
    return r;
  }
  // (divisors fixed per class: plain divisions, which the compiler folds
  // where the classes agree)
  struct Mags {
    uint32_t npix, posw, pergroup, tiles_m;
  };
  __device__ static constexpr Mags mags(const GemmArgs&, int) { return Mags{0, 0, 0, 0}; }
  __device__ static uint32_t div(int, uint32_t x, uint32_t d, uint32_t) { return x / d; }
};

}  // namespace cbd
