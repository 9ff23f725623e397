// cbd_plan.cpp -- host planner: validates a problem, splits it into
// stride-residue sub-GEMMs and zero regions, picks a kernel family and packs
// the launch arguments.  Pure host code; needs no GPU.
//
// Per axis (stride S, dilation D, pad P, taps F, input extent L), a tap f
// feeds dX position h iff h + P - f*D is a non-negative multiple of S whose
// quotient is a valid output index (the adjoint of the forward window
// h = o*S + f*D - P).  With g = gcd(S, D), T = S/g, delta = D/g:
//   * the taps reaching one position form one residue class f = i (mod T),
//     i in [0, T); class i holds ceil((F - i)/T) taps (none if i >= F);
//   * class i serves the dX phase phi_i = (D*i - P) mod S, positions
//     h = phi_i + S*t, t < ceil((L - phi_i)/S);
//   * tap i + T*j of that class reads output row t + beta_i - delta*j with
//     beta_i = (phi_i + P - D*i)/S (an exact integer);
//   * phases hit by no class with taps are never reached: written as zero.
// Every (class_h, class_w) pair with taps and positions is one GEMM (per
// group): M = C/G, N = N*pos_h*pos_w, K = (K/G)*taps_h*taps_w.  This is the
// stride-residue decomposition behind the multi-kernel backward data of
// rocMLIR PR #246 "Backward data" and the v4r1 backward-data strategy named
// in MIOpen PR #272; neither page derives it, the derivation above follows
// from the forward window alone.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "cbd_internal.h"
#include "generic_shapes.h"

namespace {

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ceil(2^32 / d) for the kernels' multiply-high division (0 for d = 1,
// which the kernels take as the identity).
uint32_t magic32(int64_t d) { return d <= 1 ? 0u : (uint32_t)((uint64_t(1) << 32) / (uint64_t)d + ((uint64_t(1) << 32) % (uint64_t)d != 0)); }
int64_t pos_mod(int64_t a, int64_t m) {
  int64_t r = a % m;
  return r < 0 ? r + m : r;
}

struct AxisClass {
  int64_t cls, taps, phase, beta, pos;
};

struct Axis {
  int64_t T, delta;
  std::vector<AxisClass> classes;
};

Axis split_axis(int64_t L, int64_t F, int64_t S, int64_t D, int64_t P) {
  Axis ax;
  const int64_t g = gcd64(S, D);
  ax.T = S / g;
  ax.delta = D / g;
  for (int64_t i = 0; i < ax.T; i++) {
    AxisClass c;
    c.cls = i;
    c.taps = i < F ? ceil_div(F - i, ax.T) : 0;
    c.phase = pos_mod(D * i - P, S);
    c.beta = (c.phase + P - D * i) / S;
    c.pos = c.phase < L ? ceil_div(L - c.phase, S) : 0;
    ax.classes.push_back(c);
  }
  return ax;
}

int64_t out_extent(int64_t L, int64_t P, int64_t D, int64_t F, int64_t S) {
  const int64_t room = L + 2 * P - D * (F - 1) - 1;
  return room < 0 ? 0 : room / S + 1;
}

cbd_status fail(cbd_status st, const std::string& msg) {
  cbd::set_error(msg);
  return st;
}

bool fast_ok(const cbd_problem& p, int64_t Cg, int64_t Kg, int64_t max_taps) {
  return p.layout == CBD_LAYOUT_NHWC && p.dtype == CBD_BF16 && Kg % cbd::kFastBK == 0 &&
         Kg <= (int64_t)cbd::kFastBK * cbd::kFastMaxKTiles && Cg % 8 == 0 &&
         max_taps <= cbd::kFastMaxTaps;
}

// The 16x16x16-MFMA grouped kernel: bf16 NHWC, 8, 16 or 32 channels per
// group, groups in blocks whose channels make a 256-byte slice, taps one dY
// row apart.
bool grouped_wide_ok(const cbd_problem& p, int64_t Cg, int64_t Kg, int64_t max_taps, int64_t delta_h) {
  return p.layout == CBD_LAYOUT_NHWC && p.dtype == CBD_BF16 && Cg == Kg &&
         (Cg == 8 || Cg == 16 || Cg == 32) && p.g % (256 / (2 * Cg)) == 0 && delta_h == 1 &&
         max_taps <= cbd::kGroupedMaxTaps;
}

bool grouped_ok(const cbd_problem& p, int64_t Cg, int64_t Kg, int64_t max_taps) {
  return p.layout == CBD_LAYOUT_NHWC && Cg == Kg && (Cg == 1 || Cg == 2 || Cg == 4 || Cg == 8) &&
         p.g <= cbd::kGroupedThreads && cbd::kGroupedThreads % p.g == 0 &&
         max_taps <= cbd::kGroupedMaxTaps;
}

// Row-block family geometry for rb dX rows per workgroup (see
// kern_nchw_rows.hip); lds = 0 when the staged tiles cannot fit.
cbd::RowsGeom rows_geom(const cbd_problem& p, const std::vector<cbd_subgemm_t>& subs, int64_t Cg,
                        int64_t Kg, int64_t rb, int64_t es) {
  cbd::RowsGeom r;
  std::memset(&r, 0, sizeof(r));
  int64_t wo_lo = INT64_MAX, wo_hi = INT64_MIN;
  for (const auto& s : subs) {
    wo_lo = std::min<int64_t>(wo_lo, s.beta_w - (int64_t)s.delta_w * (s.taps_w - 1));
    wo_hi = std::max<int64_t>(wo_hi, 16 * ceil_div(s.pos_w, 16) + s.beta_w);
  }
  // Staged dY rows: the widest span over every residue of a block's first
  // row modulo the stride (t ranges unclamped, so a superset of any block's).
  int64_t nr = 1;
  for (int64_t b = 0; b < p.stride_h; b++) {
    const int64_t h0 = b * rb;
    int64_t lo = INT64_MAX, hi = INT64_MIN;
    for (const auto& s : subs) {
      const int64_t num_lo = h0 - s.phase_h, num_hi = h0 + rb - 1 - s.phase_h;
      const int64_t t_lo = num_lo >= 0 ? ceil_div(num_lo, p.stride_h) : -((-num_lo) / p.stride_h);
      const int64_t t_hi = num_hi >= 0 ? num_hi / p.stride_h : -ceil_div(-num_hi, p.stride_h);
      if (t_lo > t_hi) continue;
      lo = std::min<int64_t>(lo, t_lo + s.beta_h - (int64_t)s.delta_h * (s.taps_h - 1));
      hi = std::max<int64_t>(hi, t_hi + s.beta_h);
    }
    if (lo <= hi) nr = std::max<int64_t>(nr, hi - lo + 1);
  }
  const int64_t rw = wo_hi - wo_lo;
  const int64_t kg4 = 16 * ceil_div(Kg, 16);  // k steps of 4 in whole groups of four
  auto pad16 = [](int64_t v) { return v + ((16 - v % 64) % 64 + 64) % 64; };  // -> 16 (mod 64)
  const int64_t ks = pad16(nr * rw);
  const int64_t nch = ceil_div(nr * rw, 64);
  const int64_t yx = p.y * p.x;
  const int64_t ksw = pad16(16 * yx);
  const bool wvec = es == 4 && Cg % 16 == 0 && kg4 * 4 * yx <= int64_t(cbd::kRowsMaxWLoads) * cbd::kRowsThreads;
  const int64_t cst = pad16(rb * p.wi);
  const int64_t lds = 4 * (kg4 * ks + kg4 * ksw + 16 * cst);
  const int64_t rowb = p.wi * es;
  const int64_t vb = rowb % 16 == 0 ? 16 : rowb % 8 == 0 ? 8 : rowb % 4 == 0 ? 4 : 2;
  const int64_t chunks = p.wi / (vb / es);
  // Each wave stages kg4/4 dY planes of nch chunks from registers.
  if (nch > cbd::kRowsMaxChunks || (kg4 / 4) * cbd::kRowsMaxChunks > cbd::kRowsMaxDyLoads) return r;
  if (lds > cbd::kLdsPerCu || 16 * rb * chunks >= (int64_t(1) << 31)) return r;
  r.rb = (int32_t)rb;
  r.row_blocks = (int32_t)ceil_div(p.hi, rb);
  r.c_blocks = (int32_t)ceil_div(Cg, 16);
  r.nr = (int32_t)nr;
  r.rw = (int32_t)rw;
  r.wo_lo = (int32_t)wo_lo;
  r.kg4 = (int32_t)kg4;
  r.ks = (int32_t)ks;
  r.nch = (int32_t)nch;
  r.ksw = (int32_t)ksw;
  r.wvec = wvec ? 1 : 0;
  r.cst = (int32_t)cst;
  r.w_off = (int32_t)(kg4 * ks);
  r.st_off = (int32_t)(kg4 * ks + kg4 * ksw);
  r.vb = (int32_t)vb;
  r.lds_bytes = (int32_t)lds;
  r.mag_plane = magic32(nr * rw);
  r.mag_rw = magic32(rw);
  r.mag_perk = magic32(16 * p.y * p.x);
  r.mag_yx = magic32(p.y * p.x);
  r.mag_perc = magic32(rb * chunks);
  r.mag_chunks = magic32(chunks);
  return r;
}

// Rows per workgroup for the row-block family, as B balanced blocks of
// ceil(Hi / B) rows: the fewest blocks that give 256 workgroups (one per CU);
// when no B does, the most blocks whose first block still holds four
// 16-position units (one per wave).  lds = 0 if no block size fits LDS.
cbd::RowsGeom rows_choose(const cbd_problem& p, const std::vector<cbd_subgemm_t>& subs, int64_t Cg, int64_t Kg,
                          int64_t es) {
  cbd::RowsGeom best, fallback;
  std::memset(&best, 0, sizeof(best));
  std::memset(&fallback, 0, sizeof(fallback));
  if (subs.empty()) return best;
  const int64_t cb = ceil_div(Cg, 16);
  const int64_t bmax = std::min<int64_t>(p.hi, 4096);
  for (int64_t nb = 1; nb <= bmax; nb++) {
    const int64_t rb = ceil_div(p.hi, nb);
    if (ceil_div(p.hi, rb) != nb) continue;  // the same blocks as a smaller count
    const cbd::RowsGeom g = rows_geom(p, subs, Cg, Kg, rb, es);
    if (g.lds_bytes == 0) continue;
    if (p.n * p.g * cb * nb >= 256) return g;
    int64_t units = 0;
    for (const auto& s : subs)
      for (int64_t h = s.phase_h; h < rb; h += p.stride_h)
        if ((h - s.phase_h) / p.stride_h < s.pos_h) units += ceil_div(s.pos_w, 16);
    if (units >= 4) best = g;
    if (fallback.lds_bytes == 0) fallback = g;
  }
  return best.lds_bytes ? best : fallback;
}

// CBD_LOG set to anything but "" or "0": every plan built is described on
// stderr (problem, kernel choice, launch shape, sub-GEMMs, zero regions) --
// which kernel runs a problem, and why it runs at the speed it does, without
// a debugger.
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("CBD_LOG");
    return v && *v && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

const char* kernel_name(int32_t k, int64_t variant) {
  if (k == CBD_KERNEL_NHWC_BF16) return "nhwc_bf16 (256x256 tiles)";
  if (k == CBD_KERNEL_GENERIC) return "generic";
  if (k == CBD_KERNEL_NCHW_ROWS) return "nchw_rows (row blocks)";
  static const char* const grouped[] = {"grouped/direct", "grouped/rows", "grouped/pipelined-dot",
                                        "grouped/pipelined-4x4x4-mfma", "grouped/pipelined-16x16x16-mfma",
                                        "grouped/pipelined-4x4x4-mfma, phases merged"};
  return variant >= 0 && variant < 6 ? grouped[variant] : "grouped";
}

void log_plan(const cbd_plan_s& pl) {
  const cbd_problem& p = pl.prob;
  const cbd_plan_info_t& i = pl.info;
  std::fprintf(stderr,
               "[cbd] plan: N=%lld G=%lld C=%lld K=%lld Hi=%lld Wi=%lld Y=%lld X=%lld stride=(%d,%d) "
               "pad=(%d,%d) dil=(%d,%d) %s %s -> Ho=%lld Wo=%lld\n",
               (long long)p.n, (long long)p.g, (long long)p.c, (long long)p.k, (long long)p.hi,
               (long long)p.wi, (long long)p.y, (long long)p.x, p.stride_h, p.stride_w, p.pad_h, p.pad_w,
               p.dil_h, p.dil_w, p.layout == CBD_LAYOUT_NHWC ? "NHWC/KYXC" : "NCHW/KCYX",
               p.dtype == CBD_BF16 ? "bf16" : "f32", (long long)i.ho, (long long)i.wo);
  std::fprintf(stderr,
               "[cbd]   kernel %s: tile %dx%dx%d, %d threads, grid %lld (+%lld zero-fill), %d launch(es), "
               "static level %lld, ksplit %lld, rows/wg %lld, cols/wg %lld, LDS %lld B, workspace %lld B, "
               "align dy/w/dx %d/%d/%d\n",
               kernel_name(i.kernel, i.variant), i.tile_m, i.tile_n, i.tile_k, i.threads_main,
               (long long)i.grid_main, (long long)i.grid_zero, i.launches, (long long)i.static_shape,
               (long long)i.ksplit, (long long)i.rows_per_wg, (long long)i.cols_per_wg,
               (long long)i.lds_dynamic, (long long)i.workspace_bytes, i.align_dy, i.align_w, i.align_dx);
  std::fprintf(stderr, "[cbd]   useful %.6g GFLOP, executed %.6g GMAC, %lld zeroed elements\n",
               (double)i.useful_flops * 1e-9, (double)i.executed_macs * 1e-9, (long long)i.zero_elems);
  for (const cbd_subgemm_t& s : pl.subs)
    std::fprintf(stderr,
                 "[cbd]   sub-GEMM %d: class (%d,%d) phase (%d,%d) beta (%d,%d) taps %dx%d positions "
                 "%lldx%lld  M=%lld N=%lld K=%lld  tiles [%lld, %lld)\n",
                 s.id, s.class_h, s.class_w, s.phase_h, s.phase_w, s.beta_h, s.beta_w, s.taps_h, s.taps_w,
                 (long long)s.pos_h, (long long)s.pos_w, (long long)s.m, (long long)s.n, (long long)s.k,
                 (long long)s.tile_begin, (long long)(s.tile_begin + s.tiles));
  for (const cbd_zero_region_t& z : pl.zeros)
    std::fprintf(stderr, "[cbd]   zero region: phase (%d,%d), %lldx%lld positions\n", z.phase_h, z.phase_w,
                 (long long)z.pos_h, (long long)z.pos_w);
}

// Whole-block epilogue writing pairs of dX elements (value, 0): NCHW with
// stride 2 along W and an even width.
bool zblock_pairs(const cbd_problem& p) {
  return p.layout == CBD_LAYOUT_NCHW && p.stride_w == 2 && p.wi % 2 == 0;
}

// Every field of a compiled generic-family shape equals the plan's.
bool generic_shape_matches(const cbd::ShapeKey& k, const cbd::GemmArgs& a, const cbd_problem& p, int64_t threads) {
  if (k.layout != p.layout || k.dtype != p.dtype || k.bm != a.tile_m || k.bn != a.tile_n ||
      k.nw * 64 != threads)
    return false;
  if (k.N != a.N || k.G != a.G || k.C != a.C || k.K != a.K || k.Cg != a.Cg || k.Kg != a.Kg || k.Hi != a.Hi ||
      k.Wi != a.Wi || k.Ho != a.Ho || k.Wo != a.Wo || k.Y != a.Y || k.X != a.X || k.Sh != a.Sh || k.Sw != a.Sw)
    return false;
  if (k.tstep_h != a.tstep_h || k.tstep_w != a.tstep_w || k.delta_h != a.delta_h || k.delta_w != a.delta_w ||
      k.tiles_m != a.tiles_m || k.total_tiles != a.total_tiles || k.xcd_remap != a.xcd_remap ||
      k.num_sub != a.num_sub || k.zblock != a.zblock || a.num_sub > cbd::kShapeMaxSub)
    return false;
  for (int q = 0; q < a.num_sub; q++) {
    const cbd::SubDesc &x = k.sub[q], &y = a.sub[q];
    if (x.phase_h != y.phase_h || x.phase_w != y.phase_w || x.beta_h != y.beta_h || x.beta_w != y.beta_w ||
        x.taps_h != y.taps_h || x.taps_w != y.taps_w || x.cls_h != y.cls_h || x.cls_w != y.cls_w ||
        x.pos_h != y.pos_h || x.pos_w != y.pos_w || x.tile_begin != y.tile_begin)
      return false;
  }
  return true;
}

// Every field of a compiled grouped-kernel shape equals the plan's (the tile
// fields hold rows and positions per workgroup).
bool grouped_shape_matches(const cbd::ShapeKey& k, const cbd::GemmArgs& a, const cbd_problem& p, int64_t threads) {
  if (k.layout != p.layout || k.dtype != p.dtype || k.bm != a.grp_rows || k.bn != a.grp_cols ||
      k.nw * 64 != threads)
    return false;
  if (k.N != a.N || k.G != a.G || k.C != a.C || k.K != a.K || k.Cg != a.Cg || k.Kg != a.Kg || k.Hi != a.Hi ||
      k.Wi != a.Wi || k.Ho != a.Ho || k.Wo != a.Wo || k.Y != a.Y || k.X != a.X || k.Sh != a.Sh || k.Sw != a.Sw)
    return false;
  if (k.tstep_h != a.tstep_h || k.tstep_w != a.tstep_w || k.delta_h != a.delta_h || k.delta_w != a.delta_w ||
      k.total_tiles != a.total_tiles || k.num_sub != a.num_sub || a.num_sub > cbd::kShapeMaxSub)
    return false;
  for (int q = 0; q < a.num_sub; q++) {
    const cbd::SubDesc &x = k.sub[q], &y = a.sub[q];
    if (x.phase_h != y.phase_h || x.phase_w != y.phase_w || x.beta_h != y.beta_h || x.beta_w != y.beta_w ||
        x.taps_h != y.taps_h || x.taps_w != y.taps_w || x.cls_h != y.cls_h || x.cls_w != y.cls_w ||
        x.pos_h != y.pos_h || x.pos_w != y.pos_w || x.tile_begin != y.tile_begin)
      return false;
  }
  return true;
}

// Shortest K loop of any class, in k tiles of the family (split-K gives
// each split at least one).
int64_t min_class_ktiles(const std::vector<cbd_subgemm_t>& subs, int32_t kernel, int64_t Kg, int64_t bk) {
  if (kernel != CBD_KERNEL_NHWC_BF16 && (kernel != CBD_KERNEL_GENERIC || bk <= 0)) return 0;
  int64_t m = INT64_MAX;
  for (const auto& s : subs)
    m = std::min<int64_t>(m, kernel == CBD_KERNEL_NHWC_BF16 ? s.k / cbd::kFastBK
                                                              : int64_t(s.taps_h) * s.taps_w * ceil_div(Kg, bk));
  return subs.empty() ? 0 : m;
}

// Workgroups per tile of the planner's split-K configuration (1: none).
// Large-tile kernel only, and only below the measured crossover (64 tiles:
// a quarter of the CUs); then as many splits as keep the grid within 128
// workgroups, a power of two, and every split at least one k tile per wave
// (measured on the headline problem's batch shards: N = 1 best at 8
// splits, N = 2 at 4, N >= 4 unsplit).  The generic family already spreads
// K over the waves of a workgroup: splitting it across workgroups measured
// slower on every problem tried (the finalising launch and the partial
// tiles cost more than the shorter K loop saves), so it splits only when
// asked.
int64_t auto_ksplit(int32_t kernel, int64_t tiles, int64_t kt_min) {
  if (kernel != CBD_KERNEL_NHWC_BF16 || tiles <= 0 || tiles >= 64) return 1;
  const int64_t waves = 4;
  int64_t s = 1;
  while (tiles * s * 2 <= 128 && kt_min / (s * 2) >= waves) s *= 2;
  return s;
}

}  // namespace

extern "C" cbd_status cbd_plan_ex(const cbd_problem* problem, const cbd_plan_options* options,
                                  cbd_plan_t** out_plan) {
  if (!problem || !out_plan) return fail(CBD_ERR_INVALID_ARG, "NULL problem or out_plan");
  *out_plan = nullptr;
  const cbd_problem p = *problem;
  int32_t force = CBD_KERNEL_AUTO;
  bool no_split = false;
  int32_t rows_opt = 0;
  bool grouped_dot = false;
  int32_t cols_opt = 0;
  int32_t ksplit_opt = 0;
  bool per_class = false;
  int32_t static_mode = 0;
  int32_t merge_opt = 0;
  if (options) {
    for (int i = 0; i < 3; i++)
      if (options->reserved[i]) return fail(CBD_ERR_INVALID_ARG, "options.reserved must be zero");
    if (options->merge_phases < -1 || options->merge_phases > 1)
      return fail(CBD_ERR_INVALID_ARG, "options.merge_phases must be -1, 0 or 1");
    merge_opt = options->merge_phases;
    if (options->static_shape < -1 || options->static_shape > 1)
      return fail(CBD_ERR_INVALID_ARG, "options.static_shape must be -1, 0 or 1");
    static_mode = options->static_shape;
    if (options->per_class != 0 && options->per_class != 1)
      return fail(CBD_ERR_INVALID_ARG, "options.per_class must be 0 or 1");
    per_class = options->per_class == 1;
    if (options->ksplit < 0 || options->ksplit > 64)
      return fail(CBD_ERR_INVALID_ARG, "options.ksplit must be 0..64");
    ksplit_opt = options->ksplit;
    if (options->cols_per_wg < 0 || options->cols_per_wg > (1 << 20))
      return fail(CBD_ERR_INVALID_ARG, "options.cols_per_wg must be 0 or a position count");
    cols_opt = options->cols_per_wg;
    if (options->grouped_dot != 0 && options->grouped_dot != 1)
      return fail(CBD_ERR_INVALID_ARG, "options.grouped_dot must be 0 or 1");
    grouped_dot = options->grouped_dot == 1;
    if (options->rows_per_wg < -1 || options->rows_per_wg > (1 << 20))
      return fail(CBD_ERR_INVALID_ARG, "options.rows_per_wg must be -1, 0 or a row count");
    rows_opt = options->rows_per_wg;
    if (options->no_split != 0 && options->no_split != 1)
      return fail(CBD_ERR_INVALID_ARG, "options.no_split must be 0 or 1");
    no_split = options->no_split == 1;
    force = options->force_kernel;
    if (force < CBD_KERNEL_AUTO || force > CBD_KERNEL_NCHW_ROWS)
      return fail(CBD_ERR_INVALID_ARG, "unknown force_kernel");
  }
  if (p.n < 1 || p.g < 1 || p.c < 1 || p.k < 1 || p.hi < 1 || p.wi < 1 || p.y < 1 || p.x < 1)
    return fail(CBD_ERR_INVALID_ARG, "sizes must be >= 1");
  if (p.stride_h < 1 || p.stride_w < 1 || p.dil_h < 1 || p.dil_w < 1)
    return fail(CBD_ERR_INVALID_ARG, "stride and dilation must be >= 1");
  if (p.pad_h < 0 || p.pad_w < 0) return fail(CBD_ERR_INVALID_ARG, "padding must be >= 0");
  if (p.c % p.g || p.k % p.g) return fail(CBD_ERR_INVALID_ARG, "groups must divide C and K");
  if (p.layout != CBD_LAYOUT_NCHW && p.layout != CBD_LAYOUT_NHWC)
    return fail(CBD_ERR_INVALID_ARG, "unknown layout");
  if (p.dtype != CBD_F32 && p.dtype != CBD_BF16) return fail(CBD_ERR_INVALID_ARG, "unknown dtype");
  // Keep every intermediate comfortably inside 64-bit arithmetic before the
  // size checks below.
  const int64_t kDimMax = int64_t(1) << 31;
  if (p.n >= kDimMax || p.c >= kDimMax || p.k >= kDimMax || p.hi >= kDimMax ||
      p.wi >= kDimMax || p.y >= kDimMax || p.x >= kDimMax)
    return fail(CBD_ERR_UNSUPPORTED, "dimension beyond 2^31");
  if (p.pad_h > (1 << 20) || p.pad_w > (1 << 20) || p.dil_h > 64 || p.dil_w > 64 ||
      p.stride_h > 64 || p.stride_w > 64)
    return fail(CBD_ERR_UNSUPPORTED, "pad > 2^20, dilation > 64 or stride > 64");
  if ((int64_t)p.stride_h * p.stride_w > cbd::kMaxSub)
    return fail(CBD_ERR_UNSUPPORTED, "stride_h * stride_w > 64");

  const int64_t Ho = out_extent(p.hi, p.pad_h, p.dil_h, p.y, p.stride_h);
  const int64_t Wo = out_extent(p.wi, p.pad_w, p.dil_w, p.x, p.stride_w);
  if (Ho < 1 || Wo < 1) return fail(CBD_ERR_INVALID_ARG, "filter larger than padded input");
  const int64_t Cg = p.c / p.g, Kg = p.k / p.g;
  const int64_t es = p.dtype == CBD_F32 ? 4 : 2;
  const double lim = 2147483647.0;  // tensors must stay below 2^31 bytes
  if ((double)p.n * p.c * p.hi * p.wi * es > lim || (double)p.n * p.k * Ho * Wo * es > lim ||
      (double)p.k * Cg * p.y * p.x * es > lim)
    return fail(CBD_ERR_UNSUPPORTED, "a tensor reaches 2^31 bytes (32-bit buffer addressing)");

  const Axis ah = split_axis(p.hi, p.y, p.stride_h, p.dil_h, p.pad_h);
  const Axis aw = split_axis(p.wi, p.x, p.stride_w, p.dil_w, p.pad_w);

  cbd_plan_s* pl = new (std::nothrow) cbd_plan_s();
  if (!pl) return fail(CBD_ERR_NO_MEMORY, "plan allocation failed");
  pl->prob = p;
  std::memset(&pl->info, 0, sizeof(pl->info));
  std::memset(&pl->gemm, 0, sizeof(pl->gemm));
  std::memset(&pl->zero, 0, sizeof(pl->zero));

  // Sub-GEMMs and reached phases.
  std::vector<cbd_subgemm_t> subs;
  int64_t max_taps = 0;
  std::vector<char> reached((size_t)(p.stride_h * p.stride_w), 0);
  if (no_split) {
    // Zero-insertion form: one "class" over all dX positions with all taps;
    // the kernels test each (position, tap) term for stride divisibility.
    cbd_subgemm_t s;
    std::memset(&s, 0, sizeof(s));
    s.taps_h = (int32_t)p.y;
    s.taps_w = (int32_t)p.x;
    s.tstep_h = s.tstep_w = 1;
    s.delta_h = (int32_t)p.dil_h;
    s.delta_w = (int32_t)p.dil_w;
    s.pos_h = p.hi;
    s.pos_w = p.wi;
    s.m = Cg;
    s.n = p.n * p.hi * p.wi;
    s.k = Kg * p.y * p.x;
    subs.push_back(s);
    std::fill(reached.begin(), reached.end(), 1);
    max_taps = p.y * p.x;
  }
  for (const AxisClass& ch : (no_split ? std::vector<AxisClass>() : ah.classes)) {
    for (const AxisClass& cw : aw.classes) {
      if (ch.taps * cw.taps == 0 || ch.pos * cw.pos == 0) continue;
      cbd_subgemm_t s;
      std::memset(&s, 0, sizeof(s));
      s.class_h = (int32_t)ch.cls;
      s.class_w = (int32_t)cw.cls;
      s.phase_h = (int32_t)ch.phase;
      s.phase_w = (int32_t)cw.phase;
      s.beta_h = (int32_t)ch.beta;
      s.beta_w = (int32_t)cw.beta;
      s.taps_h = (int32_t)ch.taps;
      s.taps_w = (int32_t)cw.taps;
      s.tstep_h = (int32_t)ah.T;
      s.tstep_w = (int32_t)aw.T;
      s.delta_h = (int32_t)ah.delta;
      s.delta_w = (int32_t)aw.delta;
      s.pos_h = ch.pos;
      s.pos_w = cw.pos;
      s.m = Cg;
      s.n = p.n * ch.pos * cw.pos;
      s.k = Kg * ch.taps * cw.taps;
      subs.push_back(s);
      reached[(size_t)(ch.phase * p.stride_w + cw.phase)] = 1;
      max_taps = std::max(max_taps, ch.taps * cw.taps);
    }
  }
  // Longest-processing-time order: classes with the largest K launch first.
  std::stable_sort(subs.begin(), subs.end(),
                   [](const cbd_subgemm_t& x, const cbd_subgemm_t& y) { return x.k > y.k; });

  // Kernel family.  The row-block family is chosen only when forced: on
  // every NCHW problem measured it ran slower than the implicit GEMM (its
  // staging, one workgroup per row block and 16 channels, is latency bound).
  int kernel;
  const bool rows_able = p.layout == CBD_LAYOUT_NCHW && !no_split && !per_class && ksplit_opt < 2;
  cbd::RowsGeom rgeom;
  std::memset(&rgeom, 0, sizeof(rgeom));
  if (rows_able && force == CBD_KERNEL_NCHW_ROWS) rgeom = rows_choose(p, subs, Cg, Kg, es);
  if (force == CBD_KERNEL_AUTO) {
    if (fast_ok(p, Cg, Kg, max_taps) && Cg >= 128)
      kernel = CBD_KERNEL_NHWC_BF16;
    else if (!no_split && (grouped_ok(p, Cg, Kg, max_taps) ||
                           grouped_wide_ok(p, Cg, Kg, max_taps, ah.delta)))
      kernel = CBD_KERNEL_GROUPED;
    else
      kernel = CBD_KERNEL_GENERIC;
  } else {
    kernel = force;
    if (kernel == CBD_KERNEL_NCHW_ROWS && rgeom.lds_bytes == 0) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "row-block kernel needs NCHW, the residue split without per_class "
                                       "or ksplit, at least one sub-GEMM, and its staged tiles within LDS");
    }
    if (kernel == CBD_KERNEL_NHWC_BF16 && !fast_ok(p, Cg, Kg, max_taps)) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "NHWC bf16 kernel needs NHWC, bf16, K/G % 64 == 0, C/G % 8 == 0, <= 16 taps per class");
    }
    if (kernel == CBD_KERNEL_GROUPED && no_split) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "the grouped kernels have no zero-insertion (no_split) mode");
    }
    if (kernel == CBD_KERNEL_GROUPED && !grouped_ok(p, Cg, Kg, max_taps) &&
        !grouped_wide_ok(p, Cg, Kg, max_taps, ah.delta)) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "grouped kernels need NHWC, C/G == K/G in {1,2,4,8} with G | 256, "
                                       "or bf16 with C/G in {16,32}, taps one dY row apart; <= 9 taps per class");
    }
  }

  int64_t bm = 0, bn = 0, bk = 0, threads = 0;
  if (kernel == CBD_KERNEL_GENERIC) {
    // 32-wide tiles where 64 would be mostly padding (C/G <= 32), and 32x32
    // tiles unless 64-wide ones still give every CU four workgroups: a
    // workgroup's time here is its chain of gathers along K, so more, shorter
    // chains finish sooner (measured: 64 channels, N = 32, 28x28, stride 2,
    // 3x3 and 1x1 filters, 392 and 98 tiles of 64x64: 32x32 tiles 9 % and
    // 6 % faster; 8-wide k tiles on 32x32 tiles another 4-10 %).
    bm = Cg <= 32 ? 32 : cbd::kGenericBM;
    threads = cbd::kGenericThreads;
    int64_t grid64 = 0;
    for (const auto& s : subs) grid64 += p.g * ceil_div(Cg, bm) * ceil_div(s.n, cbd::kGenericBN);
    if (grid64 < 4 * 256) {
      bm = 32;
      bn = 32;
    } else {
      bn = cbd::kGenericBN;
    }
    // At most 16 channels per group: 16-row tiles (a 32-row tile would be
    // half padding), 16 wide too when the grid is small (measured: 16
    // channels, N = 2, 14x14, 3x3: 16x16 tiles 22 % faster than 32x32; for
    // 32 channels, 32x16 tiles were slower than 32x32).
    if (Cg <= 16 && bm == 32 && bn == 32) {
      bm = 16;
      int64_t grid1632 = 0;
      for (const auto& s : subs) grid1632 += p.g * ceil_div(Cg, 16) * ceil_div(s.n, 32);
      if (grid1632 < 512) bn = 16;
    }
    bk = cbd::generic_bk((int)bm, (int)bn);
    // Long K on a small grid of 32x32 tiles: eight waves per workgroup share
    // the K loop (a wave's gather chain halves; measured: 32 channels, 3x3,
    // N = 32, 14-16 pixels, 36 k tiles on 196-256 workgroups, 6 % faster;
    // with short K or many workgroups eight waves were slower).  f32 KCYX
    // classes with a row-load pattern run k tiles of 4 k rows (8 for one or
    // two taps) over all their taps: 8 such tiles for those 32-channel
    // problems, where four waves are 8 % faster than eight.
    if (bm == 32 && bn == 32) {
      int64_t grid32 = 0, kt = 0;
      const bool rows = p.dtype == CBD_F32 && p.layout == CBD_LAYOUT_NCHW && !no_split;
      for (const auto& s : subs) {
        grid32 += p.g * ceil_div(Cg, 32) * ceil_div(s.n, 32);
        const int taps = s.taps_h * s.taps_w;
        const bool rl = rows && cbd::row_pattern(s.taps_h, s.taps_w, s.class_w, (int)p.x, s.tstep_w) != 0;
        kt = std::max<int64_t>(kt, rl ? ceil_div(Kg, taps <= 2 ? 8 : 4) : int64_t(taps) * ceil_div(Kg, bk));
      }
      if (grid32 < 512 && kt >= 32) threads = 8 * 64;
      // Every class reading W by rows with one to four taps (stride 2, for
      // one): two waves per workgroup, each with two k tiles in flight
      // (measured, descriptor-driven: 64 channels, 3x3, stride 2, N = 8-64,
      // 784-3136 tiles, 5-14 % faster than four waves; shape-specialised,
      // the workload problem 10.6 against 10.8 us; with nine-tap classes
      // two waves were 19-22 % slower).
      bool rows_s2 = rows && ksplit_opt < 2 && !subs.empty();
      for (const auto& s : subs) {
        const int rp = cbd::row_pattern(s.taps_h, s.taps_w, s.class_w, (int)p.x, s.tstep_w);
        rows_s2 = rows_s2 && rp >= 1 && rp <= 4;
      }
      if (rows_s2 && threads == 4 * 64) threads = 2 * 64;
    }
  } else if (kernel == CBD_KERNEL_NHWC_BF16) {
    bm = cbd::kFastBM; bn = cbd::kFastBN; bk = cbd::kFastBK; threads = cbd::kFastThreads;
  } else if (kernel == CBD_KERNEL_NCHW_ROWS) {
    bm = 16; bn = 16; bk = 4; threads = cbd::kRowsThreads;
  } else {
    threads = cbd::kGroupedThreads;
  }

  // Grouped kernels (C/G <= 4 and 16-byte pixels first):
  //  * pipelined kernels (taps one dY row apart): a workgroup walks R output
  //    rows of one class and image with a ring of taps_h + 1 dY rows (each
  //    padded to 4 KiB) in LDS; R is sized so that the grid is about one
  //    round of resident workgroups.  bf16 with 4 channels per group and
  //    32 or 64 groups runs the products on 4x4x4 MFMA (its slots also hold
  //    3 columns past the row, read by a partial quad of positions), the
  //    rest on dot-product instructions;
  //  * row kernel: one workgroup per output row of a class, the row's dY
  //    rows staged in LDS;
  //  * direct kernel otherwise: positions per thread so that the grid is
  //    ~2048 workgroups.
  int64_t iters = 1;
  int64_t slots = 0;
  int64_t grp_lds = 0;
  int64_t grp_rows = 0, grp_cols = 0;
  bool grp_mfma = false, grp_wide = false, grp_merged = false;
  int64_t merged_tiles = 0;
  if (kernel == CBD_KERNEL_GROUPED && (Cg == 16 || Cg == 32) && rows_opt < 0) {
    delete pl;
    return fail(CBD_ERR_UNSUPPORTED, "16 or 32 channels per group run only on the pipelined kernel "
                                     "(rows_per_wg = -1)");
  }
  if (kernel == CBD_KERNEL_GROUPED && !subs.empty() && rows_opt >= 0 &&
      grouped_wide_ok(p, Cg, Kg, max_taps, ah.delta)) {
    // 16x16x16-MFMA kernel: workgroup = (image, R rows, a 256-byte slice of
    // groups, CB positions); ring slots of CB + span columns (whole KiB)
    // plus the output buffer of 16-position chunks.  Whole rows unless that
    // leaves fewer than 3 workgroups per compute unit.
    grp_wide = true;
    const int64_t gblocks = p.g / (256 / (2 * Cg));
    int64_t max_pos_h = 0, max_pos_w = 0;
    for (const auto& s : subs) {
      max_pos_h = std::max<int64_t>(max_pos_h, s.pos_h);
      max_pos_w = std::max<int64_t>(max_pos_w, s.pos_w);
    }
    auto lds_wide = [&](int64_t cb) {
      int64_t r = 0;
      for (const auto& s : subs) {
        const int64_t seg = std::min<int64_t>(cb, s.pos_w);
        const int64_t rowb = (seg + aw.delta * (s.taps_w - 1)) * 256;
        r = std::max<int64_t>(r, (s.taps_h + 1) * ceil_div(rowb, 1024) * 1024 + 16 * ceil_div(seg, 16) * 256);
      }
      return r;
    };
    int64_t cb = 16 * ceil_div(max_pos_w, 16);
    if (cols_opt > 0) {
      cb = std::min<int64_t>(cb, 16 * ceil_div(cols_opt, 16));
    } else {
      for (int64_t k = 2; lds_wide(cb) > cbd::kLdsPerCu / 3 && cb > 16; k++)
        cb = 16 * ceil_div(max_pos_w, 16 * k);
    }
    grp_cols = cb;
    grp_lds = lds_wide(cb);
    if (grp_lds > cbd::kLdsPerCu) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "grouped MFMA kernel: a 16-position block's rows exceed LDS");
    }
    int64_t units = 0;
    for (const auto& s : subs) units += p.n * s.pos_h * gblocks * ceil_div(s.pos_w, cb);
    if (rows_opt > 0) {
      grp_rows = std::min<int64_t>(rows_opt, max_pos_h);
    } else {
      // Rows per workgroup so that the grid fills up to four workgroups per
      // compute unit (fewer where LDS holds fewer).  A workgroup's fixed cost
      // (the filter taps into registers, the ring's first rows) is paid once
      // per row block, so where that leaves blocks of four rows or fewer the
      // grid halves (twice the rows each), and halves again below three rows;
      // then the rows are split evenly over the blocks of a column.  Measured
      // on the grouped sweep (N = 32, 3x3, graph replays): 32 channels per
      // group at 7x7 13.0 -> 10.2 us, at 14x14 17.6 -> 14.3 us, 8 per group
      // at 14x14 12.5 -> 8.9 us; shapes with longer blocks (7 rows or more)
      // ran slower on half the grid (16 per group, 56x56 stride 2:
      // 23.3 -> 32.5 us) and keep it.
      const int64_t per_cu = std::min<int64_t>(4, cbd::kLdsPerCu / grp_lds);
      auto rows_at = [&](int64_t wgs_per_cu) {
        const int64_t resident = 256 * std::min<int64_t>(wgs_per_cu, per_cu);
        return std::min<int64_t>(max_pos_h, std::max<int64_t>(1, ceil_div(units, resident)));
      };
      grp_rows = rows_at(4);
      if (grp_rows <= 4) grp_rows = rows_at(2);
      if (grp_rows <= 2) grp_rows = rows_at(1);
      grp_rows = ceil_div(max_pos_h, ceil_div(max_pos_h, grp_rows));
    }
  } else if (kernel == CBD_KERNEL_GROUPED && !subs.empty()) {
    // The row and direct kernels put one group per lane of a 256-lane
    // workgroup: C/G in {1, 2, 4, 8} and G dividing 256.  (With no
    // sub-GEMM at all there is no main launch, only the zero-fill.)
    if (!grouped_ok(p, Cg, Kg, max_taps)) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "grouped problem for the row / direct kernels needs C/G == K/G in "
                                       "{1,2,4,8} with G dividing 256 (the 16x16x16-MFMA kernel was not "
                                       "taken: rows_per_wg = -1, or a geometry it does not serve)");
    }
    slots = cbd::kGroupedThreads / p.g;
    const int64_t pixb = p.c * es;
    const bool mfma_ok = !grouped_dot && p.dtype == CBD_BF16 && Cg == 4 && (p.g == 32 || p.g == 64);
    int64_t need = 0, ring_dot = 0, max_pos_h = 0, max_pos_w = 0;
    for (const auto& s : subs) {
      const int64_t rowb = (s.pos_w + aw.delta * (s.taps_w - 1)) * pixb;
      need = std::max<int64_t>(need, s.taps_h * rowb);
      ring_dot = std::max<int64_t>(ring_dot, (s.taps_h + 1) * ceil_div(rowb, 4096) * 4096);
      max_pos_h = std::max<int64_t>(max_pos_h, s.pos_h);
      max_pos_w = std::max<int64_t>(max_pos_w, s.pos_w);
    }
    // MFMA kernel, column blocks of cb positions: ring slots of cb + span + 3
    // columns (whole KiB) plus the output row buffer.
    auto lds_mfma = [&](int64_t cb) {
      int64_t r = 0;
      for (const auto& s : subs) {
        const int64_t seg = std::min<int64_t>(cb, s.pos_w);
        const int64_t rowb = (seg + aw.delta * (s.taps_w - 1) + 3) * pixb;
        r = std::max<int64_t>(r, (s.taps_h + 1) * ceil_div(rowb, 1024) * 1024 + 4 * ceil_div(seg, 4) * pixb);
      }
      return r;
    };
    const bool row_ok = Cg <= 4 && pixb % 16 == 0;
    const bool pipe_ok = row_ok && rows_opt >= 0 && ah.delta == 1 && !subs.empty();
    int64_t ring = ring_dot;
    if (pipe_ok && mfma_ok) {
      // Whole rows unless that leaves fewer than 3 workgroups per compute
      // unit; then the widest multiple of 4 that fits (or the forced width).
      int64_t cb = 4 * ceil_div(max_pos_w, 4);
      if (cols_opt > 0) {
        cb = std::min<int64_t>(cb, 4 * ceil_div(cols_opt, 4));
      } else {
        for (int64_t k = 2; lds_mfma(cb) > cbd::kLdsPerCu / 3 && cb > 4; k++)
          cb = 4 * ceil_div(max_pos_w, 4 * k);
      }
      if (lds_mfma(cb) <= cbd::kLdsPerCu) {
        grp_mfma = true;
        grp_cols = cb;
        ring = lds_mfma(cb);
      }
    }
    // Merged phases: stride 2 x 2, each of the four phases a class, taps
    // one dY row and column apart, at most 4 taps per class.  A workgroup
    // walks class rows of one image and a block of cb class columns for all
    // four phases: its ring holds the union of the phases' dY rows (span_h +
    // 1 in use, one more being filled) over the union of their columns, and
    // its output buffer two dX row segments of 2 * 4*ceil(cb/4) pixels.
    bool merge_ok = grp_mfma && !per_class && p.stride_h == 2 && p.stride_w == 2 && ah.delta == 1 &&
                    aw.delta == 1 && subs.size() == 4;
    int64_t lo_h = 0, hi_h = 0, lo_w = 0, hi_w = 0, mph = 0, mpw = 0;
    if (merge_ok) {
      int seen = 0;
      lo_h = lo_w = INT64_MAX;
      hi_h = hi_w = INT64_MIN;
      for (const auto& s : subs) {
        seen |= 1 << (s.phase_h * 2 + s.phase_w);
        if (s.taps_h * s.taps_w > 4) merge_ok = false;
        lo_h = std::min<int64_t>(lo_h, s.beta_h - (s.taps_h - 1));
        hi_h = std::max<int64_t>(hi_h, s.beta_h);
        lo_w = std::min<int64_t>(lo_w, s.beta_w - (s.taps_w - 1));
        hi_w = std::max<int64_t>(hi_w, s.beta_w);
        mph = std::max<int64_t>(mph, s.pos_h);
        mpw = std::max<int64_t>(mpw, s.pos_w);
      }
      if (seen != 15) merge_ok = false;
    }
    auto lds_merged = [&](int64_t cb) {
      const int64_t seg = std::min<int64_t>(cb, mpw);
      const int64_t rowb = (seg + (hi_w - lo_w) + 3) * pixb;
      return (hi_h - lo_h + 2) * ceil_div(rowb, 1024) * 1024 + 2 * 8 * ceil_div(seg, 4) * pixb;
    };
    if (merge_opt == 1 && !merge_ok) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "merge_phases = 1: needs the grouped 4x4x4-MFMA kernel at stride 2 x 2 "
                                       "with every phase a class of at most 4 taps, taps one dY row and "
                                       "column apart, and not per_class");
    }
    // Only on request: measured slower than one class per workgroup (c5-s2
    // 19.3 against 11.8 us: a third as many workgroups, each row four times
    // the work and its 28 KiB of dX stores drained before the next row).
    if (merge_ok && merge_opt == 1) {
      int64_t cb = 4 * ceil_div(mpw, 4);
      if (cols_opt > 0) {
        cb = std::min<int64_t>(cb, 4 * ceil_div(cols_opt, 4));
      } else {
        for (int64_t k = 2; lds_merged(cb) > cbd::kLdsPerCu / 3 && cb > 4; k++)
          cb = 4 * ceil_div(mpw, 4 * k);
      }
      if (lds_merged(cb) <= cbd::kLdsPerCu) {
        grp_merged = true;
        grp_cols = cb;
        ring = lds_merged(cb);
      } else if (merge_opt == 1) {
        delete pl;
        return fail(CBD_ERR_UNSUPPORTED, "merge_phases = 1: a column block's rows exceed LDS");
      }
    }
    if (grp_merged) {
      const int64_t units = p.n * mph * ceil_div(mpw, grp_cols);  // (image, class row, column block)
      if (rows_opt > 0) {
        grp_rows = std::min<int64_t>(rows_opt, mph);
      } else {
        const int64_t resident = 256 * std::min<int64_t>(4, cbd::kLdsPerCu / ring);
        grp_rows = std::min<int64_t>(mph, std::max<int64_t>(1, ceil_div(units, resident)));
      }
      grp_lds = ring;
      merged_tiles = p.n * ceil_div(mph, grp_rows) * ceil_div(mpw, grp_cols);
    } else if (pipe_ok && ring <= cbd::kLdsPerCu) {
      int64_t units = 0;  // (image, class row, column block)
      for (const auto& s : subs) units += p.n * s.pos_h * (grp_mfma ? ceil_div(s.pos_w, grp_cols) : 1);
      if (rows_opt > 0) {
        grp_rows = std::min<int64_t>(rows_opt, max_pos_h);
      } else {
        const int64_t resident = 256 * std::min<int64_t>(4, cbd::kLdsPerCu / ring);
        grp_rows = std::min<int64_t>(max_pos_h, std::max<int64_t>(1, ceil_div(units, resident)));
      }
      grp_lds = ring;
    } else if (row_ok && need <= cbd::kGroupedRowLds) {
      grp_lds = need;
    } else {
      int64_t total_pos = 0;
      for (const auto& s : subs) total_pos += s.n;
      iters = std::max<int64_t>(1, std::min<int64_t>(64, ceil_div(total_pos, slots * 2048)));
    }
  }

  // Split-K (large-tile and generic families): S workgroups per tile, each
  // at least one k tile of every class.
  int64_t ksplit = 1;
  if (ksplit_opt >= 2) {
    if (kernel != CBD_KERNEL_NHWC_BF16 && kernel != CBD_KERNEL_GENERIC) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "ksplit needs the NHWC bf16 (large-tile) or the generic kernel");
    }
    if (per_class) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "ksplit and per_class do not combine");
    }
    ksplit = ksplit_opt;
    for (const auto& s : subs)
      ksplit = std::min<int64_t>(ksplit, kernel == CBD_KERNEL_NHWC_BF16
                                             ? s.k / cbd::kFastBK
                                             : int64_t(s.taps_h) * s.taps_w * ceil_div(Kg, bk));
    ksplit = std::max<int64_t>(ksplit, 1);
  }

  // Shape-specialised instances of the large-tile kernel.  Level 1: k tiles
  // per tap and taps per class fixed at compile time (K/G = 2048, one tap
  // per class).  Level 2: the whole geometry fixed (C = K = 2048, G = 1,
  // Hi = 1, a 1x2 filter at stride 2 along W, no padding or dilation, Wi
  // even, so class r writes dX pixel 2p + r from dY pixel p; N and Wi stay
  // free).  Each computes the same bits as the descriptor-driven kernel; the
  // most specialised one that matches is used unless the caller asks for the
  // descriptor-driven kernel.
  int static_shape = 0;
  {
    bool ok1 = kernel == CBD_KERNEL_NHWC_BF16 && ksplit == 1 && Kg == 64 * cbd::kFastBK &&
               !no_split && !subs.empty();
    for (const auto& s : subs) ok1 = ok1 && s.taps_h * s.taps_w == 1;
    // (Level 2 takes a class from its tile index, so not one launch per class.)
    bool ok2 = ok1 && !per_class && p.g == 1 && Cg == 2048 && p.hi == 1 && p.y == 1 && p.x == 2 &&
               p.stride_w == 2 && p.pad_h == 0 && p.pad_w == 0 && p.dil_w == 1 && p.wi % 2 == 0 &&
               subs.size() == 2;
    for (size_t i = 0; ok2 && i < subs.size(); i++)
      ok2 = subs[i].phase_w == (int32_t)i && subs[i].class_w == (int32_t)i && subs[i].beta_w == 0 &&
            subs[i].phase_h == 0 && subs[i].beta_h == 0 && subs[i].pos_h == 1 && subs[i].pos_w == Wo;
    if (static_mode == 1 && kernel != CBD_KERNEL_GENERIC && kernel != CBD_KERNEL_GROUPED && !ok1) {
      delete pl;
      return fail(CBD_ERR_UNSUPPORTED, "no shape-specialised instance for this problem "
                                       "(built: NHWC bf16, K/G = 2048, one tap per class, residue split, "
                                       "no K split; and the generic family's listed workload shapes)");
    }
    static_shape = static_mode < 0 ? 0 : ok2 ? 2 : ok1 ? 1 : 0;
  }

  // Tiles per class (contiguous ranges of the logical grid, in LPT order).
  int64_t tile = 0;
  int64_t tiles_m = kernel == CBD_KERNEL_GROUPED ? 1 : ceil_div(Cg, bm);
  bool equal_k = true;
  int64_t exec = 0;
  for (size_t i = 0; i < subs.size(); i++) {
    cbd_subgemm_t& s = subs[i];
    s.id = (int32_t)i;
    s.tile_begin = tile;
    if (kernel == CBD_KERNEL_NCHW_ROWS)
      s.tiles = 0, s.tile_begin = 0;  // every workgroup serves every class
    else if (grp_merged)
      s.tiles = 0, s.tile_begin = 0;  // every workgroup serves every class
    else if (kernel == CBD_KERNEL_GROUPED)
      s.tiles = grp_wide      ? p.n * ceil_div(s.pos_h, grp_rows) * (p.g / (256 / (2 * Cg))) *
                                    ceil_div(s.pos_w, grp_cols)
                : grp_mfma      ? p.n * ceil_div(s.pos_h, grp_rows) * ceil_div(s.pos_w, grp_cols)
                : grp_rows > 0  ? p.n * ceil_div(s.pos_h, grp_rows)
                : grp_lds > 0 ? p.n * s.pos_h
                              : ceil_div(s.n, slots * iters);
    else
      s.tiles = p.g * tiles_m * ceil_div(s.n, bn) * ksplit;
    tile += s.tiles;
    if (s.k != subs[0].k) equal_k = false;
    exec += p.g * s.m * s.n * s.k;
  }
  if (kernel == CBD_KERNEL_NCHW_ROWS) tile = p.n * p.g * rgeom.c_blocks * rgeom.row_blocks;
  if (grp_merged) tile = merged_tiles;
  // A launch must stay below 2^32 work-items.
  if (tile * threads >= (int64_t(1) << 32)) {
    delete pl;
    return fail(CBD_ERR_UNSUPPORTED, "grid too large");
  }

  // Zero regions: every phase pair with positions that no class reaches.
  std::vector<cbd_zero_region_t> zeros;
  for (int64_t ph = 0; ph < p.stride_h; ph++) {
    for (int64_t pw = 0; pw < p.stride_w; pw++) {
      if (reached[(size_t)(ph * p.stride_w + pw)]) continue;
      const int64_t nh = ph < p.hi ? ceil_div(p.hi - ph, p.stride_h) : 0;
      const int64_t nw = pw < p.wi ? ceil_div(p.wi - pw, p.stride_w) : 0;
      if (nh * nw == 0) continue;
      cbd_zero_region_t z;
      z.phase_h = (int32_t)ph;
      z.phase_w = (int32_t)pw;
      z.pos_h = nh;
      z.pos_w = nw;
      zeros.push_back(z);
    }
  }

  // Kernel arguments.
  cbd::GemmArgs& a = pl->gemm;
  a.N = (int32_t)p.n; a.G = (int32_t)p.g; a.C = (int32_t)p.c; a.K = (int32_t)p.k;
  a.Cg = (int32_t)Cg; a.Kg = (int32_t)Kg;
  a.Hi = (int32_t)p.hi; a.Wi = (int32_t)p.wi; a.Ho = (int32_t)Ho; a.Wo = (int32_t)Wo;
  a.Y = (int32_t)p.y; a.X = (int32_t)p.x;
  // no_split: positions are dX positions themselves (S = 1 in the position
  // map), every tap (T = 1); the true stride, pad and dilation go alongside.
  a.Sh = no_split ? 1 : p.stride_h; a.Sw = no_split ? 1 : p.stride_w;
  a.tstep_h = no_split ? 1 : (int32_t)ah.T; a.tstep_w = no_split ? 1 : (int32_t)aw.T;
  a.delta_h = (int32_t)ah.delta; a.delta_w = (int32_t)aw.delta;
  a.no_split = no_split ? 1 : 0;
  a.str_h = p.stride_h; a.str_w = p.stride_w;
  a.pad_h = p.pad_h; a.pad_w = p.pad_w;
  a.dil_h = p.dil_h; a.dil_w = p.dil_w;
  a.dy_bytes = (uint32_t)(p.n * p.k * Ho * Wo * es);
  a.w_bytes = (uint32_t)(p.k * Cg * p.y * p.x * es);
  a.dx_bytes = (uint32_t)(p.n * p.c * p.hi * p.wi * es);
  a.num_sub = (int32_t)subs.size();
  a.total_tiles = (int32_t)tile;
  a.tiles_m = (int32_t)tiles_m;
  a.tile_n = (int32_t)(kernel == CBD_KERNEL_GROUPED ? (grp_lds > 0 ? subs[0].pos_w : slots * iters) : bn);
  a.tile_m = (int32_t)bm;
  // XCD-contiguous tile ranges pay when one panel is shared by many tiles;
  // with unequal K they would also hand the long tiles to a few XCDs.
  a.xcd_remap = (kernel != CBD_KERNEL_GROUPED && equal_k && tile >= 64) ? 1 : 0;
  a.iters = (int32_t)iters;
  a.grp_lds = (int32_t)grp_lds;
  a.grp_rows = (int32_t)grp_rows;
  a.grp_mfma = grp_mfma ? 1 : 0;
  a.grp_wide = grp_wide ? 1 : 0;
  a.grp_merged = grp_merged ? 1 : 0;
  a.grp_cols = (int32_t)grp_cols;
  a.ksplit = ksplit > 1 ? (int32_t)ksplit : 0;
  a.static_shape = static_shape;
  a.gen_waves = kernel == CBD_KERNEL_GENERIC ? (int32_t)(threads / 64) : 0;
  a.ws = nullptr;
  pl->grid_finalize = ksplit <= 1                    ? 0
                      : kernel == CBD_KERNEL_GENERIC ? tile / ksplit
                                                     : tile / ksplit * (cbd::kFastBN / 8);
  for (size_t i = 0; i < subs.size(); i++) {
    cbd::SubDesc& d = a.sub[i];
    const cbd_subgemm_t& s = subs[i];
    d.phase_h = s.phase_h; d.phase_w = s.phase_w;
    d.beta_h = s.beta_h; d.beta_w = s.beta_w;
    d.taps_h = s.taps_h; d.taps_w = s.taps_w;
    d.cls_h = s.class_h; d.cls_w = s.class_w;
    d.pos_h = (int32_t)s.pos_h; d.pos_w = (int32_t)s.pos_w;
    d.tile_begin = (int32_t)s.tile_begin;
    a.class_begin[i] = d.tile_begin;
    if (kernel == CBD_KERNEL_GENERIC && i < (size_t)cbd::kMagSub) {
      const int64_t npix = s.pos_h * s.pos_w;
      a.mag_npix[i] = magic32(npix);
      a.mag_posw[i] = magic32(s.pos_w);
      a.mag_pergroup[i] = magic32(tiles_m * ceil_div(p.n * npix, bn));
    }
  }
  a.mag_tiles_m = magic32(tiles_m);
  // Generic family, one class at phase (0,0) whose lattice is every S x S
  // block of dX (a 1x1 filter at stride S, for one): the main kernel's
  // epilogue writes each block whole, zeros included, instead of leaving
  // the other phases to zero-fill workgroups.
  const bool zblock = kernel == CBD_KERNEL_GENERIC && !per_class && !no_split && ksplit == 1 &&
                      subs.size() == 1 && p.stride_h * p.stride_w > 1 && p.stride_h * p.stride_w <= 16 &&
                      subs[0].phase_h == 0 && subs[0].phase_w == 0 &&
                      subs[0].pos_h == ceil_div(p.hi, p.stride_h) && subs[0].pos_w == ceil_div(p.wi, p.stride_w);
  a.zblock = zblock ? 1 : 0;
  // Generic family, f32 KCYX: the row-load patterns of the classes (the
  // launch picks an instance compiled with just those).
  a.row_pats = 0;
  if (kernel == CBD_KERNEL_GENERIC && p.dtype == CBD_F32 && p.layout == CBD_LAYOUT_NCHW && !no_split)
    for (const auto& s : subs)
      a.row_pats |= 1 << cbd::row_pattern(s.taps_h, s.taps_w, s.class_w, (int)p.x, s.tstep_w);
  a.row_pats &= cbd::kRowPatsAll;
  // Generic family: the shape-specialised instance whose compiled geometry
  // is exactly this plan's, if one was built.
  a.static_id = 0;
  if (kernel == CBD_KERNEL_GENERIC && static_mode >= 0 && ksplit == 1 && !no_split && !per_class) {
    for (int i = 0; i < cbd::kGenericShapes; i++) {
      if (generic_shape_matches(cbd::kGenericShapeKeys[i], a, p, threads)) {
        static_shape = 2;
        a.static_shape = 2;
        a.static_id = i;
        break;
      }
    }
  }
  // Grouped 4x4x4-MFMA kernel: likewise.
  if (kernel == CBD_KERNEL_GROUPED && grp_mfma && !grp_merged && static_mode >= 0 && !per_class) {
    for (int i = 0; i < cbd::kGroupedShapes; i++) {
      if (grouped_shape_matches(cbd::kGroupedShapeKeys[i], a, p, threads)) {
        static_shape = 2;
        a.static_shape = 2;
        a.static_id = i;
        break;
      }
    }
  }
  if (static_mode == 1 && (kernel == CBD_KERNEL_GENERIC || kernel == CBD_KERNEL_GROUPED) && static_shape == 0) {
    delete pl;
    return fail(CBD_ERR_UNSUPPORTED, "no shape-specialised instance for this plan "
                                     "(built for the listed workload shapes only)");
  }

  cbd::ZeroArgs& z = pl->zero;
  z.N = (int32_t)p.n; z.C = (int32_t)p.c; z.Hi = (int32_t)p.hi; z.Wi = (int32_t)p.wi;
  z.Sh = p.stride_h; z.Sw = p.stride_w;
  z.layout = p.layout;
  z.esize = (int32_t)es;
  z.chunk = (p.layout == CBD_LAYOUT_NHWC && (p.c * es) % 16 == 0) ? 16 : (int32_t)es;
  z.num_regions = (int32_t)zeros.size();
  z.dx_bytes = a.dx_bytes;
  int64_t items = 0, zero_elems = 0;
  for (size_t i = 0; i < zeros.size(); i++) {
    cbd::ZeroDesc& d = z.reg[i];
    d.phase_h = zeros[i].phase_h; d.phase_w = zeros[i].phase_w;
    d.pos_h = (int32_t)zeros[i].pos_h; d.pos_w = (int32_t)zeros[i].pos_w;
    d.item_begin = items;
    d.per_pos = (uint32_t)(p.layout == CBD_LAYOUT_NHWC ? p.c * es / z.chunk : 1);
    d.mag_h = magic32(d.pos_h);
    d.mag_w = magic32(d.pos_w);
    d.mag_pp = magic32(d.per_pos);
    const int64_t npos = p.n * zeros[i].pos_h * zeros[i].pos_w;
    items += p.layout == CBD_LAYOUT_NHWC ? npos * (p.c * es / z.chunk) : npos * p.c;
    zero_elems += npos * p.c;
  }
  z.total_items = items;
  if (items >= (int64_t(1) << 32)) {
    delete pl;
    return fail(CBD_ERR_UNSUPPORTED, "zero-fill grid too large");
  }

  // Generic family with few zero regions: fold the zero-fill into the main
  // launch as extra workgroups (one launch instead of two).
  int64_t grid_zero = ceil_div(items, int64_t(cbd::kZeroThreads) * cbd::kZeroItemsPerThread);
  int64_t grid_main = tile;
  // The row-block family, and the generic family's whole-block epilogue,
  // write unreached positions themselves.
  if (kernel == CBD_KERNEL_NCHW_ROWS || zblock) grid_zero = 0;
  a.rg = rgeom;
  std::memset(&a.fz, 0, sizeof(a.fz));
  if (kernel == CBD_KERNEL_GENERIC && !per_class && !zblock && items > 0 &&
      (int64_t)zeros.size() <= cbd::kMaxFusedZero &&
      threads == cbd::kZeroThreads &&
      (tile + grid_zero) * threads < (int64_t(1) << 32)) {
    cbd::FusedZero& f = a.fz;
    f.num_regions = z.num_regions;
    f.layout = z.layout; f.esize = z.esize; f.chunk = z.chunk;
    f.C = z.C; f.Hi = z.Hi; f.Wi = z.Wi; f.Sh = z.Sh; f.Sw = z.Sw;
    f.total_items = items;
    for (size_t i = 0; i < zeros.size(); i++) f.reg[i] = z.reg[i];
    grid_main = tile + grid_zero;
    grid_zero = 0;
  }

  cbd_plan_info_t& info = pl->info;
  info.ho = Ho;
  info.wo = Wo;
  info.num_subgemms = (int32_t)subs.size();
  info.num_zero_regions = (int32_t)zeros.size();
  info.kernel = kernel;
  info.tile_m = (int32_t)bm;
  info.tile_n = (int32_t)a.tile_n;
  info.tile_k = (int32_t)bk;
  info.threads_main = (int32_t)threads;
  info.grid_main = grid_main;
  info.grid_zero = grid_zero;
  info.launches = (grid_main > 0 ? (per_class ? (int32_t)subs.size() : 1) : 0) + (grid_zero > 0 ? 1 : 0) +
                  (ksplit > 1 ? 1 : 0);
  pl->per_class = per_class;
  info.useful_flops = 2 * p.n * p.c * Kg * Ho * Wo * p.y * p.x;
  info.executed_macs = exec;
  info.zero_elems = zero_elems;
  info.lds_dynamic = kernel == CBD_KERNEL_NCHW_ROWS ? rgeom.lds_bytes : grp_lds;
  info.rows_per_wg = kernel == CBD_KERNEL_NCHW_ROWS ? rgeom.rb : grp_rows;
  info.cols_per_wg = grp_cols;
  info.ksplit = ksplit;
  info.static_shape = static_shape;
  info.workspace_bytes = ksplit > 1 ? tile * bm * bn * 4 : 0;  // one f32 partial per (tile, split)
  info.auto_ksplit = 1;
  info.auto_workspace_bytes = 0;
  info.zero_in_epilogue = (zblock || kernel == CBD_KERNEL_NCHW_ROWS) && zero_elems > 0 ? 1 : 0;
  info.reserved_ = 0;
  // Pointer alignment: the generic family gathers and stores single
  // elements; a zero-fill of NHWC rows writes 16-byte chunks; the other
  // families move 16-byte vectors.
  if (kernel == CBD_KERNEL_GENERIC) {
    info.align_dy = info.align_w = (int32_t)es;
    info.align_dx = zblock ? (zblock_pairs(p) ? 2 * (int32_t)es : (int32_t)es)
                    : (zero_elems > 0 && z.chunk == 16) ? 16 : (int32_t)es;
  } else if (kernel == CBD_KERNEL_NCHW_ROWS) {
    // element loads of dY (16-byte loads of W when its rows allow);
    // whole dX rows in the widest store that divides a row
    info.align_dy = (int32_t)es;
    info.align_w = rgeom.wvec ? 16 : (int32_t)es;
    info.align_dx = rgeom.vb;
  } else {
    info.align_dy = info.align_w = info.align_dx = 16;
  }
  info.variant = kernel != CBD_KERNEL_GROUPED ? 0
                 : grp_merged                  ? 5
                 : grp_wide                    ? 4
                 : grp_mfma                    ? 3
                 : grp_rows > 0                ? 2
                 : grp_lds > 0                 ? 1
                                               : 0;

  pl->subs = std::move(subs);
  pl->zeros = std::move(zeros);
  if (log_enabled()) log_plan(*pl);

  // The planner's own split-K configuration (ksplit option 0), kept beside
  // the plan and run by cbd_run_ws when the caller's workspace holds it.
  if (ksplit_opt == 0 && !per_class) {
    const int64_t auto_s = auto_ksplit(kernel, tile, min_class_ktiles(pl->subs, kernel, Kg, bk));
    if (auto_s >= 2) {
      cbd_plan_options o;
      std::memset(&o, 0, sizeof(o));
      if (options) o = *options;
      o.force_kernel = kernel;
      o.ksplit = (int32_t)auto_s;
      cbd_plan_t* alt = nullptr;
      if (cbd_plan_ex(problem, &o, &alt) == CBD_OK && alt->info.ksplit >= 2) {
        pl->split_alt = alt;
        pl->info.auto_ksplit = alt->info.ksplit;
        pl->info.auto_workspace_bytes = alt->info.workspace_bytes;
      } else {
        delete alt;
      }
      cbd::set_error("");
    }
  }
  *out_plan = pl;
  return CBD_OK;
}

extern "C" cbd_status cbd_plan(const cbd_problem* problem, cbd_plan_t** out_plan) {
  return cbd_plan_ex(problem, nullptr, out_plan);
}

extern "C" void cbd_plan_destroy(cbd_plan_t* plan) { delete plan; }

extern "C" cbd_status cbd_plan_info(const cbd_plan_t* plan, cbd_plan_info_t* out) {
  if (!plan || !out) return fail(CBD_ERR_INVALID_ARG, "NULL plan or out");
  *out = plan->info;
  return CBD_OK;
}

extern "C" cbd_status cbd_plan_subgemm(const cbd_plan_t* plan, int32_t i, cbd_subgemm_t* out) {
  if (!plan || !out) return fail(CBD_ERR_INVALID_ARG, "NULL plan or out");
  if (i < 0 || (size_t)i >= plan->subs.size()) return fail(CBD_ERR_INVALID_ARG, "sub-GEMM index out of range");
  *out = plan->subs[(size_t)i];
  return CBD_OK;
}

extern "C" cbd_status cbd_plan_zero_region(const cbd_plan_t* plan, int32_t i, cbd_zero_region_t* out) {
  if (!plan || !out) return fail(CBD_ERR_INVALID_ARG, "NULL plan or out");
  if (i < 0 || (size_t)i >= plan->zeros.size()) return fail(CBD_ERR_INVALID_ARG, "zero-region index out of range");
  *out = plan->zeros[(size_t)i];
  return CBD_OK;
}
