// Planner fuzz for a sanitizer build (host only): cbd_plan_ex on random
// problems and options, including degenerate and out-of-range ones.  Every
// call must return a status (never crash); every accepted plan must satisfy
// the planner's own invariants.  Built with -fsanitize=address,undefined by
// tests/test_sanitizers.py together with the planner source.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>

#include "cbd_internal.h"

namespace cbd {
void set_error(const std::string&) {}
}  // namespace cbd

static int fail(const char* what, const cbd_problem& p) {
  std::fprintf(stderr, "invariant failed: %s (N=%lld G=%lld C=%lld K=%lld H=%lld W=%lld %lldx%lld s=%d,%d p=%d,%d d=%d,%d l=%d t=%d)\n",
               what, (long long)p.n, (long long)p.g, (long long)p.c, (long long)p.k, (long long)p.hi,
               (long long)p.wi, (long long)p.y, (long long)p.x, p.stride_h, p.stride_w, p.pad_h, p.pad_w,
               p.dil_h, p.dil_w, p.layout, p.dtype);
  return 1;
}

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 100000;
  std::mt19937_64 rng(argc > 2 ? std::atoll(argv[2]) : 1);
  auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
  auto uni = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); };
  long accepted = 0;
  for (long it = 0; it < iters; it++) {
    cbd_problem p;
    std::memset(&p, 0, sizeof(p));
    const int64_t g = rng() % 4 == 0 ? pick({1, 2, 3, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 260, 512, 1024})
                                     : uni(1, 8);
    const int64_t cg = rng() % 3 == 0 ? pick({1, 2, 4, 8, 16, 32}) : uni(1, 300);
    const int64_t kg = rng() % 2 ? cg : (rng() % 3 == 0 ? pick({32, 64, 2048}) : uni(1, 300));
    p.n = rng() % 50 == 0 ? uni(-1, 0) : uni(1, 40);
    p.g = rng() % 200 == 0 ? 0 : g;
    p.c = g * cg + (rng() % 100 == 0 ? 1 : 0);
    p.k = g * kg;
    p.hi = rng() % 20 == 0 ? pick({1, 2, 512, 4096, 65536}) : uni(1, 80);
    p.wi = rng() % 20 == 0 ? pick({1, 2, 512, 4096, 65536}) : uni(1, 80);
    p.y = uni(1, 7);
    p.x = uni(1, 7);
    p.stride_h = (int32_t)(rng() % 30 == 0 ? pick({0, 65, 100}) : uni(1, 5));
    p.stride_w = (int32_t)(rng() % 30 == 0 ? pick({0, 16, 64}) : uni(1, 5));
    p.pad_h = (int32_t)(rng() % 40 == 0 ? pick({-1, 1 << 21}) : uni(0, 4));
    p.pad_w = (int32_t)uni(0, 4);
    p.dil_h = (int32_t)(rng() % 40 == 0 ? pick({0, 65}) : uni(1, 4));
    p.dil_w = (int32_t)uni(1, 4);
    p.layout = (int32_t)(rng() % 50 == 0 ? 7 : uni(0, 1));
    p.dtype = (int32_t)(rng() % 50 == 0 ? 9 : uni(0, 1));
    cbd_plan_options o;
    std::memset(&o, 0, sizeof(o));
    o.force_kernel = (int32_t)uni(-1, 3);
    o.no_split = rng() % 8 == 0;
    o.rows_per_wg = (int32_t)pick({0, 0, 0, -1, 1, 3, 64});
    o.grouped_dot = rng() % 6 == 0;
    o.cols_per_wg = (int32_t)pick({0, 0, 4, 13, 16, 20});
    o.ksplit = (int32_t)pick({0, 0, 0, 2, 3, 8, 64});
    o.per_class = rng() % 8 == 0;
    o.static_shape = (int32_t)pick({0, 0, -1, 1});
    cbd_plan_t* pl = nullptr;
    const cbd_status st = cbd_plan_ex(&p, rng() % 4 ? &o : nullptr, &pl);
    if (st != CBD_OK) {
      if (pl) return fail("non-OK status left a plan", p);
      continue;
    }
    accepted++;
    cbd_plan_info_t in;
    if (cbd_plan_info(pl, &in) != CBD_OK) return fail("info", p);
    int64_t macs = 0, tiles = 0;
    for (int32_t i = 0; i < in.num_subgemms; i++) {
      cbd_subgemm_t s;
      if (cbd_plan_subgemm(pl, i, &s) != CBD_OK || s.id != i) return fail("subgemm id", p);
      if (s.m <= 0 || s.n <= 0 || s.k <= 0) return fail("empty sub-GEMM", p);
      if (in.kernel == CBD_KERNEL_NCHW_ROWS) {
        if (s.tiles != 0 || s.tile_begin != 0) return fail("row-block classes own no tile range", p);
      } else {
        if (s.tiles <= 0) return fail("sub-GEMM without tiles", p);
        if (s.tile_begin != tiles) return fail("tile ranges not contiguous", p);
      }
      tiles += s.tiles;
      macs += p.g * s.m * s.n * s.k;
    }
    if (macs != in.executed_macs) return fail("executed MACs", p);
    if (in.num_subgemms > 0 && in.grid_main < tiles) return fail("grid below tile count", p);
    if (in.kernel == CBD_KERNEL_NCHW_ROWS && (in.grid_zero != 0 || in.lds_dynamic <= 0 || in.lds_dynamic > 160 * 1024))
      return fail("row-block launch shape", p);
    if (in.num_subgemms == 0 && in.grid_main != 0 && in.grid_zero != 0) return fail("grid without sub-GEMM", p);
    for (int32_t i = 0; i < in.num_zero_regions; i++) {
      cbd_zero_region_t z;
      if (cbd_plan_zero_region(pl, i, &z) != CBD_OK || z.pos_h <= 0 || z.pos_w <= 0) return fail("zero region", p);
    }
    for (int32_t a : {in.align_dy, in.align_w, in.align_dx})
      if (a <= 0 || (a & (a - 1))) return fail("alignment not a power of two", p);
    if (in.useful_flops != 2 * p.n * p.c * (p.k / p.g) * in.ho * in.wo * p.y * p.x) return fail("useful flops", p);
    cbd_plan_destroy(pl);
  }
  std::printf("plans: %ld, accepted %ld\n", iters, accepted);
  return 0;
}
