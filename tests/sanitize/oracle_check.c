/* Oracle identities for a sanitizer build (host only): on small random
 * problems with integer-valued operands, exact in double precision,
 *   <conv_fwd(x, W), dY> == <x, bwd_data(dY, W)>        (adjoint),
 *   bwd_data == bwd_data_zero_insert == bwd_data_at     (three forms).
 * Built with -fsanitize=address,undefined by tests/test_sanitizers.py
 * together with the oracle source; it only calls the oracle's C entry
 * points. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int cbd_oracle_out_hw(const int64_t* p, int64_t* ho_wo);
int cbd_oracle_conv_fwd(const int64_t* p, const double* x, const double* w, double* y);
int cbd_oracle_bwd_data(const int64_t* p, const double* dy, const double* w, double* dx);
int cbd_oracle_bwd_data_at(const int64_t* p, const double* dy, const double* w, int64_t npts,
                           const int64_t* pts, double* out);
int cbd_oracle_bwd_data_zero_insert(const int64_t* p, const double* dy, const double* w, double* dx,
                                    int64_t* geom);

static uint64_t st = 88172645463325252ull;
static int64_t rnd(int64_t lo, int64_t hi) {
  st ^= st << 13; st ^= st >> 7; st ^= st << 17;
  return lo + (int64_t)(st % (uint64_t)(hi - lo + 1));
}

int main(int argc, char** argv) {
  const int count = argc > 1 ? atoi(argv[1]) : 300;
  int done = 0;
  for (int it = 0; done < count && it < 100 * count; it++) {
    int64_t p[15];
    const int64_t g = rnd(1, 3), cg = rnd(1, 3), kg = rnd(1, 3);
    p[0] = rnd(1, 2); p[1] = g; p[2] = g * cg; p[3] = g * kg; p[4] = rnd(1, 9); p[5] = rnd(1, 9);
    p[6] = rnd(1, 4); p[7] = rnd(1, 4); p[8] = rnd(1, 3); p[9] = rnd(1, 3); p[10] = rnd(0, 2);
    p[11] = rnd(0, 2); p[12] = rnd(1, 2); p[13] = rnd(1, 2); p[14] = rnd(0, 1);
    int64_t hw[2];
    if (cbd_oracle_out_hw(p, hw) || hw[0] < 1 || hw[1] < 1) continue;
    const int64_t nx = p[0] * p[2] * p[4] * p[5], ny = p[0] * p[3] * hw[0] * hw[1];
    const int64_t nw = p[3] * cg * p[6] * p[7];
    double* x = malloc(sizeof(double) * nx);
    double* dy = malloc(sizeof(double) * ny);
    double* w = malloc(sizeof(double) * nw);
    double* y = malloc(sizeof(double) * ny);
    double* dx = malloc(sizeof(double) * nx);
    double* dz = malloc(sizeof(double) * nx);
    double* da = malloc(sizeof(double) * nx);
    int64_t* pts = malloc(sizeof(int64_t) * 4 * nx);
    for (int64_t i = 0; i < nx; i++) x[i] = (double)rnd(-2, 2);
    for (int64_t i = 0; i < ny; i++) dy[i] = (double)rnd(-2, 2);
    for (int64_t i = 0; i < nw; i++) w[i] = (double)rnd(-2, 2);
    int64_t geom[4];
    if (cbd_oracle_conv_fwd(p, x, w, y) || cbd_oracle_bwd_data(p, dy, w, dx) ||
        cbd_oracle_bwd_data_zero_insert(p, dy, w, dz, geom)) {
      fprintf(stderr, "oracle refused a valid problem\n");
      return 1;
    }
    /* every element through the per-point entry, in (n, channel, h, w) order */
    int64_t k = 0;
    for (int64_t n = 0; n < p[0]; n++)
      for (int64_t c = 0; c < p[2]; c++)
        for (int64_t h = 0; h < p[4]; h++)
          for (int64_t v = 0; v < p[5]; v++) {
            pts[4 * k] = n; pts[4 * k + 1] = c; pts[4 * k + 2] = h; pts[4 * k + 3] = v;
            k++;
          }
    if (cbd_oracle_bwd_data_at(p, dy, w, nx, pts, da)) return 1;
    double lhs = 0, rhs = 0;
    for (int64_t i = 0; i < ny; i++) lhs += y[i] * dy[i];
    for (int64_t i = 0; i < nx; i++) rhs += x[i] * dx[i];
    if (lhs != rhs) { fprintf(stderr, "adjoint identity: %g != %g\n", lhs, rhs); return 1; }
    for (int64_t i = 0; i < nx; i++)
      if (dx[i] != dz[i]) { fprintf(stderr, "zero-insertion form differs\n"); return 1; }
    for (int64_t i = 0; i < nx; i++) {
      const int64_t n = pts[4 * i], c = pts[4 * i + 1], h = pts[4 * i + 2], v = pts[4 * i + 3];
      const int64_t off = p[14] == 0 ? ((n * p[2] + c) * p[4] + h) * p[5] + v
                                     : ((n * p[4] + h) * p[5] + v) * p[2] + c;
      if (da[i] != dx[off]) { fprintf(stderr, "per-point form differs\n"); return 1; }
    }
    free(x); free(dy); free(w); free(y); free(dx); free(dz); free(da); free(pts);
    done++;
  }
  printf("problems: %d\n", done);
  return done == count ? 0 : 1;
}
