/*
 * cbd_oracle.c -- plain, slow, obviously-correct CPU reference for 2-D
 * convolution backward-data (dX = conv_bwd_data(dY, W)).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU product path includes, links
 * or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no header, helper or
 * table with the HIP library.
 *
 * What it follows (pages as cited; no code is taken from them):
 *  - Problem statement (filter/input/output layouts gkcyx / ngchw / ngkhw,
 *    N, C, K, Hi, Wi, Y, X, per-axis pad / stride / dilation, groups):
 *    rocMLIR PR #246 "Backward data", the tested driver command lines at the
 *    end of the thread.
 *  - NHWC / KYXC layouts, bf16 operands widened to f32, products and sums in
 *    f32, output truncated to bf16: fusilli issue #101, the BOO listing
 *    (import shapes, the 7-D contraction with extf/mulf/addf, the truncf).
 *  - Zero-insertion + flipped-filter form (the "cross form" below): the same
 *    BOO listing -- weight flip along x, dY inserted at offset 1 with stride 2
 *    into a 513-wide zero tensor, then a plain correlation.
 *  - Backward-data is defined as the adjoint (transpose) of the forward
 *    convolution in x; that definition is written out below as a gather.
 *
 * Every sum is taken in double precision.  Inputs are the exact operand
 * values (fp32 or bf16) widened to double by the caller.
 *
 * Problem vector p[] (int64), shared by every entry point:
 *   p[0]=N p[1]=G p[2]=C (total) p[3]=K (total) p[4]=Hi p[5]=Wi p[6]=Y p[7]=X
 *   p[8]=stride_h p[9]=stride_w p[10]=pad_h p[11]=pad_w p[12]=dil_h
 *   p[13]=dil_w p[14]=layout (0: ngchw/ngkhw/gkcyx, 1: NHWC/NHWK/KYXC)
 *
 * Parity pins (tests/test_oracle_pins.py) cover every function here; none is
 * "parity unpinned".
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t N, G, C, K, Hi, Wi, Y, X, Sh, Sw, Ph, Pw, Dh, Dw, layout;
  int64_t Cg, Kg, Ho, Wo;
} prob_t;

/* Output extent of a forward convolution along one axis: the number of
 * window positions of a (dilated) filter over the zero-padded input. */
static int64_t out_extent(int64_t in, int64_t pad, int64_t dil, int64_t taps,
                          int64_t stride) {
  int64_t span = dil * (taps - 1) + 1;
  int64_t room = in + 2 * pad - span;
  if (room < 0) return 0;
  return room / stride + 1;
}

static int unpack(const int64_t* p, prob_t* q) {
  q->N = p[0]; q->G = p[1]; q->C = p[2]; q->K = p[3]; q->Hi = p[4];
  q->Wi = p[5]; q->Y = p[6]; q->X = p[7]; q->Sh = p[8]; q->Sw = p[9];
  q->Ph = p[10]; q->Pw = p[11]; q->Dh = p[12]; q->Dw = p[13];
  q->layout = p[14];
  if (q->G < 1 || q->C % q->G || q->K % q->G) return -1;
  if (q->Sh < 1 || q->Sw < 1 || q->Dh < 1 || q->Dw < 1) return -1;
  if (q->Ph < 0 || q->Pw < 0) return -1;
  q->Cg = q->C / q->G;
  q->Kg = q->K / q->G;
  q->Ho = out_extent(q->Hi, q->Ph, q->Dh, q->Y, q->Sh);
  q->Wo = out_extent(q->Wi, q->Pw, q->Dw, q->X, q->Sw);
  return 0;
}

/* Memory offsets.  Channel numbering is group-major: input channel
 * g*(C/G)+c, output channel g*(K/G)+k, filter row g*(K/G)+k. */
static int64_t off_x(const prob_t* q, int64_t n, int64_t g, int64_t c,
                     int64_t h, int64_t w) {
  int64_t ch = g * q->Cg + c;
  if (q->layout == 0) return ((n * q->C + ch) * q->Hi + h) * q->Wi + w;
  return ((n * q->Hi + h) * q->Wi + w) * q->C + ch;
}
static int64_t off_y(const prob_t* q, int64_t n, int64_t g, int64_t k,
                     int64_t h, int64_t w) {
  int64_t ch = g * q->Kg + k;
  if (q->layout == 0) return ((n * q->K + ch) * q->Ho + h) * q->Wo + w;
  return ((n * q->Ho + h) * q->Wo + w) * q->K + ch;
}
static int64_t off_w(const prob_t* q, int64_t g, int64_t k, int64_t c,
                     int64_t y, int64_t x) {
  int64_t row = g * q->Kg + k;
  if (q->layout == 0) return ((row * q->Cg + c) * q->Y + y) * q->X + x;
  return ((row * q->Y + y) * q->X + x) * q->Cg + c;
}

/* Which output index a (input index, tap) pair feeds in the forward
 * convolution: out*stride + tap*dil - pad = in.  Returns -1 if the pair
 * feeds no output (not on the stride lattice, or outside [0, out_n)). */
static int64_t feeding_output(int64_t in, int64_t tap, int64_t stride,
                              int64_t pad, int64_t dil, int64_t out_n) {
  int64_t t = in + pad - tap * dil;
  if (t < 0 || t % stride != 0) return -1;
  t /= stride;
  return t < out_n ? t : -1;
}

int cbd_oracle_out_hw(const int64_t* p, int64_t* ho_wo) {
  prob_t q;
  if (unpack(p, &q)) return -1;
  ho_wo[0] = q.Ho;
  ho_wo[1] = q.Wo;
  return 0;
}

/* Forward convolution (used only by the adjoint and finite-difference pins):
 * y[n,g,k,ho,wo] = sum_{c,y,x} x[n,g,c, ho*Sh + y*Dh - Ph, wo*Sw + x*Dw - Pw]
 *                  * W[g,k,c,y,x], with x outside the image taken as zero. */
int cbd_oracle_conv_fwd(const int64_t* p, const double* x, const double* w,
                        double* yout) {
  prob_t q;
  if (unpack(p, &q)) return -1;
#pragma omp parallel for collapse(3) schedule(static)
  for (int64_t n = 0; n < q.N; n++)
    for (int64_t g = 0; g < q.G; g++)
      for (int64_t k = 0; k < q.Kg; k++)
        for (int64_t ho = 0; ho < q.Ho; ho++)
          for (int64_t wo = 0; wo < q.Wo; wo++) {
            double acc = 0.0;
            for (int64_t c = 0; c < q.Cg; c++)
              for (int64_t ky = 0; ky < q.Y; ky++) {
                int64_t h = ho * q.Sh + ky * q.Dh - q.Ph;
                if (h < 0 || h >= q.Hi) continue;
                for (int64_t kx = 0; kx < q.X; kx++) {
                  int64_t wi = wo * q.Sw + kx * q.Dw - q.Pw;
                  if (wi < 0 || wi >= q.Wi) continue;
                  acc += x[off_x(&q, n, g, c, h, wi)] *
                         w[off_w(&q, g, k, c, ky, kx)];
                }
              }
            yout[off_y(&q, n, g, k, ho, wo)] = acc;
          }
  return 0;
}

/* Backward-data, gather form of the adjoint:
 * dX[n,g,c,hi,wi] = sum over k, and over taps (y,x) for which hi and wi lie
 * on the stride lattice of an in-range output (ho,wo), of
 * dY[n,g,k,ho,wo] * W[g,k,c,y,x].  Positions that no tap reaches get 0. */
int cbd_oracle_bwd_data(const int64_t* p, const double* dy, const double* w,
                        double* dx) {
  prob_t q;
  if (unpack(p, &q)) return -1;
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)(q.Cg ? q.Cg : 1));
#pragma omp for collapse(3) schedule(static)
    for (int64_t n = 0; n < q.N; n++)
      for (int64_t g = 0; g < q.G; g++)
        for (int64_t hi = 0; hi < q.Hi; hi++)
          for (int64_t wi = 0; wi < q.Wi; wi++) {
            for (int64_t c = 0; c < q.Cg; c++) acc[c] = 0.0;
            for (int64_t ky = 0; ky < q.Y; ky++) {
              int64_t ho = feeding_output(hi, ky, q.Sh, q.Ph, q.Dh, q.Ho);
              if (ho < 0) continue;
              for (int64_t kx = 0; kx < q.X; kx++) {
                int64_t wo = feeding_output(wi, kx, q.Sw, q.Pw, q.Dw, q.Wo);
                if (wo < 0) continue;
                for (int64_t k = 0; k < q.Kg; k++) {
                  double d = dy[off_y(&q, n, g, k, ho, wo)];
                  for (int64_t c = 0; c < q.Cg; c++)
                    acc[c] += d * w[off_w(&q, g, k, c, ky, kx)];
                }
              }
            }
            for (int64_t c = 0; c < q.Cg; c++)
              dx[off_x(&q, n, g, c, hi, wi)] = acc[c];
          }
    free(acc);
  }
  return 0;
}

/* The same definition evaluated at chosen positions only.  pts holds npts
 * quadruples (n, channel, hi, wi) with channel in [0, C). */
int cbd_oracle_bwd_data_at(const int64_t* p, const double* dy, const double* w,
                           int64_t npts, const int64_t* pts, double* out) {
  prob_t q;
  if (unpack(p, &q)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < npts; i++) {
    int64_t n = pts[4 * i], ch = pts[4 * i + 1];
    int64_t hi = pts[4 * i + 2], wi = pts[4 * i + 3];
    int64_t g = ch / q.Cg, c = ch % q.Cg;
    double acc = 0.0;
    for (int64_t ky = 0; ky < q.Y; ky++) {
      int64_t ho = feeding_output(hi, ky, q.Sh, q.Ph, q.Dh, q.Ho);
      if (ho < 0) continue;
      for (int64_t kx = 0; kx < q.X; kx++) {
        int64_t wo = feeding_output(wi, kx, q.Sw, q.Pw, q.Dw, q.Wo);
        if (wo < 0) continue;
        for (int64_t k = 0; k < q.Kg; k++)
          acc += dy[off_y(&q, n, g, k, ho, wo)] * w[off_w(&q, g, k, c, ky, kx)];
      }
    }
    out[i] = acc;
  }
  return 0;
}

/* Cross form: zero-insert dY, flip the filter, correlate.
 * Along each axis, dY is spread onto a zero line of length
 * L_in + D*(T-1) with stride S, starting at D*(T-1) - P (entries that land
 * outside the line are dropped); then
 *   dX[hi] = sum_t Z[hi + t*D] * W[T-1-t]
 * summed over k, i.e. a stride-1 correlation with the flipped, dilated
 * filter whose K and C roles are exchanged.  Written from the structure of
 * the BOO listing in fusilli issue #101 (flip of the x tap, insert_slice at
 * offset 1 with stride 2 into a 513-wide zero tensor, f32 contraction). */
int cbd_oracle_bwd_data_zero_insert(const int64_t* p, const double* dy,
                                    const double* w, double* dx,
                                    int64_t* z_geom) {
  prob_t q;
  if (unpack(p, &q)) return -1;
  int64_t Lh = q.Dh * (q.Y - 1) - q.Ph, Lw = q.Dw * (q.X - 1) - q.Pw;
  int64_t Hz = q.Hi + q.Dh * (q.Y - 1), Wz = q.Wi + q.Dw * (q.X - 1);
  if (z_geom) { z_geom[0] = Hz; z_geom[1] = Wz; z_geom[2] = Lh; z_geom[3] = Lw; }
  size_t zsz = (size_t)(q.N * q.K * Hz * Wz);
  double* z = (double*)calloc(zsz ? zsz : 1, sizeof(double));
  double* wf = (double*)malloc(sizeof(double) * (size_t)(q.G * q.Kg * q.Cg * q.Y * q.X + 1));
  if (!z || !wf) { free(z); free(wf); return -2; }
  /* Z is kept in [n][k_total][hz][wz] order, whatever the operand layout. */
  for (int64_t n = 0; n < q.N; n++)
    for (int64_t g = 0; g < q.G; g++)
      for (int64_t k = 0; k < q.Kg; k++)
        for (int64_t ho = 0; ho < q.Ho; ho++) {
          int64_t hz = Lh + ho * q.Sh;
          if (hz < 0 || hz >= Hz) continue;
          for (int64_t wo = 0; wo < q.Wo; wo++) {
            int64_t wz = Lw + wo * q.Sw;
            if (wz < 0 || wz >= Wz) continue;
            z[((n * q.K + g * q.Kg + k) * Hz + hz) * Wz + wz] =
                dy[off_y(&q, n, g, k, ho, wo)];
          }
        }
  /* Flipped filter wf[g][c][k][t_y][t_x] = W[g,k,c,Y-1-t_y,X-1-t_x]. */
  for (int64_t g = 0; g < q.G; g++)
    for (int64_t c = 0; c < q.Cg; c++)
      for (int64_t k = 0; k < q.Kg; k++)
        for (int64_t ty = 0; ty < q.Y; ty++)
          for (int64_t tx = 0; tx < q.X; tx++)
            wf[(((g * q.Cg + c) * q.Kg + k) * q.Y + ty) * q.X + tx] =
                w[off_w(&q, g, k, c, q.Y - 1 - ty, q.X - 1 - tx)];
#pragma omp parallel for collapse(3) schedule(static)
  for (int64_t n = 0; n < q.N; n++)
    for (int64_t g = 0; g < q.G; g++)
      for (int64_t c = 0; c < q.Cg; c++)
        for (int64_t hi = 0; hi < q.Hi; hi++)
          for (int64_t wi = 0; wi < q.Wi; wi++) {
            double acc = 0.0;
            for (int64_t k = 0; k < q.Kg; k++)
              for (int64_t ty = 0; ty < q.Y; ty++)
                for (int64_t tx = 0; tx < q.X; tx++)
                  acc += z[((n * q.K + g * q.Kg + k) * Hz + hi + ty * q.Dh) * Wz +
                           wi + tx * q.Dw] *
                         wf[(((g * q.Cg + c) * q.Kg + k) * q.Y + ty) * q.X + tx];
            dx[off_x(&q, n, g, c, hi, wi)] = acc;
          }
  free(z);
  free(wf);
  return 0;
}

/* Round double -> nearest fp32 (ties to even; the C conversion under the
 * default rounding mode). */
void cbd_oracle_round_f32(int64_t n, const double* in, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = (float)in[i];
}

/* Round fp32 -> bf16 (the upper half of an IEEE binary32), nearest with ties
 * to even: add half an ulp of the kept part, plus one more when the kept
 * part is odd, and drop the low 16 bits.  NaN inputs are kept quiet NaN. */
void cbd_oracle_round_bf16(int64_t n, const float* in, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) {
    uint32_t b;
    memcpy(&b, &in[i], 4);
    if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu)) {
      out[i] = (uint16_t)((b >> 16) | 0x0040u);
      continue;
    }
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7fffu + lsb;
    out[i] = (uint16_t)(b >> 16);
  }
}

int cbd_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
