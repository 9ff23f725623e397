// kern_nchw_rows.hip -- the row-block family: backward-data for NCHW / KCYX
// problems with few channels per group (the small fp32 problems of the
// rocMLIR PR #246 "Backward data" thread and their stride-2 relatives).
//
// The same stride-residue classes as the GEMM families drive the work
// (class (i_h, i_w) owns the taps i + T*j, serves the dX phase phi + S*t and
// reads dY row t + beta - delta*j), but a workgroup owns a block of whole dX
// rows instead of a GEMM tile:
//
//   workgroup = (image n, group g, 16-channel block c0, dX rows [h0, h1))
//
//   1. stage in LDS, once: the dY rows every class needs for these dX rows,
//      all K/G channels, with zero halo rows / columns where a tap falls off
//      dY's edge ([k][row][col], k planes padded so that the four k rows of
//      an MFMA operand fall on distinct banks); and all Y*X taps of W for
//      the 16 channels ([k][c*Y*X + tap], W's own order); zero the dX
//      staging tile;
//   2. every class's positions in these rows, in units of 16 consecutive
//      positions of one dX row: one 16x16 block (16 channels x 16 positions)
//      accumulated over (tap, k) with v_mfma_f32_16x16x4_f32 straight from
//      LDS; units go round-robin to the four waves, two at a time sharing
//      each W fragment, with the next k steps' fragments read while the
//      current ones multiply, four accumulators per unit (k step mod 4,
//      summed in a fixed order);
//   3. results land in the dX staging tile at their phase positions; after
//      a barrier the whole rows -- unreached phases included, as +0 -- leave
//      with the widest aligned stores.
//
// So a stride-2 problem writes complete, coalesced dX rows with no separate
// zero-fill launch, and the K loop never waits on global memory.  bf16
// operands are widened to f32 when staged (exact); results are rounded to
// the output dtype (nearest even) when stored.
#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int THREADS = kRowsThreads;  // 4 waves

template <int DT>
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (DT == 0) return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  return dev::bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// floor(a / b) for b > 0 and any a.
__device__ inline int floordiv(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

template <int DT>
__global__ __launch_bounds__(THREADS, 2) void nchw_rows_kernel(const GemmArgs a) {
  extern __shared__ float lds[];
  const RowsGeom& R = a.rg;
  constexpr uint32_t ES = DT == 0 ? 4 : 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Every kernel-argument line this kernel reads, fetched in one batch of
  // scalar loads (read at their first uses, each would wait on the one
  // before: block decode -> class descriptors -> staging geometry).
  {
    const int h0_ = a.N, h1_ = a.num_sub, h2_ = a.rg.rb, h3_ = a.rg.mag_chunks, h4_ = a.class_begin[8];
    const int h5_ = a.sub[0].phase_h, h6_ = a.sub[1].tile_begin, h7_ = a.sub[3].taps_w;
    const void* p0_ = a.dy;
    const void* p1_ = a.dx;
    asm volatile("" ::"s"(h0_), "s"(h1_), "s"(h2_), "s"(h3_), "s"(h4_), "s"(h5_), "s"(h6_), "s"(h7_), "s"(p0_),
                 "s"(p1_));
  }
  // ---- workgroup -> (n, g, row block, channel block)
  int b = blockIdx.x;
  const int cb = b % R.c_blocks;
  b /= R.c_blocks;
  const int rbk = b % R.row_blocks;
  b /= R.row_blocks;
  const int g = b % a.G;
  const int n = b / a.G;
  const int c0 = cb * 16;
  const int h0 = rbk * R.rb, h1 = min(h0 + R.rb, a.Hi);

  // First staged dY row: the lowest row any class reads for dX rows [h0, h1).
  int ho_lo = 0x7fffffff;
  for (int q = 0; q < a.num_sub; q++) {
    const SubDesc& s = a.sub[q];
    const int t_lo = max(0, floordiv(h0 - s.phase_h + a.Sh - 1, a.Sh));
    const int t_hi = min(s.pos_h - 1, floordiv(h1 - 1 - s.phase_h, a.Sh));
    if (t_lo <= t_hi) ho_lo = min(ho_lo, t_lo + s.beta_h - a.delta_h * (s.taps_h - 1));
  }
  if (ho_lo == 0x7fffffff) ho_lo = 0;

  float* const ydy = lds;               // [kg4][ks]: dY rows ho_lo ..., columns wo_lo ...
  float* const wt = lds + R.w_off;      // [kg4][ksw]: channel c, tap at c*Y*X + tap
  float* const st = lds + R.st_off;     // [16][cst]: dX rows h0 ... (row r at r*Wi)

  // dX staging tile to zero (unreached positions stay +0).
  for (int i = tid * 4; i < 16 * R.cst; i += THREADS * 4) *(f32x4*)(st + i) = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- 1. staging.  Every load is issued before any is written to LDS
  // (one memory latency, not one per element).  dY: wave w stages the k
  // planes k = w (mod 4); a lane's elements of a plane (chunks of 64) and
  // whether each lies inside dY are the same for every plane, so they are
  // worked out once.
  const int YX = a.Y * a.X;
  // W, when the block's 16 channels are whole (C/G % 16 == 0): the 16*Y*X
  // values of a filter row k are contiguous, read with 16-byte loads in
  // memory order.  Issued before the dY loads so that both batches are in
  // flight together.
  const bool wvec = DT == 0 && R.wvec;
  f32x4 vw[kRowsMaxWLoads];
  const int w_per_k = 4 * YX;  // 16-byte pieces per filter row
  const int w_total = R.kg4 * w_per_k;
  if (wvec) {
    const auto rw = dev::rsrc(a.w, a.w_bytes);
#pragma unroll
    for (int i = 0; i < kRowsMaxWLoads; i++) {
      const int v = tid + i * THREADS;
      const int k = v / w_per_k, r = v - (v / w_per_k) * w_per_k;
      const bool ok = v < w_total && k < a.Kg;
      const uint32_t off = ok ? (uint32_t)(((g * a.Kg + k) * a.Cg + c0) * YX) * ES + (uint32_t)r * 16u : dev::kOOB;
      if (i * THREADS < w_total)
        vw[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    }
  }
  float vy[kRowsMaxDyLoads];
  {
    const auto rdy = dev::rsrc(a.dy, a.dy_bytes);
    const int F = R.nr * R.rw;
    const int planes = R.kg4 >> 2;
    int goff[kRowsMaxChunks];
    bool inb[kRowsMaxChunks];
#pragma unroll
    for (int c = 0; c < kRowsMaxChunks; c++) {
      const int f = c * 64 + lane;
      const int row = f / R.rw, col = f - (f / R.rw) * R.rw;
      const int ho = ho_lo + row, wo = R.wo_lo + col;
      inb[c] = c < R.nch && f < F && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
      goff[c] = ho * a.Wo + wo;
    }
    const int kbase = (n * a.K + g * a.Kg) * a.Ho * a.Wo;
#pragma unroll
    for (int i = 0; i < kRowsMaxDyLoads; i++) {
      const int pl = i / kRowsMaxChunks, c = i % kRowsMaxChunks;
      const int k = wave + 4 * pl;
      if (pl < planes && c < R.nch) {
        const bool ok = inb[c] && k < a.Kg;
        vy[i] = load_elem<DT>(rdy, ok ? (uint32_t)(kbase + k * a.Ho * a.Wo + goff[c]) * ES : dev::kOOB);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsMaxDyLoads; i++) {
      const int pl = i / kRowsMaxChunks, c = i % kRowsMaxChunks;
      const int k = wave + 4 * pl;
      const int f = c * 64 + lane;
      if (pl < planes && c < R.nch && f < F) ydy[k * R.ks + f] = vy[i];
    }
  }
  if (wvec) {
#pragma unroll
    for (int i = 0; i < kRowsMaxWLoads; i++) {
      const int v = tid + i * THREADS;
      const int k = v / w_per_k, r = v - (v / w_per_k) * w_per_k;
      if (v < w_total) *(f32x4*)(wt + k * R.ksw + 4 * r) = vw[i];
    }
  } else {
    const auto rw = dev::rsrc(a.w, a.w_bytes);
    const int per_k = 16 * YX;
    const int total = R.kg4 * per_k;
    for (int e0 = tid; e0 < total; e0 += 8 * THREADS) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int e = e0 + i * THREADS;
        const int k = e / per_k, r = e - (e / per_k) * per_k;  // r = c*Y*X + tap
        const bool ok = e < total && k < a.Kg && c0 + r / YX < a.Cg;
        v[i] = load_elem<DT>(rw, ok ? (uint32_t)(((g * a.Kg + k) * a.Cg + c0) * YX + r) * ES : dev::kOOB);
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int e = e0 + i * THREADS;
        const int k = e / per_k, r = e - (e / per_k) * per_k;
        if (e < total) wt[k * R.ksw + r] = v[i];
      }
    }
  }
  __syncthreads();

  // ---- 2. units: (class, dX row of the class's phase in [h0, h1), 16
  // positions), round-robin over the waves in class order; a wave takes its
  // units of a class two at a time (units i and i + 4), which share every W
  // fragment.  Per tap the k steps go in groups of four with the next
  // group's fragments read while this group's MFMAs run; each unit keeps
  // four accumulators (k step mod 4, summed in a fixed order).
  const int kq = R.kg4 >> 2;  // k steps of 4, a multiple of 4
  const int lk = lane >> 4, ln = lane & 15;
  const int ks4 = 4 * R.ks, kw4 = 4 * R.ksw;
  int u = 0;
  for (int q = 0; q < a.num_sub; q++) {
    const SubDesc s = a.sub[q];
    const int t_lo = max(0, floordiv(h0 - s.phase_h + a.Sh - 1, a.Sh));
    const int t_hi = min(s.pos_h - 1, floordiv(h1 - 1 - s.phase_h, a.Sh));
    if (t_lo > t_hi) continue;
    const int ncol = (s.pos_w + 15) >> 4;
    const int units = (t_hi - t_lo + 1) * ncol;
    for (int i = (wave - u) & 3; i < units; i += 8) {
      const bool two = i + 4 < units;
      const int i1 = two ? i + 4 : i;
      const int tr0 = i / ncol, j0 = i - tr0 * ncol;
      const int tr1 = i1 / ncol, j1 = i1 - tr1 * ncol;
      const int th0 = t_lo + tr0, th1 = t_lo + tr1;
      f32x4 p[4] = {}, r[4] = {};  // unit 0, unit 1: accumulators by k step mod 4
      for (int jh = 0; jh < s.taps_h; jh++) {
        const int row0 = th0 + s.beta_h - a.delta_h * jh - ho_lo;  // in [0, nr)
        const int row1 = th1 + s.beta_h - a.delta_h * jh - ho_lo;
        const float* yr0 = ydy + lk * R.ks + row0 * R.rw + 16 * j0 + s.beta_w - R.wo_lo + ln;
        const float* yr1 = ydy + lk * R.ks + row1 * R.rw + 16 * j1 + s.beta_w - R.wo_lo + ln;
        for (int jw = 0; jw < s.taps_w; jw++) {
          const int tap = (s.cls_h + a.tstep_h * jh) * a.X + s.cls_w + a.tstep_w * jw;
          const float* y0 = yr0 - a.delta_w * jw;
          const float* y1 = yr1 - a.delta_w * jw;
          const float* wp = wt + lk * R.ksw + ln * YX + tap;
          // kq is a multiple of 4 (K/G padded to 16): every group is whole.
          // The next group's fragments are read before this group's MFMAs;
          // past the last group the read repeats the last group (unused).
          float fa[4], fb0[4], fb1[4];
#pragma unroll
          for (int v = 0; v < 4; v++) {
            fa[v] = wp[v * kw4];
            fb0[v] = y0[v * ks4];
            fb1[v] = y1[v * ks4];
          }
          for (int kb = 0; kb < kq; kb += 4) {
            const int nb = min(kb + 4, kq - 4);
            float na[4], nb0[4], nb1[4];
#pragma unroll
            for (int v = 0; v < 4; v++) {
              na[v] = wp[(nb + v) * kw4];
              nb0[v] = y0[(nb + v) * ks4];
              nb1[v] = y1[(nb + v) * ks4];
            }
#pragma unroll
            for (int v = 0; v < 4; v++) {
              p[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[v], fb0[v], p[v], 0, 0, 0);
              r[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[v], fb1[v], r[v], 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 4; v++) {
              fa[v] = na[v];
              fb0[v] = nb0[v];
              fb1[v] = nb1[v];
            }
          }
        }
      }
      // D[m = channel 4*lk + v][n = position 16j + ln]
      const f32x4 r0 = (p[0] + p[1]) + (p[2] + p[3]), r1 = (r[0] + r[1]) + (r[2] + r[3]);
      const int tw0 = 16 * j0 + ln, tw1 = 16 * j1 + ln;
      if (tw0 < s.pos_w) {
        float* dst = st + (s.phase_h + a.Sh * th0 - h0) * a.Wi + s.phase_w + a.Sw * tw0;
#pragma unroll
        for (int v = 0; v < 4; v++) dst[(4 * lk + v) * R.cst] = r0[v];
      }
      if (two && tw1 < s.pos_w) {
        float* dst = st + (s.phase_h + a.Sh * th1 - h0) * a.Wi + s.phase_w + a.Sw * tw1;
#pragma unroll
        for (int v = 0; v < 4; v++) dst[(4 * lk + v) * R.cst] = r1[v];
      }
    }
    u += units;
  }
  __syncthreads();

  // ---- 3. whole dX rows out: channel c, row r, chunk of vb bytes.
  {
    const auto rdx = dev::rsrc(a.dx, a.dx_bytes);
    const int eps = R.vb / (int)ES;          // elements per store
    const uint32_t chunks = (uint32_t)(a.Wi / eps);
    const uint32_t per_c = (uint32_t)R.rb * chunks;
    const uint32_t total = 16u * per_c;
    const int nrows = h1 - h0;
    for (uint32_t e = tid; e < total; e += THREADS) {
      const uint32_t c = dev::fdiv(e, per_c, R.mag_perc);
      const uint32_t rem = e - c * per_c;
      const uint32_t r = dev::fdiv(rem, chunks, R.mag_chunks);
      const uint32_t ch = rem - r * chunks;
      const bool ok = (int)r < nrows && c0 + (int)c < a.Cg;
      const uint32_t off =
          ok ? (uint32_t)((((n * a.C + g * a.Cg + c0 + (int)c) * a.Hi + h0 + (int)r) * a.Wi) + (int)ch * eps) * ES
             : dev::kOOB;
      const float* src = st + c * (uint32_t)R.cst + r * (uint32_t)a.Wi + ch * (uint32_t)eps;
      if constexpr (DT == 0) {
        if (R.vb == 16) {
          const f32x4 v = *(const f32x4*)src;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), rdx, off, 0, 0);
        } else if (R.vb == 8) {
          __builtin_amdgcn_raw_buffer_store_b64(u2{__float_as_uint(src[0]), __float_as_uint(src[1])}, rdx, off, 0,
                                                0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(src[0]), rdx, off, 0, 0);
        }
      } else {
        if (R.vb == 16) {
          const u4 v = {dev::bf16_pack2(src[0], src[1]), dev::bf16_pack2(src[2], src[3]),
                        dev::bf16_pack2(src[4], src[5]), dev::bf16_pack2(src[6], src[7])};
          __builtin_amdgcn_raw_buffer_store_b128(v, rdx, off, 0, 0);
        } else if (R.vb == 8) {
          __builtin_amdgcn_raw_buffer_store_b64(u2{dev::bf16_pack2(src[0], src[1]), dev::bf16_pack2(src[2], src[3])},
                                                rdx, off, 0, 0);
        } else if (R.vb == 4) {
          __builtin_amdgcn_raw_buffer_store_b32(dev::bf16_pack2(src[0], src[1]), rdx, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)dev::bf16_rne(src[0]), rdx, off, 0, 0);
        }
      }
    }
  }
}

}  // namespace

int launch_nchw_rows(const GemmArgs& a, int dtype, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  const void* k = dtype == CBD_F32 ? (const void*)&nchw_rows_kernel<0> : (const void*)&nchw_rows_kernel<1>;
  return (int)hipLaunchKernel(k, dim3((unsigned)grid), dim3(THREADS), args, (size_t)a.rg.lds_bytes,
                              (hipStream_t)stream);
}

}  // namespace cbd
