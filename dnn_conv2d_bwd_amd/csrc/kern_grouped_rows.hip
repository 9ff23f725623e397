// kern_grouped_rows.hip -- grouped backward-data with C/G == K/G in {1, 2, 4}
// (ResNeXt-style 32 groups of 4 is the motivating shape), one workgroup per
// output row of a stride-residue class.
//
// Per class the work is the same direct sum as kern_grouped_direct.hip (tap
// j of class position t reads dY row t + beta - delta*j), reorganised so
// that the kernel is bound by moving dY and dX, not by address arithmetic:
//   * the workgroup stages the class's taps_h dY rows it needs -- each a
//     contiguous run of pos_w + delta_w*(taps_w-1) NHWC pixels, all G groups
//     -- into LDS with 16-byte coalesced loads (taps off dY's edge read 0);
//   * lane = group (G divides 256), slot = tid / G; a slot walks the row's
//     positions tw = slot, slot + slots, ... so one wave's LDS reads and dX
//     stores cover whole contiguous pixel rows;
//   * the lane keeps its group's filter slice for the class's taps (<= 9)
//     in registers; in bf16 as (k, k+1) pairs so one v_dot2_f32_bf16 does
//     two multiply-adds with f32 accumulation straight from packed dY;
//   * rows are dealt to the 8 XCDs in chunks of 8 consecutive rows, so the
//     dY rows shared by neighbouring output rows meet in one L2.
#include "cbd_device.h"
#include "cbd_internal.h"
#include "grouped_vec.h"

namespace cbd {
namespace {

using namespace grp;

template <int DT, int CG>
__global__ __launch_bounds__(kGroupedThreads) void grouped_rows_kernel(const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char rows[];
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int VB = CG * ES;  // bytes of one group's channels at one pixel
  constexpr int MT = kGroupedMaxTaps;
  constexpr bool DOT2 = DT == 1 && CG >= 2;

  dev::prefetch_args(a);
  const int tid = threadIdx.x;
  const int G = a.G;
  const int g = tid & (G - 1);
  const int slot = tid / G;
  const int slots = kGroupedThreads / G;

  const int row = dev::chunked_block(blockIdx.x, a.total_tiles);
  const SubDesc s = a.sub[dev::find_class(a, row)];
  const int local = row - s.tile_begin;
  const int n = local / s.pos_h;
  const int th = local - n * s.pos_h;
  const int span = a.delta_w * (s.taps_w - 1);
  const int cols = s.pos_w + span;
  const int col0 = s.beta_w - span;  // dY column held in LDS column 0
  const int pixb = a.C * ES;         // bytes of one NHWC pixel (multiple of 16)
  const int rowb = cols * pixb;
  const int cshift = __builtin_ctz(pixb >> 4);  // 16-byte chunks per pixel = 2^cshift

  const auto rdy = dev::rsrc(a.dy, a.dy_bytes);
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);

  // ---- stage dY rows th + beta_h - delta_h*jh, columns col0 .. col0+cols-1.
  for (int jh = 0; jh < s.taps_h; jh++) {
    const int ho = th + s.beta_h - a.delta_h * jh;
    const bool hok = ho >= 0 && ho < a.Ho;
    const int rpix = (n * a.Ho + ho) * a.Wo;
    for (int i = tid; i < (cols << cshift); i += kGroupedThreads) {
      const int col = i >> cshift;
      const int wo = col0 + col;
      const bool ok = hok && wo >= 0 && wo < a.Wo;
      const uint32_t off =
          ok ? (uint32_t)(rpix + wo) * (uint32_t)pixb + (uint32_t)((i - (col << cshift)) << 4) : dev::kOOB;
      *(u4*)(rows + jh * rowb + (i << 4)) = __builtin_amdgcn_raw_buffer_load_b128(rdy, off, 0, 0);
    }
  }

  // ---- the group's filter slice for this class's taps.
  const int ntaps = s.taps_h * s.taps_w;
  const int YX = a.Y * a.X;
  float wr[DOT2 ? 1 : MT][DOT2 ? 1 : CG][CG];          // [tap][k][c], f32 path
  uint32_t wp[DOT2 ? MT : 1][CG][DOT2 ? CG / 2 : 1];   // [tap][c][k pair], bf16 pairs
  int toff[MT];  // LDS byte offset of tap tp relative to column tw
#pragma unroll
  for (int tp = 0; tp < MT; tp++) {
    const bool on = tp < ntaps;
    const int jh = on ? tp / s.taps_w : 0;
    const int jw = on ? tp - jh * s.taps_w : 0;
    const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
    toff[tp] = jh * rowb + (span - a.delta_w * jw) * pixb + g * VB;
    Vec<VB> wv[CG];
#pragma unroll
    for (int k = 0; k < CG; k++)
      wv[k] = load_vec<VB>(rw, on ? (uint32_t)(((g * CG + k) * YX + ty * a.X + tx) * CG) * ES : dev::kOOB);
    if constexpr (DOT2) {
#pragma unroll
      for (int c = 0; c < CG; c++)
#pragma unroll
        for (int kp = 0; kp < CG / 2; kp++) {
          const uint32_t lo = (wv[2 * kp].w[c >> 1] >> (16 * (c & 1))) & 0xffffu;
          const uint32_t hi = (wv[2 * kp + 1].w[c >> 1] >> (16 * (c & 1))) & 0xffffu;
          wp[tp][c][kp] = lo | (hi << 16);
        }
    } else {
#pragma unroll
      for (int k = 0; k < CG; k++)
#pragma unroll
        for (int c = 0; c < CG; c++)
          wr[tp][k][c] = DT == 0 ? __uint_as_float(wv[k].w[c])
                                 : dev::bf16_to_f32((wv[k].w[c >> 1] >> (16 * (c & 1))) & 0xffffu);
    }
  }
  __syncthreads();

  // ---- positions of the row.
  const int hi = s.phase_h + a.Sh * th;
  const uint32_t xrow = (uint32_t)((n * a.Hi + hi) * a.Wi) * (uint32_t)pixb + (uint32_t)(g * VB);
  for (int tw = slot; tw < s.pos_w; tw += slots) {
    float acc[CG];
#pragma unroll
    for (int c = 0; c < CG; c++) acc[c] = 0.f;
    const char* base = rows + tw * pixb;
#pragma unroll
    for (int tp = 0; tp < MT; tp++) {
      if (tp < ntaps) {
        const Vec<VB> v = lds_vec<VB>(base + toff[tp]);
        if constexpr (DOT2) {
#pragma unroll
          for (int c = 0; c < CG; c++)
#pragma unroll
            for (int kp = 0; kp < CG / 2; kp++)
              acc[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w[kp]),
                                                       __builtin_bit_cast(bf16x2_t, wp[tp][c][kp]),
                                                       acc[c], false);
        } else {
#pragma unroll
          for (int k = 0; k < CG; k++) {
            const float d = DT == 0 ? __uint_as_float(v.w[k])
                                    : dev::bf16_to_f32((v.w[k >> 1] >> (16 * (k & 1))) & 0xffffu);
#pragma unroll
            for (int c = 0; c < CG; c++) acc[c] = __builtin_fmaf(d, wr[tp][k][c], acc[c]);
          }
        }
      }
    }
    Vec<VB> o;
    if constexpr (DT == 0) {
#pragma unroll
      for (int c = 0; c < CG; c++) o.w[c] = __float_as_uint(acc[c]);
    } else if constexpr (CG == 1) {
      o.w[0] = dev::bf16_rne(acc[0]);
    } else {
#pragma unroll
      for (int c = 0; c < CG; c += 2) o.w[c >> 1] = dev::bf16_pack2(acc[c], acc[c + 1]);
    }
    const int wi = s.phase_w + a.Sw * tw;
    store_vec<VB>(rdx, xrow + (uint32_t)(wi * pixb), o);
  }
}

template <int DT, int CG>
int launch_one(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_rows_kernel<DT, CG>, dim3((unsigned)grid),
                              dim3(kGroupedThreads), args, (size_t)a.grp_lds, (hipStream_t)stream);
}

template <int DT>
int launch_dt(const GemmArgs& a, int64_t grid, void* stream) {
  switch (a.Cg) {
    case 1: return launch_one<DT, 1>(a, grid, stream);
    case 2: return launch_one<DT, 2>(a, grid, stream);
    case 4: return launch_one<DT, 4>(a, grid, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_grouped_rows(const GemmArgs& a, int dtype, int64_t grid, void* stream) {
  return dtype == CBD_F32 ? launch_dt<0>(a, grid, stream) : launch_dt<1>(a, grid, stream);
}

}  // namespace cbd
