// kern_grouped_pipe.hip -- grouped backward-data with C/G == K/G in {1, 2, 4}
// for classes whose taps step one dY row at a time (delta_h == 1, i.e.
// dilation 1 or gcd(stride, dilation) == dilation): one workgroup walks R
// consecutive output rows of one class and image, keeping the dY rows in
// an LDS ring.
//
// Output row t of a class reads dY rows t + beta_h - j (j < taps_h); row
// t+1 needs one new dY row and drops one.  Ring slot of dY row h = h mod
// (taps_h + 1).  Iteration t: wait for row t + beta_h, barrier (every wave
// is done with row t-1, whose oldest dY row's slot is free), start the
// global -> LDS copy of row t + 1 + beta_h into that slot, then compute row t
// from the other taps_h slots while the copy flies.  The copy is
// buffer_load ... lds (no VGPRs): each wave issues the same number of
// 64 x 16-byte instructions per row (rows padded to 4 KiB), so the wait is
// a fixed vmcnt.  Columns and rows off dY's edge load as zeros.
//
// Compute as in kern_grouped_rows.hip: lane = group, filter slice in
// registers (bf16 as k pairs for v_dot2_f32_bf16), positions strided over
// the workgroup's slots so one wave's LDS reads and dX stores cover whole
// pixel rows.
#include "cbd_device.h"
#include "cbd_internal.h"
#include "grouped_vec.h"

namespace cbd {
namespace {

using namespace grp;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One group's output channels at one position: sum over the class's NT taps
// of the staged dY vector times the filter slice.
template <int DT, int CG, int NT, int VB, typename WP, typename WR>
__device__ __forceinline__ void dot_taps(const Vec<VB> (&v)[NT], const WP& wp, const WR& wr,
                                         float (&acc)[CG]) {
  constexpr bool DOT2 = DT == 1 && CG >= 2;
#pragma unroll
  for (int c = 0; c < CG; c++) acc[c] = 0.f;
#pragma unroll
  for (int tp = 0; tp < NT; tp++) {
    if constexpr (DOT2) {
#pragma unroll
      for (int c = 0; c < CG; c++)
#pragma unroll
        for (int kp = 0; kp < CG / 2; kp++)
          acc[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v[tp].w[kp]),
                                                   __builtin_bit_cast(bf16x2_t, wp[tp][c][kp]),
                                                   acc[c], false);
    } else {
#pragma unroll
      for (int k = 0; k < CG; k++) {
        const float d = DT == 0 ? __uint_as_float(v[tp].w[k])
                                : dev::bf16_to_f32((v[tp].w[k >> 1] >> (16 * (k & 1))) & 0xffffu);
#pragma unroll
        for (int c = 0; c < CG; c++) acc[c] = __builtin_fmaf(d, wr[tp][k][c], acc[c]);
      }
    }
  }
}

template <int DT, int CG>
__device__ __forceinline__ Vec<CG * (DT == 0 ? 4 : 2)> pack_out(const float (&acc)[CG]) {
  Vec<CG * (DT == 0 ? 4 : 2)> o;
  if constexpr (DT == 0) {
#pragma unroll
    for (int c = 0; c < CG; c++) o.w[c] = __float_as_uint(acc[c]);
  } else if constexpr (CG == 1) {
    o.w[0] = dev::bf16_rne(acc[0]);
  } else {
#pragma unroll
    for (int c = 0; c < CG; c += 2) o.w[c >> 1] = dev::bf16_pack2(acc[c], acc[c + 1]);
  }
  return o;
}

// Per-workgroup constants of one (class, image, row block).
struct PipeCtx {
  int n, th0, th1;
  int span, col0, pixb, pshift, rowb, ni, slotb, nslot;
  int g, slot, slots, wave, lane;
};

// The workgroup's rows for a class of NT = taps_h * taps_w taps.  NT is a
// template parameter so that the tap loop unrolls without per-tap branches:
// every LDS read of a position is issued before the first multiply-add.
template <int DT, int CG, int NT>
__device__ __forceinline__ void pipe_rows(const GemmArgs& a, const SubDesc& s, const PipeCtx& q,
                                          char* ring) {
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int VB = CG * ES;
  constexpr bool DOT2 = DT == 1 && CG >= 2;
  constexpr int KP = CG / 2 > 0 ? CG / 2 : 1;
  // Two positions per pass, except f32 with 4 channels (its filter slice
  // alone takes up to 144 registers).
  constexpr bool PAIR = !(DT == 0 && CG == 4);

  const i32x4 dyd = {(int)(uint32_t)(uintptr_t)a.dy, (int)(((uintptr_t)a.dy >> 32) & 0xffff),
                     (int)a.dy_bytes, 0x00020000};
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;

  // Copy dY row ho (zeros off the edge) into its ring slot: each wave issues
  // exactly ni instructions of 64 lanes x 16 bytes.
  auto copy_row = [&](int ho, int sl) {
    const bool hok = ho >= 0 && ho < a.Ho;
    const int rpix = (q.n * a.Ho + ho) * a.Wo;
    for (int i = 0; i < q.ni; i++) {
      const int b = (i << 12) + (q.wave << 10) + (q.lane << 4);  // byte of the staged row
      const int col = b >> q.pshift;
      const int wo = q.col0 + col;
      const bool ok = hok && b < q.rowb && wo >= 0 && wo < a.Wo;
      const uint32_t off = ok ? (uint32_t)(rpix + wo) * (uint32_t)q.pixb + (uint32_t)(b & (q.pixb - 1))
                              : dev::kOOB;
      const uint32_t m0v =
          __builtin_amdgcn_readfirstlane(ring_base + (uint32_t)(sl * q.slotb + (i << 12) + (q.wave << 10)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                   :: "s"(m0v), "v"(off), "s"(dyd) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  // Filter slice of the group for the class's taps.
  const int YX = a.Y * a.X;
  float wr[DOT2 ? 1 : NT][CG][CG];
  uint32_t wp[DOT2 ? NT : 1][CG][KP];
  int jhs[NT], qoff[NT];  // tap row; LDS byte offset of the tap's column relative to tw
#pragma unroll
  for (int tp = 0; tp < NT; tp++) {
    const int jh = tp / s.taps_w;
    const int jw = tp - jh * s.taps_w;
    const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
    jhs[tp] = jh;
    qoff[tp] = (q.span - a.delta_w * jw) * q.pixb + q.g * VB;
    Vec<VB> wv[CG];
#pragma unroll
    for (int k = 0; k < CG; k++)
      wv[k] = load_vec<VB>(rw, (uint32_t)(((q.g * CG + k) * YX + ty * a.X + tx) * CG) * ES);
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

  // Ring slot of dY row h: h mod nslot.  top = slot of row th + beta_h,
  // advanced by one (cyclically) per output row.
  int top = (q.th0 + s.beta_h) % q.nslot;
  if (top < 0) top += q.nslot;
  auto back = [&](int j) { return top - j < 0 ? top - j + q.nslot : top - j; };  // slot of row th+beta_h-j

  // Prologue: the taps_h rows of the first output row.
  for (int jh = s.taps_h - 1; jh >= 0; jh--) copy_row(q.th0 + s.beta_h - jh, back(jh));

  for (int th = q.th0; th < q.th1; th++) {
    // This wave's copies of row th + beta_h (and older) have landed and its
    // reads of row th-1 are done; the barrier makes both hold for every
    // wave.  The memory clobber keeps the compiler from moving LDS reads
    // across it.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int next = top + 1 == q.nslot ? 0 : top + 1;
    if (th + 1 < q.th1) copy_row(th + 1 + s.beta_h, next);
    const int hi = s.phase_h + a.Sh * th;
    const uint32_t xrow = (uint32_t)((q.n * a.Hi + hi) * a.Wi) * (uint32_t)q.pixb + (uint32_t)(q.g * VB);
    int soff[NT];
#pragma unroll
    for (int tp = 0; tp < NT; tp++) soff[tp] = back(jhs[tp]) * q.slotb + qoff[tp];
    if constexpr (PAIR) {
      // Two positions per pass (tw and tw + slots; the second clamped to a
      // valid column and its store dropped when past the row's end).
      for (int tw = q.slot; tw < s.pos_w; tw += 2 * q.slots) {
        const int tw2 = tw + q.slots;
        const bool two = tw2 < s.pos_w;
        const char* b0 = ring + (tw << q.pshift);
        const char* b1 = ring + ((two ? tw2 : tw) << q.pshift);
        Vec<VB> v0[NT], v1[NT];
#pragma unroll
        for (int tp = 0; tp < NT; tp++) {
          v0[tp] = lds_vec<VB>(b0 + soff[tp]);
          v1[tp] = lds_vec<VB>(b1 + soff[tp]);
        }
        float acc0[CG], acc1[CG];
        dot_taps<DT, CG, NT>(v0, wp, wr, acc0);
        dot_taps<DT, CG, NT>(v1, wp, wr, acc1);
        store_vec<VB>(rdx, xrow + ((uint32_t)(s.phase_w + a.Sw * tw) << q.pshift), pack_out<DT, CG>(acc0));
        store_vec<VB>(rdx, two ? xrow + ((uint32_t)(s.phase_w + a.Sw * tw2) << q.pshift) : dev::kOOB,
                      pack_out<DT, CG>(acc1));
      }
    } else {
      for (int tw = q.slot; tw < s.pos_w; tw += q.slots) {
        const char* b0 = ring + (tw << q.pshift);
        Vec<VB> v0[NT];
#pragma unroll
        for (int tp = 0; tp < NT; tp++) v0[tp] = lds_vec<VB>(b0 + soff[tp]);
        float acc0[CG];
        dot_taps<DT, CG, NT>(v0, wp, wr, acc0);
        store_vec<VB>(rdx, xrow + ((uint32_t)(s.phase_w + a.Sw * tw) << q.pshift), pack_out<DT, CG>(acc0));
      }
    }
    top = next;
  }
}

template <int DT, int CG>
__global__ __launch_bounds__(kGroupedThreads) void grouped_pipe_kernel(const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  constexpr int ES = DT == 0 ? 4 : 2;

  dev::prefetch_args(a);
  PipeCtx q;
  const int tid = threadIdx.x;
  q.lane = tid & 63;
  q.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  q.g = tid & (a.G - 1);
  q.slot = tid / a.G;
  q.slots = kGroupedThreads / a.G;

  // workgroup -> (class, image n, row block)
  const int t = dev::chunked_block(blockIdx.x, a.total_tiles);
  const SubDesc s = a.sub[dev::find_class(a, t)];
  const int R = a.grp_rows;
  const int blocks = (s.pos_h + R - 1) / R;
  const int local = t - s.tile_begin;
  q.n = local / blocks;
  q.th0 = (local - q.n * blocks) * R;
  q.th1 = q.th0 + R < s.pos_h ? q.th0 + R : s.pos_h;

  q.span = a.delta_w * (s.taps_w - 1);
  q.col0 = s.beta_w - q.span;
  q.pixb = a.C * ES;  // power of two, >= 16
  q.pshift = __builtin_ctz(q.pixb);
  q.rowb = (s.pos_w + q.span) * q.pixb;
  q.ni = __builtin_amdgcn_readfirstlane((q.rowb + 4095) >> 12);  // copy instructions per row
  q.slotb = q.ni << 12;
  q.nslot = s.taps_h + 1;

  static_assert(kGroupedMaxTaps == 9, "the switch below covers 1..9 taps");
  switch (s.taps_h * s.taps_w) {
    case 1: pipe_rows<DT, CG, 1>(a, s, q, ring); break;
    case 2: pipe_rows<DT, CG, 2>(a, s, q, ring); break;
    case 3: pipe_rows<DT, CG, 3>(a, s, q, ring); break;
    case 4: pipe_rows<DT, CG, 4>(a, s, q, ring); break;
    case 5: pipe_rows<DT, CG, 5>(a, s, q, ring); break;
    case 6: pipe_rows<DT, CG, 6>(a, s, q, ring); break;
    case 7: pipe_rows<DT, CG, 7>(a, s, q, ring); break;
    case 8: pipe_rows<DT, CG, 8>(a, s, q, ring); break;
    default: pipe_rows<DT, CG, kGroupedMaxTaps>(a, s, q, ring); break;
  }
}

template <int DT, int CG>
int launch_one(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_pipe_kernel<DT, CG>, dim3((unsigned)grid),
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

int launch_grouped_pipe(const GemmArgs& a, int dtype, int64_t grid, void* stream) {
  return dtype == CBD_F32 ? launch_dt<0>(a, grid, stream) : launch_dt<1>(a, grid, stream);
}

}  // namespace cbd
