// kern_igemm_generic.hip -- implicit-GEMM backward-data for any layout and
// dtype (the fallback family, and the family of the small fp32 problems).
// One launch covers every stride-residue class: each workgroup decodes
// (class, group, M-tile, N-tile) from its id.
//
// Per class (i_h, i_w) and group g the GEMM is
//   M = C/G (dX channel c), N = N*pos_h*pos_w (dX positions of the class's
//   phase lattice), K = (K/G) * taps_h * taps_w (dY channel k, tap j_h, j_w);
//   A[c][(j,k)] = W[g,k,c, cls_h + T_h*j_h, cls_w + T_w*j_w]
//   B[(j,k)][(n,t_h,t_w)] = dY[n,g,k, t_h + beta_h - delta_h*j_h,
//                                     t_w + beta_w - delta_w*j_w]  (0 off the edge)
//   dX[n,g,c, phase_h + S_h*t_h, phase_w + S_w*t_w] = (A*B)[c][(n,t_h,t_w)].
// The per-residue split is the stride handling the rocMLIR PR #246
// "Backward data" thread builds one kernel per gemm id for (and the v4r1
// backward-data strategy of MIOpen PR #272 names); here the ids are
// workgroup ranges of one grid.
//
// The problems this family serves are small: a workgroup's time is the
// chain of global-load latencies along K, not MFMA work.  So the K loop is
// split across the NW waves of a workgroup (4, or 8 for long K loops on small
// grids; wave w takes k tiles w, w+NW, ...),
// each wave computes the whole BM x BN tile from its own LDS staging area
// with v_mfma_f32_16x16x4_f32 and keeps the next tile's gathers in flight
// (register double buffer; no workgroup barrier inside the loop), and the
// four partial tiles are summed in a fixed order through LDS at the end
// (deterministic).  Tiles are 64, 32 or 16 on each side, chosen by the
// planner (32x32 unless 64-wide tiles still give every CU four workgroups;
// 16 rows for at most 16 channels per group); k tiles are 8 wide on tiles of
// up to 32x32, 16 on larger ones.  Operands are gathered
// element-wise with buffer loads (out-of-range -> 0: padding, ragged tiles,
// taps off dY's edge) and converted to f32; bf16 products are exact in f32.
// f32 KCYX classes whose taps in a filter row lie within three consecutive
// elements (3x3 filters at stride 1 or 2, among others) instead read W one
// filter row per two- or three-element load and run K tap by tap over k
// tiles of 4 (or 8) k rows ("row loads", below).
//
// Split-K (a plan with ksplit S >= 2, for grids too small to fill the GPU):
// the S workgroups of a tile are S consecutive logical tiles; workgroup sp
// takes k tiles [KT*sp/S, KT*(sp+1)/S) and writes its f32 partial tile to
// the caller's workspace; a second kernel sums the S partials in split
// order and writes dX.
#include "cbd_device.h"
#include "cbd_internal.h"
#include "cbd_geo.h"
#include "generic_shapes.h"

namespace cbd {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// Pins a select: keeps the compiler from turning `cond ? off : kOOB` into a
// branch around the load (which would also force vmcnt(0) at the joins).
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// One element at byte offset voff + soff (soff wave-uniform: the scalar
// offset of the buffer instruction), converted to f32.
template <int DT>
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  if constexpr (DT == 0) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  } else {
    return dev::bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
  }
}

// Two adjacent elements (lo at byte_off).
template <int DT>
__device__ inline void store_pair(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float lo, float hi) {
  if constexpr (DT == 0) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = {__float_as_uint(lo), __float_as_uint(hi)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(dev::bf16_pack2(lo, hi), r, byte_off, 0, 0);
  }
}

template <int DT>
__device__ inline void store_elem(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  if constexpr (DT == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)dev::bf16_rne(v), r, byte_off, 0, 0);
  }
}

// WID (2 or 3) consecutive f32 elements at byte offset voff + soff: one
// multi-element load per lane.
template <int WID>
__device__ inline void load_row(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float (&v)[WID]) {
  if constexpr (WID == 2) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
  } else {
    static_assert(WID == 3, "row loads are 2 or 3 elements");
    typedef uint32_t u3 __attribute__((ext_vector_type(3)));
    const u3 x = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z);
  }
}

// NS: the zero-insertion form (no residue split: each tap's dY index needs a
// divisibility test); otherwise a tap's dY index is the position plus a
// wave-uniform shift.
template <int DT, int LAYOUT, int BM, int BN, int NW, bool NS, class Geo>
__global__ __launch_bounds__(NW * 64, 2) void igemm_generic_kernel(const void* dy_p, const void* w_p, void* dx_p,
                                                                   const GemmArgs a) {
  constexpr int BK = generic_bk(BM, BN);    // 8 (32x32 tiles) or 16
  constexpr int THREADS = NW * 64;          // NW (4 or 8) waves, each its own k tiles
  constexpr int MB = BM / 16, NB = BN / 16;
  constexpr int AE = BK * BM / 64, BE = BK * BN / 64;  // gathers per lane per tile
  // k tiles in flight per wave: eight on the small-grid shapes (eight-wave
  // workgroups, 16x16 tiles), where one wave's chain of memory round trips
  // sets the time; two elsewhere, where the extra registers would cost
  // occupancy (measured: c1 4.97 -> 4.29 us and the 3x3 32-channel
  // problems 8.05 -> 7.73 us with eight; the stride-2 64-channel problems
  // 17.1 -> 18.0 and 7.5 -> 8.5 us).
  constexpr int DEPTH = (AE + BE <= 8 && (NW == 8 || BM * BN <= 256)) ? 8 : 2;
  constexpr int RED = (NW > 4 ? NW / 2 : 2) * BM * BN;  // NW/2 (at least two) partial tiles at a time
  constexpr int LDSF = RED;
  constexpr uint32_t ES = DT == 0 ? 4 : 2;
  __shared__ float lds[LDSF];

  if constexpr (!Geo::kStatic) dev::prefetch_args(a);
  const int N = Geo::N(a), C = Geo::C(a), K = Geo::K(a), Cg = Geo::Cg(a), Kg = Geo::Kg(a);
  const int Hi = Geo::Hi(a), Wi = Geo::Wi(a), Ho = Geo::Ho(a), Wo = Geo::Wo(a);
  const int Yf = Geo::Y(a), Xf = Geo::X(a), Sh = Geo::Sh(a), Sw = Geo::Sw(a);
  const int tstep_h = Geo::tstep_h(a), tstep_w = Geo::tstep_w(a);
  const int delta_h = Geo::delta_h(a), delta_w = Geo::delta_w(a);
  const int tiles_m = Geo::tiles_m(a), total_tiles = Geo::total_tiles(a);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control

  if ((int)blockIdx.x >= total_tiles) {  // zero-fill folded into this launch (four-wave plans)
    if constexpr (NW != 4) return;
    const FusedZero& z = a.fz;
    const auto rdx = dev::rsrc(dx_p, Geo::dx_bytes(a));
    const uint32_t base =
        (uint32_t)(blockIdx.x - total_tiles) * (kGenericThreads * kZeroItemsPerThread) + tid;
#pragma unroll
    for (int i = 0; i < kZeroItemsPerThread; i++) {
      const uint32_t item = base + (uint32_t)(i * kGenericThreads);
      if ((int64_t)item < z.total_items)
        dev::zero_item(rdx, z.layout, z.esize, z.chunk, z.C, z.Hi, z.Wi, z.Sh, z.Sw, z.reg,
                       z.num_regions, item);
    }
    return;
  }

  const int t = dev::logical_tile(blockIdx.x, total_tiles, Geo::xcd_remap(a));
  // (descriptor-driven: the class index selects the divisor reciprocals)
  const int ci = Geo::kStatic ? 0 : Geo::sub_index(a, t);
  const SubDesc s = Geo::kStatic ? Geo::sub(a, t) : Geo::sub_at(a, ci);
  const auto mg = Geo::mags(a, ci);
  const int npix_img = s.pos_h * s.pos_w;
  const int npos = N * npix_img;
  const int tiles_n = (npos + BN - 1) / BN;
  const int per_group = tiles_m * tiles_n;
  const int S = Geo::ksplit(a) > 1 ? Geo::ksplit(a) : 1;
  const int lt = t - s.tile_begin;
  const int local = S > 1 ? lt / S : lt;
  const int sp = lt - local * S;  // split index (0 without split-K)
  const int g = (int)Geo::div(ci, (uint32_t)local, (uint32_t)per_group, mg.pergroup);
  const int rem = local - g * per_group;
  const int mt = (int)Geo::div(0, (uint32_t)rem, (uint32_t)tiles_m, mg.tiles_m);
  const int m0 = (rem - mt * tiles_m) * BM;
  const int n0 = mt * BN;

  const int YX = Yf * Xf;
  const auto rdy = dev::rsrc(dy_p, Geo::dy_bytes(a));
  // W of this group only: k rows past K/G fall outside it and read 0.
  const uint32_t wg_bytes = (uint32_t)(Kg * Cg * YX) * ES;
  const auto rw = dev::rsrc((const char*)w_p + (size_t)__builtin_amdgcn_readfirstlane(g) * wg_bytes, wg_bytes);
  const auto rdx = dev::rsrc(dx_p, Geo::dx_bytes(a));

  const int kpt = (Kg + BK - 1) / BK;
  // Order of the class's K = (tap, k) pairs.  Classes of 1, 2 or 4 taps run
  // tap-fastest: element d = q4 + 4*ks of a k tile is tap d % T of k row
  // k0 + d / T, so a lane keeps one tap for the whole loop and the four
  // lanes of a channel read taps of one W block (KCYX: all taps of a
  // channel are contiguous) instead of four k rows of it.  Other classes
  // (and the zero-insertion form) run k-fastest within one tap per k tile.
  const int T = s.taps_h * s.taps_w;
  const bool tapfast = !NS && (T == 1 || T == 2 || T == 4);
  const int KT = tapfast ? (Kg * T + BK - 1) / BK : T * kpt;
  const int kbeg = S > 1 ? KT * sp / S : 0, kend = S > 1 ? KT * (sp + 1) / S : KT;  // this workgroup's k tiles

  // Gather roles, in the operand layout of v_mfma_f32_16x16x4_f32 (so the
  // gathered values feed the MFMAs directly, with no pass through LDS):
  // lane l holds A[m = l % 16][k = l / 16] and B[k = l / 16][n = l % 16] of
  // each 16 x 4 block.  A element (bm, ks): channel m0 + 16*bm + l % 16, k
  // row 4*ks + l / 16; B element (bn, ks): position n0 + 16*bn + l % 16, the
  // same k row.  Each lane's part of an address is fixed (A) or fixed per
  // tap (B); the k tile's part is wave-uniform and goes to the load's scalar
  // offset.
  constexpr int KS = BK / 4;  // k steps of 4 per k tile
  const int r16 = lane & 15, q4 = lane >> 4;
  const int a_ks = Cg * YX;  // W elements between k rows (both layouts)
  uint32_t a_lane[MB];
#pragma unroll
  for (int bm = 0; bm < MB; bm++) {
    const int c = m0 + 16 * bm + r16;
    a_lane[bm] = c < Cg ? (uint32_t)(LAYOUT == 0 ? (q4 * Cg + c) * YX : q4 * a_ks + c) * ES : dev::kOOB;
  }
  const int b_ks = LAYOUT == 0 ? Ho * Wo : 1;  // dY elements between k rows
  // Per 16-position block: the dY element of (k row q4, dY pixel (pth, ptw)
  // of image pn); a tap adds a wave-uniform pixel shift (times K for NHWC).
  int bpos[NB], pth[NB], ptw[NB];
  bool bp_ok[NB];
#pragma unroll
  for (int bn = 0; bn < NB; bn++) {
    const int bp = n0 + 16 * bn + r16;
    bp_ok[bn] = bp < npos;
    const int bpp = bp_ok[bn] ? bp : 0;
    const int pn = (int)Geo::div(ci, (uint32_t)bpp, (uint32_t)npix_img, mg.npix);
    const int prr = bpp - pn * npix_img;
    pth[bn] = (int)Geo::div(ci, (uint32_t)prr, (uint32_t)s.pos_w, mg.posw);
    ptw[bn] = prr - pth[bn] * s.pos_w;
    bpos[bn] = LAYOUT == 0 ? ((pn * K + g * Kg + q4) * Ho + pth[bn]) * Wo + ptw[bn]
                           : ((pn * Ho + pth[bn]) * Wo + ptw[bn]) * K + g * Kg + q4;
  }

  // k tile -> (k tile within its tap, tap row, tap column); advanced
  // without division (the walk is wave-uniform).
  struct Walk {
    int kk, jh, jw;
  };
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto walk_at = [&](int kt) {
    const int tap = kt / kpt;
    return Walk{uni(kt - tap * kpt), uni(tap / s.taps_w), uni(tap - (tap / s.taps_w) * s.taps_w)};
  };
  auto advance = [&](Walk& w, int n) {
    int kk = uni(w.kk) + n, jh = uni(w.jh), jw = uni(w.jw);
    while (kk >= kpt) {
      kk -= kpt;
      if (++jw == s.taps_w) {
        jw = 0;
        ++jh;
      }
    }
    w = Walk{kk, jh, jw};
  };

  auto gather = [&](const Walk& w, bool live, float (&av)[AE], float (&bv)[BE]) {
    const int k0 = w.kk * BK;
    const int tapoff = (s.cls_h + tstep_h * w.jh) * Xf + s.cls_w + tstep_w * w.jw;
    // (wave-uniform by construction; readfirstlane lets the compiler see it)
    const uint32_t a_s = __builtin_amdgcn_readfirstlane(
        (uint32_t)(LAYOUT == 0 ? k0 * a_ks + tapoff : (k0 * YX + tapoff) * Cg) * ES);
    const int krem = Kg - k0;  // k rows of this tile inside K/G
    int dh = 0, dw = 0;        // dY pixel shift of this tap (residue split)
    if constexpr (!NS) {
      dh = uni(s.beta_h - delta_h * w.jh);
      dw = uni(s.beta_w - delta_w * w.jw);
    }
#pragma unroll
    for (int bm = 0; bm < MB; bm++) {
      const uint32_t al = live ? a_lane[bm] : dev::kOOB;
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        av[bm * KS + ks] = load_elem<DT>(rw, opaque(al), a_s + (uint32_t)(4 * ks * a_ks) * ES);
    }
#pragma unroll
    for (int bn = 0; bn < NB; bn++) {
      bool bok;
      int shift;
      if constexpr (NS) {
        const int ho = dev::dy_index(1, pth[bn], s.beta_h, delta_h, w.jh, a.pad_h, a.dil_h, a.str_h);
        const int wo = dev::dy_index(1, ptw[bn], s.beta_w, delta_w, w.jw, a.pad_w, a.dil_w, a.str_w);
        bok = ho >= 0 && ho < Ho && wo >= 0 && wo < Wo;
        shift = LAYOUT == 0 ? (ho - pth[bn]) * Wo + (wo - ptw[bn]) : ((ho - pth[bn]) * Wo + (wo - ptw[bn])) * K;
      } else {
        bok = pth[bn] >= -dh && pth[bn] < Ho - dh && ptw[bn] >= -dw && ptw[bn] < Wo - dw;
        shift = LAYOUT == 0 ? dh * Wo + dw : (dh * Wo + dw) * K;
      }
      const uint32_t b_lane = (bok && live && bp_ok[bn]) ? (uint32_t)(bpos[bn] + shift) * ES : dev::kOOB;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const uint32_t off = q4 + 4 * ks < krem ? b_lane : dev::kOOB;
        bv[bn * KS + ks] = load_elem<DT>(rdy, opaque(off),
                                         __builtin_amdgcn_readfirstlane((uint32_t)((k0 + 4 * ks) * b_ks) * ES));
      }
    }
  };

  // Tap-fast gathers: the lane's tap tl and first k row kd0; per k step the
  // k row advances by 4 / T, per k tile by BK / T.
  const int tsh = T == 4 ? 2 : T == 2 ? 1 : 0;
  const int tl = q4 & (T - 1), kd0 = q4 >> tsh;
  const int kstep = 4 >> tsh, kpt_tf = BK >> tsh;
  uint32_t a_tf[MB], b_tf[NB];
  if (tapfast) {
    const int jh = tl / s.taps_w, jw = tl - (tl / s.taps_w) * s.taps_w;
    const int tapoff = (s.cls_h + tstep_h * jh) * Xf + s.cls_w + tstep_w * jw;
#pragma unroll
    for (int bm = 0; bm < MB; bm++) {
      const int c = m0 + 16 * bm + r16;
      a_tf[bm] = c < Cg ? (uint32_t)(LAYOUT == 0 ? (kd0 * Cg + c) * YX + tapoff : (kd0 * YX + tapoff) * Cg + c) * ES
                        : dev::kOOB;
    }
    const int dh = s.beta_h - delta_h * jh, dw = s.beta_w - delta_w * jw;
    const int shift = LAYOUT == 0 ? dh * Wo + dw : (dh * Wo + dw) * K;
#pragma unroll
    for (int bn = 0; bn < NB; bn++) {
      const bool bok = bp_ok[bn] && pth[bn] >= -dh && pth[bn] < Ho - dh && ptw[bn] >= -dw && ptw[bn] < Wo - dw;
      b_tf[bn] = bok ? (uint32_t)(bpos[bn] + (kd0 - q4) * b_ks + shift) * ES : dev::kOOB;
    }
  }
  // Tap-fast k tile kt: W rows past K/G read 0 through the group's
  // resource; dY rows past K/G are masked per lane.
  auto gather_tf = [&](int kt, float (&av)[AE], float (&bv)[BE]) {
    const int k0 = kt * kpt_tf;
    const uint32_t a_s = __builtin_amdgcn_readfirstlane((uint32_t)(k0 * a_ks) * ES);
    const int krem = Kg - k0;
#pragma unroll
    for (int bm = 0; bm < MB; bm++)
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        av[bm * KS + ks] = load_elem<DT>(rw, opaque(a_tf[bm]), a_s + (uint32_t)(ks * kstep * a_ks) * ES);
#pragma unroll
    for (int bn = 0; bn < NB; bn++)
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const uint32_t off = kd0 + ks * kstep < krem ? b_tf[bn] : dev::kOOB;
        bv[bn * KS + ks] = load_elem<DT>(
            rdy, opaque(off), __builtin_amdgcn_readfirstlane((uint32_t)((k0 + ks * kstep) * b_ks) * ES));
      }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < NB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const float (&av)[AE], const float (&bv)[BE]) {
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
      for (int bm = 0; bm < MB; bm++)
#pragma unroll
        for (int bn = 0; bn < NB; bn++)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[bm * KS + ks], bv[bn * KS + ks], acc[bm][bn],
                                                             0, 0, 0);
  };

  // Wave-strided K loop with up to DEPTH k tiles of gathers in flight (a
  // ring of registers; a slot is refilled right after its tile is used).
  // Tiles past this workgroup's k range are skipped, not gathered.
  auto kloop = [&](auto&& fetch) {
    float av[DEPTH][AE], bv[DEPTH][BE];
    int kn = kbeg + wave;  // next tile to gather
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      if (kn < kend) fetch(kn, av[d], bv[d]);
      kn += NW;
    }
    for (int kt = kbeg + wave; kt < kend; kt += DEPTH * NW) {
#pragma unroll
      for (int d = 0; d < DEPTH; d++) {
        if (kt + d * NW < kend) {
          compute(av[d], bv[d]);
          if (kn < kend) fetch(kn, av[d], bv[d]);
          kn += NW;
        }
      }
    }
  };
  // Row loads (f32 KCYX, residue split; classes whose taps in one filter
  // row lie within three consecutive elements): lane (channel c, k row q4)
  // reads the taps of one filter row of its W[k][c] block with a single
  // two- or three-element load, and K runs k-fastest within each tap:
  // k step (kg, t) of a k tile pairs W[k0 + 4kg + q4][c][tap t] with
  // dY[k0 + 4kg + q4][position shifted by tap t].  A single-element gather
  // whose lanes are Y*X elements apart costs the address path about 3.5x a
  // contiguous one, while a two- to four-element load costs 2x whatever its
  // pattern, so reading a row of taps per load cuts that work by 2.5-7x;
  // the dY gathers keep their contiguous 16-position runs.
  auto row_path = [&](auto th_c, auto tw_c, auto ts_c) {
    constexpr int TH = decltype(th_c)::value, TW = decltype(tw_c)::value, TS = decltype(ts_c)::value;
    constexpr int TT = TH * TW;
    constexpr int WID = TW == 1 ? 2 : (TW - 1) * TS + 1;  // elements per row load
    // k tiles in flight per wave: one on four-wave workgroups (64 VGPRs,
    // eight waves per SIMD: there that occupancy is worth more than a
    // second tile per wave, 11.2 against 12.0 us on the 64-channel
    // stride-2 problem); two on the two-wave workgroups the planner gives
    // grids of one- to four-tap classes (one cross-wave sum instead of two,
    // 92 VGPRs: 10.6 against 10.8 us shape-specialised, 13.0 against 13.7
    // descriptor-driven; three or four tiles were 10.9 and 11.4 us).
    constexpr int KG = TT <= 2 ? 2 : 1;       // groups of 4 k rows per k tile
    constexpr int RD = NW == 2 && TT <= 4 ? 2 : 1;
    const int KTr = (Kg + 4 * KG - 1) / (4 * KG);
    const int kb = S > 1 ? KTr * sp / S : 0, ke = S > 1 ? KTr * (sp + 1) / S : KTr;
    uint32_t wl[MB];
#pragma unroll
    for (int bm = 0; bm < MB; bm++) {
      const int c = m0 + 16 * bm + r16;
      wl[bm] = c < Cg ? (uint32_t)((q4 * Cg + c) * YX + s.cls_w) * ES : dev::kOOB;
    }
    uint32_t wrow[TH];
#pragma unroll
    for (int jh = 0; jh < TH; jh++) wrow[jh] = uni((s.cls_h + tstep_h * jh) * Xf * (int)ES);
    uint32_t bl[NB][TT];
#pragma unroll
    for (int bn = 0; bn < NB; bn++)
#pragma unroll
      for (int jh = 0; jh < TH; jh++)
#pragma unroll
        for (int jw = 0; jw < TW; jw++) {
          const int dh = s.beta_h - delta_h * jh, dw = s.beta_w - delta_w * jw;
          const bool ok = bp_ok[bn] && pth[bn] >= -dh && pth[bn] < Ho - dh && ptw[bn] >= -dw && ptw[bn] < Wo - dw;
          bl[bn][jh * TW + jw] = ok ? (uint32_t)(bpos[bn] + dh * Wo + dw) * ES : dev::kOOB;
        }
    float wv[RD][KG][MB][TH][WID], bv[RD][KG][NB][TT];
    auto fetch = [&](int kt, float (&w)[KG][MB][TH][WID], float (&b)[KG][NB][TT]) {
#pragma unroll
      for (int kg = 0; kg < KG; kg++) {
        const int k = (kt * KG + kg) * 4;
        const uint32_t a_s = uni(k * a_ks * (int)ES);
#pragma unroll
        for (int bm = 0; bm < MB; bm++)
#pragma unroll
          for (int jh = 0; jh < TH; jh++) load_row<WID>(rw, wl[bm], a_s + wrow[jh], w[kg][bm][jh]);
        const uint32_t b_s = uni(k * b_ks * (int)ES);
        if (Kg - k >= 4) {  // (wave-uniform) all four k rows inside K/G: the offsets as they are
#pragma unroll
          for (int bn = 0; bn < NB; bn++)
#pragma unroll
            for (int tt = 0; tt < TT; tt++) b[kg][bn][tt] = load_elem<DT>(rdy, bl[bn][tt], b_s);
        } else {  // dY rows past K/G read 0
          const bool kok = q4 < Kg - k;
#pragma unroll
          for (int bn = 0; bn < NB; bn++)
#pragma unroll
            for (int tt = 0; tt < TT; tt++)
              b[kg][bn][tt] = load_elem<DT>(rdy, opaque(kok ? bl[bn][tt] : dev::kOOB), b_s);
        }
      }
    };
    // Elements of a row load that no tap uses (the middle one of taps two
    // apart, the second one of a single tap): kept live until the tile's
    // MFMAs have issued, so that their registers are not handed to the next
    // load's operands while the load is still in flight (which would make
    // every following load wait for the previous one).
    auto keep_unused = [&](const float (&w)[KG][MB][TH][WID]) {
#pragma unroll
      for (int kg = 0; kg < KG; kg++)
#pragma unroll
        for (int bm = 0; bm < MB; bm++)
#pragma unroll
          for (int jh = 0; jh < TH; jh++)
#pragma unroll
            for (int e = 0; e < WID; e++)
              if (TW == 1 ? e != 0 : (e % TS != 0 || e / TS >= TW)) asm volatile("" ::"v"(w[kg][bm][jh][e]));
    };
    auto comp = [&](const float (&w)[KG][MB][TH][WID], const float (&b)[KG][NB][TT]) {
#pragma unroll
      for (int kg = 0; kg < KG; kg++)
#pragma unroll
        for (int jh = 0; jh < TH; jh++)
#pragma unroll
          for (int jw = 0; jw < TW; jw++)
#pragma unroll
            for (int bm = 0; bm < MB; bm++)
#pragma unroll
              for (int bn = 0; bn < NB; bn++)
                acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(w[kg][bm][jh][jw * TS], b[kg][bn][jh * TW + jw],
                                                                   acc[bm][bn], 0, 0, 0);
    };
    int kn = kb + wave;
#pragma unroll
    for (int d = 0; d < RD; d++) {
      if (kn < ke) fetch(kn, wv[d], bv[d]);
      kn += NW;
    }
    for (int kt = kb + wave; kt < ke; kt += RD * NW) {
#pragma unroll
      for (int d = 0; d < RD; d++) {
        if (kt + d * NW < ke) {
          comp(wv[d], bv[d]);
          keep_unused(wv[d]);
          if (kn < ke) fetch(kn, wv[d], bv[d]);
          kn += NW;
        }
      }
    }
  };
  int rpat = 0;  // row-load pattern of this class (0: none)
  if constexpr (DT == 0 && LAYOUT == 0 && !NS)
    rpat = uni(row_pattern(s.taps_h, s.taps_w, s.cls_w, Xf, tstep_w));
  constexpr int pats = MB * NB <= 4 ? Geo::kRowPats : 0;  // (larger tiles: registers)
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if ((pats & 2) && rpat == 1) {
    row_path(I1(), I1(), I0());
  } else if ((pats & 4) && rpat == 2) {
    row_path(I2(), I1(), I0());
  } else if ((pats & 8) && rpat == 3) {
    row_path(I1(), I2(), I2());
  } else if ((pats & 16) && rpat == 4) {
    row_path(I2(), I2(), I2());
  } else if ((pats & 32) && rpat == 5) {
    row_path(I3(), I3(), I1());
  } else if (tapfast) {
    kloop([&](int kt, float (&av)[AE], float (&bv)[BE]) { gather_tf(kt, av, bv); });
  } else {
    Walk wn = walk_at(kbeg + wave);  // walks in step with the tiles fetched
    kloop([&](int, float (&av)[AE], float (&bv)[BE]) {
      gather(wn, true, av, bv);
      advance(wn, NW);
    });
  }

  // Cross-wave sum in a fixed order through LDS (reusing the staging area):
  // a tree that halves the waves holding partial tiles, w += w + NW/2, ...,
  // down to two, (w0 + w2) + (w1 + w3) for four waves; the last sum is made
  // by the epilogue.
  auto red_at = [&](int slot, int bm, int bn, int v) -> float& {
    return lds[(slot * BM + bm * 16 + 4 * (lane >> 4) + v) * BN + bn * 16 + (lane & 15)];
  };
#pragma unroll
  for (int sr = NW / 2; sr >= 2; sr /= 2) {
    __syncthreads();
    if (wave >= sr && wave < 2 * sr) {
#pragma unroll
      for (int bm = 0; bm < MB; bm++)
#pragma unroll
        for (int bn = 0; bn < NB; bn++)
#pragma unroll
          for (int v = 0; v < 4; v++) red_at(wave - sr, bm, bn, v) = acc[bm][bn][v];
    }
    __syncthreads();
    if (wave < sr) {
#pragma unroll
      for (int bm = 0; bm < MB; bm++)
#pragma unroll
        for (int bn = 0; bn < NB; bn++)
#pragma unroll
          for (int v = 0; v < 4; v++) acc[bm][bn][v] += red_at(wave, bm, bn, v);
    }
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int bm = 0; bm < MB; bm++)
#pragma unroll
      for (int bn = 0; bn < NB; bn++)
#pragma unroll
        for (int v = 0; v < 4; v++) red_at(wave, bm, bn, v) = acc[bm][bn][v];
  }
  __syncthreads();

  if (S > 1) {  // split-K: the partial tile, row-major, at logical tile t
    float* const part = (float*)a.ws + (size_t)t * (BM * BN);
#pragma unroll
    for (int i = 0; i < BM * BN / THREADS; i++) {
      const int e = (tid / BN + (THREADS / BN) * i) * BN + tid % BN;
      part[e] = lds[e] + lds[BM * BN + e];
    }
    return;
  }

  // Epilogue: thread -> position n0 + tid % BN, channels tid / BN + (256/BN)*i.
  const int p = n0 + tid % BN;
  const bool pv = p < npos;
  const int pp = pv ? p : 0;
  const int n = (int)Geo::div(ci, (uint32_t)pp, (uint32_t)npix_img, mg.npix);
  const int rr = pp - n * npix_img;
  const int th = (int)Geo::div(ci, (uint32_t)rr, (uint32_t)s.pos_w, mg.posw), tw = rr - th * s.pos_w;
  const int hi = s.phase_h + Sh * th, wi = s.phase_w + Sw * tw;
  const int pbase = LAYOUT == 0 ? (n * C + g * Cg) * Hi * Wi + hi * Wi + wi
                                : ((n * Hi + hi) * Wi + wi) * C + g * Cg;
  const int cstride = LAYOUT == 0 ? Hi * Wi : 1;
  if (Geo::zblock(a)) {
    // One class at phase (0,0) over every S x S block: write the block,
    // the value at its corner and zeros at the unreached positions (in
    // element pairs along W for NCHW at stride 2 and an even width).
    const bool pairs = LAYOUT == 0 && Sw == 2 && (Wi & 1) == 0;
#pragma unroll
    for (int i = 0; i < BM * BN / THREADS; i++) {
      const int m = tid / BN + (THREADS / BN) * i;
      const float v = lds[m * BN + tid % BN] + lds[(BM + m) * BN + tid % BN];
      const int c = m0 + m;
      const bool ok = pv && c < Cg;
      const int e0 = pbase + c * cstride;
      if (pairs) {
        store_pair<DT>(rdx, ok ? (uint32_t)e0 * ES : dev::kOOB, v, 0.f);
        for (int dh = 1; dh < Sh; dh++)
          store_pair<DT>(rdx, (ok && hi + dh < Hi) ? (uint32_t)(e0 + dh * Wi) * ES : dev::kOOB, 0.f, 0.f);
      } else {
        for (int dh = 0; dh < Sh; dh++)
          for (int dw = 0; dw < Sw; dw++) {
            const int e = e0 + (LAYOUT == 0 ? dh * Wi + dw : (dh * Wi + dw) * C);
            store_elem<DT>(rdx, (ok && hi + dh < Hi && wi + dw < Wi) ? (uint32_t)e * ES : dev::kOOB,
                           (dh | dw) ? 0.f : v);
          }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < BM * BN / THREADS; i++) {
    const int m = tid / BN + (THREADS / BN) * i;
    const float v = lds[m * BN + tid % BN] + lds[(BM + m) * BN + tid % BN];
    const int c = m0 + m;
    store_elem<DT>(rdx, (pv && c < Cg) ? (uint32_t)(pbase + c * cstride) * ES : dev::kOOB, v);
  }
}

// Finalising kernel of a split-K plan: workgroup T sums the S partial tiles
// of tile T (logical tiles T*S .. T*S+S-1) in split order and writes them to
// dX as the main kernel's epilogue would.
template <int DT, int LAYOUT, int BM, int BN>
__global__ __launch_bounds__(256) void generic_finalize_kernel(const GemmArgs a) {
  constexpr uint32_t ES = DT == 0 ? 4 : 2;
  const int tid = threadIdx.x;
  const int S = a.ksplit;
  const int t0 = blockIdx.x * S;
  const SubDesc s = a.sub[dev::find_class(a, t0)];
  const int npix_img = s.pos_h * s.pos_w;
  const int npos = a.N * npix_img;
  const int tiles_n = (npos + BN - 1) / BN;
  const int per_group = a.tiles_m * tiles_n;
  const int local = (t0 - s.tile_begin) / S;
  const int g = local / per_group;
  const int rem = local - g * per_group;
  const int m0 = (rem % a.tiles_m) * BM;
  const int n0 = (rem / a.tiles_m) * BN;

  const int p = n0 + tid % BN;
  const bool pv = p < npos;
  const int pp = pv ? p : 0;
  const int n = pp / npix_img;
  const int rr = pp - n * npix_img;
  const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
  const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
  const int pbase = LAYOUT == 0 ? (n * a.C + g * a.Cg) * a.Hi * a.Wi + hi * a.Wi + wi
                                : ((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg;
  const int cstride = LAYOUT == 0 ? a.Hi * a.Wi : 1;
  const float* const part = (const float*)a.ws + (size_t)t0 * (BM * BN);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);
#pragma unroll
  for (int i = 0; i < BM * BN / 256; i++) {
    const int m = tid / BN + (256 / BN) * i;
    const int e = m * BN + tid % BN;
    float v = 0.f;
    for (int q = 0; q < S; q++) v += part[(size_t)q * (BM * BN) + e];
    const int c = m0 + m;
    store_elem<DT>(rdx, (pv && c < a.Cg) ? (uint32_t)(pbase + c * cstride) * ES : dev::kOOB, v);
  }
}

template <int DT, int LAYOUT, int BM, int BN, int NW = 4>
int launch_one(const GemmArgs& a, int64_t grid, void* stream) {
  const void* dy = a.dy;
  const void* w = a.w;
  void* dx = a.dx;
  void* args[] = {&dy, &w, &dx, const_cast<GemmArgs*>(&a)};
  const void* k = a.no_split ? (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, true, DynGeo>
                             : (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, false, DynGeo>;
  if constexpr (DT == 0 && LAYOUT == 0 && BM * BN <= 1024) {
    // f32 KCYX: an instance compiled with only the row-load patterns the
    // classes need (any pattern it lacks runs the general K order).
    constexpr int kS2 = kRowPatsStride2, k33 = kRowPatsAll & ~kRowPatsStride2;
    const int rp = a.row_pats & kRowPatsAll;
    if constexpr (NW == 2) {
      if (!a.no_split && (rp & ~kS2) == 0 && rp != 0)
        k = (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, false, DynGeoRows<kS2>>;
      return (int)hipLaunchKernel(k, dim3((unsigned)grid), dim3(NW * 64), args, 0, (hipStream_t)stream);
    }
    if (!a.no_split) {
      if (rp == 0)
        k = (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, false, DynGeoRows<0>>;
      else if ((rp & ~kS2) == 0)
        k = (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, false, DynGeoRows<kS2>>;
      else if (rp == k33)
        k = (const void*)&igemm_generic_kernel<DT, LAYOUT, BM, BN, NW, false, DynGeoRows<k33>>;
    }
  }
  return (int)hipLaunchKernel(k,
                              dim3((unsigned)grid), dim3(NW * 64), args, 0,
                              (hipStream_t)stream);
}

template <int DT, int LAYOUT, int BM, int BN>
int launch_fin(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&generic_finalize_kernel<DT, LAYOUT, BM, BN>,
                              dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
}

template <int DT, int LAYOUT>
int launch_fin_tiles(const GemmArgs& a, int64_t grid, void* stream) {
  if (a.tile_m == 64 && a.tile_n == 64) return launch_fin<DT, LAYOUT, 64, 64>(a, grid, stream);
  if (a.tile_m == 32 && a.tile_n == 64) return launch_fin<DT, LAYOUT, 32, 64>(a, grid, stream);
  if (a.tile_m == 64 && a.tile_n == 32) return launch_fin<DT, LAYOUT, 64, 32>(a, grid, stream);
  if (a.tile_m == 32 && a.tile_n == 32) return launch_fin<DT, LAYOUT, 32, 32>(a, grid, stream);
  if (a.tile_m == 16 && a.tile_n == 32) return launch_fin<DT, LAYOUT, 16, 32>(a, grid, stream);
  if (a.tile_m == 16 && a.tile_n == 16) return launch_fin<DT, LAYOUT, 16, 16>(a, grid, stream);
  return (int)hipErrorInvalidValue;
}

// A shape-specialised instance (StatGeo<T>): its tile shape and dtype/layout
// come from T's geometry.
template <class T>
int launch_stat(const GemmArgs& a, int64_t grid, void* stream) {
  constexpr int DT = T::k.dtype == CBD_F32 ? 0 : 1;
  const void* dy = a.dy;
  const void* w = a.w;
  void* dx = a.dx;
  void* args[] = {&dy, &w, &dx, const_cast<GemmArgs*>(&a)};
  const void* k =
      (const void*)&igemm_generic_kernel<DT, T::k.layout, T::k.bm, T::k.bn, T::k.nw, false, StatGeo<T>>;
  return (int)hipLaunchKernel(k, dim3((unsigned)grid), dim3(T::k.nw * 64), args, 0, (hipStream_t)stream);
}

int launch_static(const GemmArgs& a, int64_t grid, void* stream) {
  switch (a.static_id) {
#define CBD_CASE(i, T, name) \
  case i:                    \
    return launch_stat<T>(a, grid, stream);
    CBD_GENERIC_SHAPE_LIST(CBD_CASE)
#undef CBD_CASE
  }
  return (int)hipErrorInvalidValue;
}

template <int DT, int LAYOUT>
int launch_tiles(const GemmArgs& a, int64_t grid, void* stream) {
  if (a.tile_m == 64 && a.tile_n == 64) return launch_one<DT, LAYOUT, 64, 64>(a, grid, stream);
  if (a.tile_m == 32 && a.tile_n == 64) return launch_one<DT, LAYOUT, 32, 64>(a, grid, stream);
  if (a.tile_m == 64 && a.tile_n == 32) return launch_one<DT, LAYOUT, 64, 32>(a, grid, stream);
  if constexpr (DT == 0 && LAYOUT == 0) {
    // two waves: f32 KCYX plans whose classes all read W by rows (patterns 1-4)
    if (a.tile_m == 32 && a.tile_n == 32 && a.gen_waves == 2) return launch_one<DT, LAYOUT, 32, 32, 2>(a, grid, stream);
  }
  if (a.tile_m == 32 && a.tile_n == 32)
    return a.gen_waves == 8 ? launch_one<DT, LAYOUT, 32, 32, 8>(a, grid, stream)
                            : launch_one<DT, LAYOUT, 32, 32>(a, grid, stream);
  if (a.tile_m == 16 && a.tile_n == 32) return launch_one<DT, LAYOUT, 16, 32>(a, grid, stream);
  if (a.tile_m == 16 && a.tile_n == 16) return launch_one<DT, LAYOUT, 16, 16>(a, grid, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_generic(const GemmArgs& a, int layout, int dtype, int64_t grid, void* stream) {
  if (a.static_shape == 2) return launch_static(a, grid, stream);
  if (dtype == CBD_F32)
    return layout == CBD_LAYOUT_NCHW ? launch_tiles<0, 0>(a, grid, stream)
                                     : launch_tiles<0, 1>(a, grid, stream);
  return layout == CBD_LAYOUT_NCHW ? launch_tiles<1, 0>(a, grid, stream)
                                   : launch_tiles<1, 1>(a, grid, stream);
}

int launch_generic_finalize(const GemmArgs& a, int layout, int dtype, int64_t grid, void* stream) {
  if (dtype == CBD_F32)
    return layout == CBD_LAYOUT_NCHW ? launch_fin_tiles<0, 0>(a, grid, stream)
                                     : launch_fin_tiles<0, 1>(a, grid, stream);
  return layout == CBD_LAYOUT_NCHW ? launch_fin_tiles<1, 0>(a, grid, stream)
                                   : launch_fin_tiles<1, 1>(a, grid, stream);
}

}  // namespace cbd
