// cbd_kernarg.h -- plain-old-data launch arguments shared by the host planner
// and the gfx950 kernels.  Everything a kernel needs arrives by value in the
// kernel-argument segment; no device-side tables are allocated.
#pragma once
#include <stdint.h>

namespace cbd {

// Sub-GEMM (one stride-residue class) descriptors per launch.  The class
// count is at most stride_h * stride_w, which the planner caps at 64.
constexpr int kMaxSub = 64;
constexpr int kMagSub = 16;  // classes with precomputed divisor reciprocals

// ceil(2^32 / d) for d >= 2, 0 for d <= 1: x / d is umulhi(x, r) or one less.
constexpr uint32_t recip32(int64_t d) {
  return d <= 1 ? 0u
                : (uint32_t)((uint64_t(1) << 32) / (uint64_t)d + ((uint64_t(1) << 32) % (uint64_t)d != 0));
}
constexpr int kMaxZero = 64;

// One stride-residue class (i_h, i_w).  Along each axis the class owns the
// taps cls + tstep*j, j < taps; it covers the dX positions phase + S*t,
// t < pos; tap j of position t reads dY row t + beta - delta*j.
struct SubDesc {
  int32_t phase_h, phase_w;
  int32_t beta_h, beta_w;
  int32_t taps_h, taps_w;
  int32_t cls_h, cls_w;
  int32_t pos_h, pos_w;
  int32_t tile_begin;  // first logical workgroup of this class
};

// One dX phase lattice (phase_h + Sh*a, phase_w + Sw*b) that no tap reaches.
// Divisions by pos_w, pos_h and per_pos (16-byte chunks per NHWC pixel row)
// go through rounded-up reciprocals mag = ceil(2^32 / d) (0 when d = 1):
// umulhi(x, mag) is x / d or one more for every 32-bit x.
struct ZeroDesc {
  int32_t phase_h, phase_w;
  int32_t pos_h, pos_w;
  uint32_t mag_h, mag_w;
  uint32_t per_pos, mag_pp;
  int64_t item_begin;  // first work item of this region
};

// Zero-fill folded into the main launch as extra workgroups (generic family,
// at most kMaxFusedZero regions): workgroup total_tiles + i clears work items
// 256*i .. 256*i + 255 exactly as the standalone zero-fill kernel would.
constexpr int kMaxFusedZero = 4;
struct FusedZero {
  int32_t num_regions;  // 0: nothing folded in
  int32_t layout, esize, chunk;
  int32_t C, Hi, Wi, Sh, Sw;
  int32_t pad_;
  int64_t total_items;
  ZeroDesc reg[kMaxFusedZero];
};

// Row-block family (NCHW): workgroup = (image, group, 16-channel block, block
// of rb dX rows); dY rows, W taps and a dX staging tile live in LDS
// (float offsets below).  Divisions by runtime extents go through rounded-up
// reciprocals mag = ceil(2^32 / d) as for the zero-fill.
struct RowsGeom {
  int32_t rb;          // dX rows per workgroup
  int32_t row_blocks;  // ceil(Hi / rb)
  int32_t c_blocks;    // ceil((C/G) / 16)
  int32_t nr;          // dY rows staged (bound over every row block)
  int32_t rw;          // staged dY columns wo_lo ... wo_lo + rw - 1
  int32_t wo_lo;       // first staged dY column (negative: left padding)
  int32_t kg4;         // K/G rounded up to a multiple of 16 (whole groups of four k steps)
  int32_t ks;          // floats per staged k plane (>= nr*rw, = 16 mod 64)
  int32_t nch;         // 64-element chunks per staged k plane (ceil(nr*rw / 64))
  int32_t ksw;         // floats per filter row k of the W tile (>= 16*Y*X, = 16 mod 64)
  int32_t wvec;        // 1: W staged with 16-byte loads (f32, C/G % 16 == 0)
  int32_t cst;         // floats per dX staging channel plane (>= rb*Wi, multiple of 4)
  int32_t w_off;       // float offset of the W tile ([kg4][ksw]: channel c, tap at c*Y*X + tap)
  int32_t st_off;      // float offset of the dX staging tile ([16][cst])
  int32_t vb;          // bytes per dX store (16, 8, 4 or 2)
  int32_t lds_bytes;   // dynamic LDS per workgroup
  uint32_t mag_plane, mag_rw, mag_perk, mag_yx, mag_perc, mag_chunks;
};

// Row-load pattern of a residue class on the generic family (f32 KCYX):
// the taps of one filter row lie within three consecutive W elements, so
// a lane reads them with one two- or three-element load.  1 / 2: one tap
// per row (followed by an element of the same row) in 1 / 2 rows; 3 / 4:
// two taps two apart in 1 / 2 rows; 5: 3 x 3 adjacent taps; 0: none.
constexpr int row_pattern(int taps_h, int taps_w, int cls_w, int X, int tstep_w) {
  return taps_w == 1 && cls_w + 1 < X                   ? (taps_h == 1 ? 1 : taps_h == 2 ? 2 : 0)
         : taps_w == 2 && tstep_w == 2                  ? (taps_h == 1 ? 3 : taps_h == 2 ? 4 : 0)
         : taps_w == 3 && tstep_w == 1 && taps_h == 3 ? 5
                                                        : 0;
}
constexpr int kRowPatsAll = 0x3e;     // patterns 1-5
constexpr int kRowPatsStride2 = 0x1e; // patterns 1-4

struct GemmArgs {
  // problem (element counts; every tensor is < 2^31 bytes)
  int32_t N, G, C, K, Cg, Kg;
  int32_t Hi, Wi, Ho, Wo, Y, X;
  int32_t Sh, Sw;
  int32_t tstep_h, tstep_w;  // T = S / gcd(S, D)
  int32_t delta_h, delta_w;  // delta = D / gcd(S, D)
  // tensor sizes in bytes: buffer-resource record counts, so every access
  // outside a tensor reads 0 / is dropped by the hardware
  uint32_t dy_bytes, w_bytes, dx_bytes;
  int32_t num_sub;
  int32_t total_tiles;
  int32_t tiles_m;     // GEMM-M tiles per group
  int32_t tile_n;      // GEMM-N extent of one tile (positions)
  int32_t tile_m;      // GEMM-M extent of one tile (channels)
  int32_t xcd_remap;   // 1: give each XCD a contiguous range of logical tiles
  int32_t no_split;    // 1: zero-insertion form (one class, all taps, all positions)
  int32_t str_h, str_w, pad_h, pad_w, dil_h, dil_w;  // the problem's own (no_split)
  int32_t iters;       // grouped direct kernel: positions per thread
  int32_t grp_lds;     // grouped row kernel: LDS bytes per workgroup (0: direct kernel)
  int32_t grp_rows;    // grouped pipelined kernels: output rows per workgroup (0: other kernels)
  int32_t grp_mfma;    // 1: the pipelined kernel on 4x4x4 MFMA (bf16, C/G = 4, G in {32, 64})
  int32_t grp_cols;    // MFMA pipelined kernels: positions per column block of a row
  int32_t grp_wide;    // 1: the 16x16x16-MFMA kernel (bf16, C/G = K/G in {16, 32})
  int32_t grp_merged;  // 1: the 4x4x4-MFMA kernel with the four phases of a 2x2 stride in one workgroup
  int32_t gen_waves;   // generic family: waves per workgroup (4, or 8 for long K on small grids)
  int32_t ksplit;      // large-tile kernel: workgroups sharing a tile's K loop (<= 1: none)
  int32_t static_shape;  // large-tile kernel: 1 = 64 k tiles per tap, 1 tap; 2 = the fixed 2048-channel
                         // geometry; generic family: 2 = the instance generic_shapes.h lists as static_id
  int32_t static_id;
  int32_t zblock;      // generic family, one class at phase (0,0) covering every S x S block of dX: its
                       // epilogue also writes the block's unreached positions (no zero-fill)
  int32_t row_pats;    // generic family, f32 KCYX: bit p set when a class has row-load pattern p
  void* ws;            // split-K f32 partial tiles, 256 KiB per workgroup (caller's workspace)
  const void* dy;
  const void* w;
  void* dx;
  RowsGeom rg;
  // tile_begin of every class again, contiguous: a kernel finds its class
  // from one batch of scalar loads instead of one load per class.
  int32_t class_begin[kMaxSub];
  SubDesc sub[kMaxSub];
  // Rounded-up reciprocals ceil(2^32 / d) (0 for d = 1) of the generic
  // family's per-class divisors, for the first kMagSub classes: positions
  // per image (pos_h * pos_w), pos_w, and tiles per group (tiles_m *
  // tiles_n); and of tiles_m.
  uint32_t mag_npix[kMagSub], mag_posw[kMagSub], mag_pergroup[kMagSub];
  uint32_t mag_tiles_m;
  FusedZero fz;
};
// Kernel arguments travel in the 4 KiB kernel-argument segment.
static_assert(sizeof(GemmArgs) <= 4096, "GemmArgs exceeds the kernel-argument segment");


// The whole geometry of one generic-family plan, fixed at compile time in a
// shape-specialised instance.  The planner runs the instance only when every
// field equals the one of the plan it built.
constexpr int kShapeMaxSub = 4;
struct ShapeKey {
  int32_t layout, dtype, bm, bn, nw;
  int32_t N, G, C, K, Cg, Kg, Hi, Wi, Ho, Wo, Y, X, Sh, Sw;
  int32_t tstep_h, tstep_w, delta_h, delta_w;
  int32_t tiles_m, total_tiles, xcd_remap, num_sub, zblock;
  SubDesc sub[kShapeMaxSub];
};

struct ZeroArgs {
  int32_t N, C, Hi, Wi, Sh, Sw;
  int32_t layout;      // 0 NCHW, 1 NHWC
  int32_t esize;       // bytes per element (4 or 2)
  int32_t chunk;       // bytes written per work item
  int32_t num_regions;
  int64_t total_items;
  uint32_t dx_bytes;
  int32_t pad_;
  void* dx;
  ZeroDesc reg[kMaxZero];
};

}  // namespace cbd
