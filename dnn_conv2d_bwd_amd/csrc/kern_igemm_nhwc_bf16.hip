// kern_igemm_nhwc_bf16.hip -- the large-problem family: NHWC dX / NHWK dY /
// KYXC W in bf16, f32 accumulation, bf16 result (the dtype contract of the
// BOO listing in fusilli issue #101: extf to f32, mulf/addf, truncf).
//
// Same per-residue-class GEMM as the generic family (kern_igemm_generic.hip),
// specialised for C/G % 8 == 0 and K/G % 32 == 0, laid out for gfx950:
//   * 256(M = c) x 256(N = positions) workgroup tiles, 32-wide k tiles;
//     256 threads = 4 waves in 2(M) x 2(N), one per SIMD, each wave
//     128x128 = 4x4 blocks of v_mfma_f32_32x32x16_bf16 with the 256 f32
//     accumulators in AGPRs;
//   * both operands travel global -> LDS by buffer_load ... lds (no VGPR
//     staging, no VALU, no ds_write): lane l of an instruction fills 16 bytes
//     at slot l of a 1 KiB LDS block, so the row swizzle is applied by
//     choosing which global chunk each lane fetches;
//   * dY rows (position, 32 k = 64 B) are k-contiguous and feed the MFMA B
//     operand with ds_read_b128; W rows (k, 256 c = 512 B) stay c-contiguous
//     and ds_read_b64_tr_b16 transposes 4x4 bf16 blocks on the way out, giving
//     each lane the k-vector of one channel (MFMA A operand);
//   * bank-conflict-free XOR swizzles for both fragment reads;
//   * four 32 KiB LDS stages (W parts at [0, 64 KiB), dY parts above, so
//     every fragment read is a base register plus a 16-bit immediate);
//     loads run three to four k tiles ahead; one barrier per k tile, placed
//     between its two k steps, so the fragments of the next step are always
//     read one step ahead of the MFMAs that use them;
//   * a wave issues at most one instruction per four clocks and each VALU
//     instruction between MFMAs costs MFMA time, so the loop carries only
//     MFMAs, fragment reads, loads and a few scalar instructions per tile
//     (load offsets step in the scalar offset, past-the-end tiles load
//     through a zero record count); the issue order is pinned with
//     scheduling barriers;
//   * per-tap dY gather offsets (position -> byte offset, or out of range for
//     taps off dY's edge and ragged tiles) and per-position dX offsets are
//     built once per workgroup into small LDS tables; with one tap per class
//     each lane computes its dY offsets itself and the dX table is built
//     while the first tiles load;
//   * epilogue: accumulators -> bf16 (nearest-even, v_cvt_pk_bf16_f32) -> LDS
//     ([position][c], chunk ^ (row & 31)) -> 16-byte coalesced stores along
//     each dX pixel row, in four column groups so that one group's stores
//     drain while the next is converted; in the 2048-channel instance the
//     last four k tiles run one column group at a time instead, so that
//     three groups' conversions and stores overlap the remaining MFMAs;
//   * a fully shape-specialised instance for the 2048-channel 1x2 stride-2
//     problem (any batch and even width) takes the class from its tile
//     index and computes every offset with shifts and multiplies; the
//     tensors arrive as preloaded scalar kernel parameters.
#include <type_traits>

#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int BM = kFastBM, BN = kFastBN, BK = kFastBK;  // 256, 256, 32
constexpr int THREADS = kFastThreads;                    // 256: 4 waves, one per SIMD
constexpr int NSTAGE = 4;
constexpr int AROW = BM * 2;                             // 512 B: one k row of the W tile
constexpr int BROW = BK * 2;                             // 64 B: one position row of the dY tile
constexpr int ABYTES = BK * AROW;                        // 16 KiB: W part of a stage
constexpr int BBYTES = BN * BROW;                        // 16 KiB: dY part of a stage
constexpr int STAGE = ABYTES + BBYTES;                   // 32 KiB
constexpr int BBASE = NSTAGE * ABYTES;                   // dY parts follow the four W parts
constexpr int MAX_TAPS = kFastMaxTaps;                   // gather-table capacity (taps per class)
constexpr int DMA_PER_TILE = 8;                          // per wave: 4 W + 4 dY instructions
static_assert(THREADS / 64 * DMA_PER_TILE * 1024 == STAGE, "one stage = all waves' loads of a tile");
static_assert(THREADS >= BN, "one thread per position row builds the tables");

// s_waitcnt immediate: vmcnt <= n, other counters unconstrained (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// LDS swizzles (16-byte chunk index XOR a function of the row).  gfx950 LDS
// has 64 four-byte banks; a ds_read_b64(_tr) serves lanes 0-31, then 32-63,
// 256 bytes per clock, and a ds_read_b128 serves 16 lanes per clock.  With
// these maps every fragment read below touches each bank once per clock
// (verified with the SQ_LDS_BANK_CONFLICT counter).
__device__ inline int swz_w(int row) { return 4 * (row & 3); }  // W rows: 32 chunks
__device__ inline int swz_y(int row) { return (row >> 2) & 3; }  // dY rows: 4 chunks

// Channels of the fully shape-specialised instance (FIX): C = K = 2048, one
// group, one dX row (Hi = 1) of Wi = 2 Wo pixels, a 1x2 filter at stride 2
// along W with no padding or dilation -- the problem of the BOO listing in
// fusilli issue #101 at any batch and width.  Class r (filter tap x = r)
// then writes dX pixel 2p + r from dY pixel p and the weight slice
// W[:, 0, r, :]: two plain GEMMs, no descriptor or division anywhere.
constexpr int FIX_CH = 2048;

// Cache policy of the dX stores: sc0 sc1 (bits 0 and 4 of the buffer_store
// cache-policy operand), i.e. written through at system scope instead of
// held dirty in L2.  Every workgroup ends at about the same time, so dirty
// lines would otherwise all be written back in one burst when the launch
// completes; written through, they leave while later column groups of the
// epilogue are still being converted (measured: about 0.9 us less per
// launch on the 2048-channel problem, with the same bits written).
#ifndef CBD_NHWC_STORE_AUX
#define CBD_NHWC_STORE_AUX 17
#endif
constexpr int kStoreAux = CBD_NHWC_STORE_AUX;

// SPLIT: the K loop of each tile is split over a.ksplit workgroups that
// write f32 partial tiles (a separate instance, so that the plain kernel
// carries none of its registers).  SKPT, STAPS > 0: a shape-specialised
// instance with k tiles per tap and taps per class fixed at compile time
// (0: read from the descriptors at run time).  FIX: the fully specialised
// instance above (SKPT = 64, STAPS = 1), which reads nothing but its scalar
// parameters.
//
// The tensors and their byte sizes (buffer record counts) come first as
// scalar parameters, which the compiler preloads into SGPRs at wave launch:
// no kernel-argument fetch stands between the launch and the first loads.
// fix_npos / fix_tiles (positions per class, workgroups) serve FIX only.
template <bool SPLIT, int SKPT, int STAPS, bool FIX>
__global__ __launch_bounds__(THREADS, 1) void igemm_nhwc_bf16_kernel(
    const void* dy_p, const void* w_p, void* dx_p, uint32_t dy_bytes, uint32_t w_bytes,
    uint32_t dx_bytes, int32_t fix_npos, int32_t fix_tiles, const GemmArgs a) {
  static_assert(!FIX || (!SPLIT && SKPT == FIX_CH / BK && STAPS == 1), "FIX: one tap, K = 2048, no split");
  // Stages as distinct objects: the compiler can then see that fragment reads
  // of one stage do not alias the loads in flight into another.
  // W parts of the four stages at [0, 64 KiB), dY parts at [64, 128 KiB):
  // every fragment read is then one of a few base registers plus an
  // immediate below 64 KiB.
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];
  __shared__ uint32_t gtab[MAX_TAPS * BN];  // dY byte offset of (tap, position row), channel g*Kg
  __shared__ uint32_t otab[BN];             // dX byte offset of position row, channel g*Cg + m0
  __shared__ uint32_t atab[MAX_TAPS];       // W byte offset of (tap, k row 0), channel g*Cg
  // FIX: bf16 staging of one column group of the C tile (64 position rows x
  // 512 B), filled while the next group's MFMAs run; with the four stages
  // this takes the whole 160 KiB of LDS, so FIX keeps no dX table (it
  // computes dX offsets directly).
  __shared__ __attribute__((aligned(16))) char stg[FIX ? 64 * 512 : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // wm: 128-channel half, wn: 128-position half

  // Tile decode: logical tile t -> (class, group, split, m0, n0).
  SubDesc s = {};
  int t, npix_img, npos, split, g, m0, n0, fix_r = 0;
  const int S = SPLIT ? a.ksplit : 1;
  if constexpr (FIX) {
    // Two classes of fix_tiles / 2 tiles each, 8 channel tiles per position tile.
    t = dev::logical_tile(blockIdx.x, fix_tiles, fix_tiles >= 64 ? 1 : 0);
    fix_r = t >= (fix_tiles >> 1) ? 1 : 0;
    const int local = t - fix_r * (fix_tiles >> 1);
    m0 = (local & (FIX_CH / BM - 1)) * BM;
    n0 = (local / (FIX_CH / BM)) * BN;
    npos = fix_npos;
    npix_img = 0;
    split = 0;
    g = 0;
  } else {
    dev::prefetch_args(a);
    t = dev::logical_tile(blockIdx.x, a.total_tiles, a.xcd_remap);
    s = a.sub[dev::find_class(a, t)];
    npix_img = s.pos_h * s.pos_w;
    npos = a.N * npix_img;
    const int tiles_n = (npos + BN - 1) / BN;
    const int per_group = a.tiles_m * tiles_n;
    // With the K loop split over S workgroups (S = a.ksplit > 1), the S
    // workgroups of a tile are consecutive: split = t mod S (class ranges
    // start at multiples of S).
    split = (t - s.tile_begin) % S;
    const int local = (t - s.tile_begin) / S;
    g = local / per_group;
    const int rem = local - g * per_group;
    m0 = (rem % a.tiles_m) * BM;
    n0 = (rem / a.tiles_m) * BN;
  }
  const int ntaps = STAPS > 0 ? STAPS : s.taps_h * s.taps_w;
  const int Cg = FIX ? FIX_CH : a.Cg;

  // Buffer descriptors of dY and W as plain SGPR quads (the loads below are
  // written in assembly), record count = tensor bytes as in dev::rsrc.
  const i32x4 dyd = {(int)(uint32_t)(uintptr_t)dy_p, (int)(((uintptr_t)dy_p >> 32) & 0xffff),
                     (int)dy_bytes, 0x00020000};
  const i32x4 dw = {(int)(uint32_t)(uintptr_t)w_p, (int)(((uintptr_t)w_p >> 32) & 0xffff),
                    (int)w_bytes, 0x00020000};
  const auto rdx = dev::rsrc(dx_p, dx_bytes);
  // Uniform loop bounds, fixed before the divergent table build (values
  // first defined inside a divergent region would live in VGPRs).
  const int YX = FIX ? 2 : __builtin_amdgcn_readfirstlane(a.Y * a.X);
  const uint32_t wrow = FIX ? 2u * FIX_CH * 2u
                            : __builtin_amdgcn_readfirstlane((uint32_t)(YX * a.Cg) * 2u);  // bytes between k rows of W
  const int kpt = SKPT > 0 ? SKPT : __builtin_amdgcn_readfirstlane(a.Kg / BK);
  // This workgroup's k tiles: [kb, ke) of the class's ntaps * kpt (tile t =
  // tap t / kpt, k rows 32 (t mod kpt) ...); the planner keeps S <= ntaps*kpt.
  const int KTall = SKPT > 0 && STAPS > 0 ? SKPT * STAPS : __builtin_amdgcn_readfirstlane(ntaps * kpt);
  const int kb = __builtin_amdgcn_readfirstlane(split * KTall / S);
  const int ke = __builtin_amdgcn_readfirstlane((split + 1) * KTall / S);
  int KT = ke - kb;  // k tiles of this workgroup
  // Opaque to the optimiser: with a compile-time trip count (the
  // shape-specialised instance) it restructures the loop and spills.
  asm volatile("" : "+s"(KT));
  const uint32_t kpt_magic = __builtin_amdgcn_readfirstlane(0xffffffffu / (uint32_t)kpt + 1u);

  // With one tap per class (the shape-specialised instance) every tile of
  // [kb, ke) belongs to tap 0, whose load offsets each lane computes itself:
  // the first loads then go out before any table is built.
  constexpr bool ONE_TAP = STAPS == 1;

  // ---- per-workgroup tables (threads 0..255: one position row each): the
  // dY offsets of every tap (not needed with one tap), the dX offsets, and
  // the W offset of every tap.
  auto build_tables = [&]() {
    if constexpr (FIX) return;
    if (tid < BN) {
      const int p = n0 + tid;
      const bool pv = p < npos;
      const int pp = pv ? p : 0;
      const int n = pp / npix_img;
      const int rr = pp - n * npix_img;
      const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
      if constexpr (!ONE_TAP) {
        for (int tap = 0; tap < ntaps; tap++) {
          const int jh = tap / s.taps_w, jw = tap - (tap / s.taps_w) * s.taps_w;
          const int ho = dev::dy_index(a.no_split, th, s.beta_h, a.delta_h, jh, a.pad_h, a.dil_h, a.str_h);
          const int wo = dev::dy_index(a.no_split, tw, s.beta_w, a.delta_w, jw, a.pad_w, a.dil_w, a.str_w);
          const bool ok = pv && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
          gtab[tap * BN + tid] = ok ? (uint32_t)(((n * a.Ho + ho) * a.Wo + wo) * a.K + g * a.Kg) * 2u : dev::kOOB;
        }
      }
      const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
      otab[tid] = pv ? (uint32_t)(((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg + m0) * 2u : dev::kOOB;
    }
    if (!ONE_TAP && tid < ntaps) {
      const int jh = tid / s.taps_w, jw = tid - (tid / s.taps_w) * s.taps_w;
      const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
      atab[tid] = (uint32_t)(((g * a.Kg) * YX + ty * a.X + tx) * a.Cg) * 2u;
    }
  };
  if constexpr (!ONE_TAP) {
    build_tables();
    __syncthreads();
  }

  // ---- load roles.  W: instruction i (0..3) of wave w fills k rows
  // 8w + 2i + (lane >> 5), 16-byte slot lane & 31 holding channel chunk
  // (lane & 31) ^ swz_w(row).  dY: instruction i fills position rows
  // 16*(4w + i) + (lane >> 2), slot lane & 3 holding k chunk (lane & 3) ^ swz_y(row).
  uint32_t a_lane[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int row = 8 * wave + 2 * i + (lane >> 5);
    const int c = m0 + 8 * ((lane & 31) ^ swz_w(row));
    a_lane[i] = c < Cg ? (uint32_t)row * wrow + (uint32_t)c * 2u : dev::kOOB;
  }
  int b_row[4];
  uint32_t b_chunk[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    b_row[i] = 16 * (4 * wave + i) + (lane >> 2);
    b_chunk[i] = (uint32_t)(((lane & 3) ^ swz_y(b_row[i])) * 16);
  }

  // Next tile to load, per operand: a vector offset per lane that stays
  // fixed within a tap, plus a running scalar offset (the k rows of the
  // tile within its tap), so the per-tile step is one scalar add with no
  // vector instruction between the MFMAs.  Tiles past the end load through
  // a buffer descriptor whose record count is 0 (zeros into a stage that is
  // no longer read), which keeps the count of loads in flight the same on
  // every tile.
  const uint32_t a_step = (uint32_t)BK * wrow, b_step = (uint32_t)BK * 2u;
  // First tile kb: tap kb / kpt, k tile kb mod kpt within it.
  const int tap0 = __builtin_amdgcn_readfirstlane(kb / kpt);
  const uint32_t r0 = (uint32_t)(kb - tap0 * kpt);
  uint32_t a_off[4], b_off[4];
  if constexpr (FIX) {
    // dY pixel p, k chunk; W slice r (row k at k * 2 * C, tap r at r * C).
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a_off[i] = a_lane[i] + (uint32_t)fix_r * (FIX_CH * 2u);
      const int p = n0 + b_row[i];
      b_off[i] = p < npos ? (uint32_t)p * (FIX_CH * 2u) + b_chunk[i] : dev::kOOB;
    }
  } else if constexpr (ONE_TAP) {
    // Tap 0 of the class (taps y = cls_h, x = cls_w; dY row t + beta).
    // Position p = (n, th, tw) by multiply-high with m = ceil(2^32 / d):
    // the estimate is q or q + 1 for every x < 2^32 and one compare fixes it.
    const uint32_t npix = (uint32_t)npix_img, posw = (uint32_t)s.pos_w;
    const uint32_t mpix = __builtin_amdgcn_readfirstlane(0xffffffffu / npix + 1u);
    const uint32_t mw = __builtin_amdgcn_readfirstlane(0xffffffffu / posw + 1u);
    auto udiv = [](uint32_t x, uint32_t d, uint32_t m) -> uint32_t {
      const uint32_t q = __umulhi(x, m);
      return d == 1u ? x : (q * d > x ? q - 1u : q);
    };
    const uint32_t abase = (uint32_t)(((g * a.Kg) * YX + s.cls_h * a.X + s.cls_w) * a.Cg) * 2u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a_off[i] = a_lane[i] + abase;
      const int p = n0 + b_row[i];
      const bool pv = p < npos;
      const uint32_t pp = pv ? (uint32_t)p : 0u;
      const uint32_t n = udiv(pp, npix, mpix);
      const uint32_t rr = pp - n * npix;
      const uint32_t th = udiv(rr, posw, mw);
      const int ho = (int)th + s.beta_h, wo = (int)(rr - th * posw) + s.beta_w;
      const bool ok = pv && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
      b_off[i] = ok ? (uint32_t)((((int)n * a.Ho + ho) * a.Wo + wo) * a.K + g * a.Kg) * 2u + b_chunk[i]
                    : dev::kOOB;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a_off[i] = a_lane[i] + atab[tap0];
      b_off[i] = gtab[tap0 * BN + b_row[i]] + b_chunk[i];
    }
  }
  uint32_t a_soff = __builtin_amdgcn_readfirstlane(r0 * a_step);
  uint32_t b_soff = __builtin_amdgcn_readfirstlane(r0 * b_step);
  uint32_t a_rec = w_bytes, b_rec = dy_bytes;  // record counts of the next tile's loads
  // Tile t = (tap, k tile) with tap = t / kpt, by multiply-high with a
  // rounded-up reciprocal (exact for t < 17 kpt, kpt <= 4096: tiles per
  // class are at most 16 kpt, plus the 4 tiles loaded past the end).
  auto tap_of = [&](int t) -> int {
    if constexpr (SKPT > 0) return t / SKPT;
    return kpt == 1 ? t : (int)__umulhi((uint32_t)t, kpt_magic);
  };
  // Move the offsets of an operand from tile t-1 to tile t (a uniform
  // branch where a new tap starts, once per kpt tiles).
  auto advance_a = [&](int t) {
    if (!ONE_TAP && t < ke && t - tap_of(t) * kpt == 0) {
      const uint32_t base = atab[tap_of(t)];
#pragma unroll
      for (int i = 0; i < 4; i++) a_off[i] = a_lane[i] + base;
      a_soff = 0;
    } else {
      a_soff += a_step;
    }
    a_rec = t < ke ? w_bytes : 0u;
  };
  auto advance_b = [&](int t) {
    if (!ONE_TAP && t < ke && t - tap_of(t) * kpt == 0) {
      const int tap = tap_of(t);
#pragma unroll
      for (int i = 0; i < 4; i++) b_off[i] = gtab[tap * BN + b_row[i]] + b_chunk[i];
      b_soff = 0;
    } else {
      b_soff += b_step;
    }
    b_rec = t < ke ? dy_bytes : 0u;
  };
  // Load j of a tile (j < 4: W, else dY): 64 lanes x 16 bytes, global ->
  // LDS without VGPRs (buffer_load ... lds; lane l writes 16 bytes at
  // M0 + 16 l).  Written in assembly so that the compiler does not add its
  // own conservative vmcnt waits before fragment reads of other stages: the
  // waits that order these loads against LDS reads are the explicit ones in
  // the main loop and before the epilogue.  The destination stage is a
  // compile-time constant, so M0 is this wave's base (a scalar register)
  // plus an immediate.  Nothing else in this kernel uses M0.
  const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_char*)smem;
  const uint32_t mbase = __builtin_amdgcn_readfirstlane(smem_base + (uint32_t)wave * 4096u);
  auto m0_of = [&](int ds, int j) -> uint32_t {
    return mbase + (uint32_t)(j < 4 ? ds * ABYTES + j * 1024 : BBASE + ds * BBYTES + (j - 4) * 1024);
  };
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  auto issue_one = [&](auto dstc, int j) {
    constexpr int DS = decltype(dstc)::value;
    const uint32_t m0v = m0_of(DS, j);
    const uint32_t voff = j < 4 ? a_off[j] : b_off[j - 4];
    const uint32_t soff = __builtin_amdgcn_readfirstlane(j < 4 ? a_soff : b_soff);
    const i32x4 desc = j < 4 ? i32x4{dw[0], dw[1], (int)a_rec, dw[3]} : i32x4{dyd[0], dyd[1], (int)b_rec, dyd[3]};
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds\n\ts_nop 0"
                 :: "s"(m0v), "v"(voff), "s"(desc), "s"(soff) : "memory", "m0");
  };
  // The same load split in two: M0 is written one MFMA ahead of the load
  // that reads it, which covers the M0 -> LDS-load wait state without an
  // s_nop.
  auto set_m0 = [&](auto dstc, int j) {
    constexpr int DS = decltype(dstc)::value;
    const uint32_t m0v = m0_of(DS, j);
    asm volatile("s_mov_b32 m0, %0" :: "s"(m0v) : "memory", "m0");
  };
#pragma clang diagnostic pop
  auto load_m0 = [&](int j) {
    const uint32_t voff = j < 4 ? a_off[j] : b_off[j - 4];
    const uint32_t soff = __builtin_amdgcn_readfirstlane(j < 4 ? a_soff : b_soff);
    const i32x4 desc = j < 4 ? i32x4{dw[0], dw[1], (int)a_rec, dw[3]} : i32x4{dyd[0], dyd[1], (int)b_rec, dyd[3]};
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" :: "v"(voff), "s"(desc), "s"(soff) : "memory");
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // ---- fragment addresses.  A (transposed read): in 16-lane group G, lane j
  // points at k row 8*(G>>1) + 4*half + (j>>2) (+ 16*ks), channels
  // cb + 4*(j&3) .. +3 with cb = 128*wm + 32*bm + 16*(G&1); the read returns
  // to lane j the 4 k values of channel cb + j.
  const int G = lane >> 4, jl = lane & 15;
  int a_rd[4][2][2];  // [bm][ks][half]
#pragma unroll
  for (int bm = 0; bm < 4; bm++) {
    const int lc = ((wm * 128 + bm * 32 + 16 * (G & 1)) >> 3) + ((jl & 3) >> 1);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int row = ks * 16 + 8 * (G >> 1) + 4 * h + (jl >> 2);
        a_rd[bm][ks][h] = row * AROW + ((lc ^ swz_w(row)) << 4) + ((jl & 1) << 3);
      }
  }
  // B: lane reads chunk 2*ks + (lane >> 5) of position row wn*128 + 32*bn + (lane & 31).
  int b_rd[4][2];
#pragma unroll
  for (int bn = 0; bn < 4; bn++) {
    const int row = wn * 128 + bn * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      b_rd[bn][ks] = BBASE + row * BROW + (((2 * ks + (lane >> 5)) ^ swz_y(row)) << 4);
  }

  // Read r (0..11) of the fragments of k step ks, in the order the next
  // k step consumes them: A block 0 (two transposed halves), B blocks 0-3,
  // then A blocks 1-3.
  auto read_one = [&](auto stc, int ks, int r, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
    constexpr int ST = decltype(stc)::value;
    lds_char* st = (lds_char*)smem + ST * ABYTES;
    const char* sb = smem + ST * BBYTES;
    if (r >= 2 && r < 6) {
      fb[r - 2] = *(const bf16x8*)(sb + b_rd[r - 2][ks]);
    } else {
      const int i = r < 2 ? 0 : (r - 4) >> 1, h = r & 1;
      const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(st + a_rd[i][ks][h]));
      if (h == 0) { fa[i][0] = v[0]; fa[i][1] = v[1]; fa[i][2] = v[2]; fa[i][3] = v[3]; }
      else { fa[i][4] = v[0]; fa[i][5] = v[1]; fa[i][6] = v[2]; fa[i][7] = v[3]; }
    }
  };
  // 16 MFMAs on (fa, fb); one fragment read of the next k step after each
  // of the first 12, one load after every fourth, and the offset update of
  // the operand loaded in the previous half after the second.  The order is
  // pinned with scheduling barriers: a wave issues at most one instruction
  // per four clocks, so everything besides the MFMAs has to be spread thin.
  auto half = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], auto rstc, int rks,
                  bf16x8 (&ra)[4], bf16x8 (&rb)[4], auto dstc, int j0, auto&& advance,
                  auto nlc) {
    constexpr int NL = decltype(nlc)::value;  // loads in this half: 4, or 8 (W and dY of one tile)
#pragma unroll
    for (int q = 0; q < 16; q++) {
      // Boustrophedon order over the 4x4 blocks: consecutive MFMAs change
      // one operand at a time (fewer operand bits toggle between them).
      const int bm = q >> 2, bn = (bm & 1) ? 3 - (q & 3) : (q & 3);
      acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bm], fb[bn], acc[bm][bn], 0, 0, 0);
      if (q < 12) read_one(rstc, rks, q, ra, rb);
      if constexpr (NL == 4) {
        if ((q & 3) == 2) set_m0(dstc, j0 + (q >> 2));
        if ((q & 3) == 3) load_m0(j0 + (q >> 2));
      } else {
        if ((q & 1) == 0) set_m0(dstc, j0 + (q >> 1));
        if ((q & 1) == 1) load_m0(j0 + (q >> 1));
      }
      if (q == 1) advance();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop.  Iteration kt: k step 0 of tile kt (fragments already in
  // registers) issues the dY loads of tile kt+3; then, once tile kt+1 has
  // landed and every wave has finished reading tile kt (barrier), the first
  // fragments of tile kt+1 are read while k step 1 of tile kt issues the W
  // loads of tile kt+4 into tile kt's stage.  Prologue: tiles 0-2 whole and
  // the W loads of tile 3.
#pragma unroll
  for (int j = 0; j < DMA_PER_TILE; j++) issue_one(std::integral_constant<int, 0>(), j);
  advance_a(kb + 1);
  advance_b(kb + 1);
#pragma unroll
  for (int j = 0; j < DMA_PER_TILE; j++) issue_one(std::integral_constant<int, 1>(), j);
  advance_a(kb + 2);
  advance_b(kb + 2);
#pragma unroll
  for (int j = 0; j < DMA_PER_TILE; j++) issue_one(std::integral_constant<int, 2>(), j);
  advance_a(kb + 3);
  advance_b(kb + 3);
#pragma unroll
  for (int j = 0; j < DMA_PER_TILE / 2; j++) issue_one(std::integral_constant<int, 3>(), j);
  // One tap: the dX offsets are built while the first tiles are in flight
  // (the wait below also completes their LDS writes).
  if constexpr (ONE_TAP) build_tables();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((NSTAGE - 2) * DMA_PER_TILE + DMA_PER_TILE / 2));
  __builtin_amdgcn_s_barrier();
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
#pragma unroll
  for (int r = 0; r < 12; r++) read_one(std::integral_constant<int, 0>(), 0, r, fa0, fb0);
  auto iter = [&](int kt, auto stc) {
    constexpr int ST = decltype(stc)::value;
    half(fa0, fb0, stc, 1, fa1, fb1, std::integral_constant<int, (ST + 3) & (NSTAGE - 1)>(),
         DMA_PER_TILE / 2, [&]() { advance_a(kb + kt + NSTAGE); }, std::integral_constant<int, 4>());
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((NSTAGE - 2) * DMA_PER_TILE));
    __builtin_amdgcn_s_barrier();
    half(fa1, fb1, std::integral_constant<int, (ST + 1) & (NSTAGE - 1)>(), 0, fa0, fb0, stc, 0,
         [&]() { advance_b(kb + kt + NSTAGE); }, std::integral_constant<int, 4>());
  };
  // ---- FIX: the last four k tiles (all resident, one per stage) one
  // column group bn at a time -- 32 positions of each wave's half, all four
  // k tiles -- so that group bn's accumulators are final three groups
  // before the end.  Its conversion to bf16 (into the staging buffer) and
  // its dX stores then run between the MFMAs of the next group, and only
  // the last group's stores remain after the last MFMA.  Per element the
  // summation order is the main loop's (k ascending), so the result is the
  // same bits.  The A fragments of the four tiles are read once (group 0)
  // and kept; B is read per step.  Group 0 waits for tiles KT-3..KT-1 as it
  // reaches them.
  auto tail_and_store = [&]() {
    bf16x8 ta[NSTAGE][2][4];  // [tile][k step][bm]
    bf16x8 tb[2];
#pragma unroll
    for (int i = 0; i < 4; i++) ta[0][0][i] = fa0[i];
    tb[0] = fb0[0];
    // Staging: row r = 32 wn + (lane & 31) holds position wn*128 + 32 bn + (lane & 31);
    // 16-byte chunk c/8 at chunk (c/8) ^ (r & 31) (conflict-free 8-byte writes).
    lds_char* const sg = (lds_char*)stg;
    const int srow = wn * 32 + (lane & 31);
    lds_char* sw[4][4];
#pragma unroll
    for (int bm = 0; bm < 4; bm++)
#pragma unroll
      for (int qq = 0; qq < 4; qq++) {
        const int chunk = wm * 16 + bm * 4 + qq;
        sw[bm][qq] = sg + srow * 512 + ((chunk ^ (srow & 31)) << 4) + ((lane >> 5) << 3);
      }
    // Stores: thread = (row r0 = tid >> 5 of each 8, chunk sc = tid & 31);
    // item it covers staging row 8 it + r0.  dX pixel of position p is
    // 2p + fix_r (positions past npos fall beyond dX's record count).
    const int r0 = tid >> 5, sc = tid & 31;
    lds_char* sr[4];
#pragma unroll
    for (int i = 0; i < 4; i++) sr[i] = sg + (i * 8 + r0) * 512 + (((sc ^ r0) ^ (i * 8)) << 4);
    const uint32_t obase = (uint32_t)(2 * (n0 + r0) + fix_r) * (FIX_CH * 2u) + (uint32_t)m0 * 2u + (uint32_t)sc * 16u;
    auto convert_part = [&](int bn, int bm, int qq) {
      u32x2 o;
      o[0] = dev::bf16_pack2(acc[bm][bn][4 * qq + 0], acc[bm][bn][4 * qq + 1]);
      o[1] = dev::bf16_pack2(acc[bm][bn][4 * qq + 2], acc[bm][bn][4 * qq + 3]);
      *(__attribute__((address_space(3))) u32x2*)sw[bm][qq] = o;
    };
    u32x4 sv[8];  // the group's staged chunks of this thread, read at once after the fill barrier
    auto read_items = [&]() {
#pragma unroll
      for (int it = 0; it < 8; it++)
        sv[it] = *(const __attribute__((address_space(3))) u32x4*)(sr[it & 3] + (it >> 2) * (32 * 512));
    };
    auto store_item = [&](int bn, int it) {
      const uint32_t prow = (uint32_t)((it >> 2) * 128 + bn * 32 + (it & 3) * 8);  // position row - r0
      __builtin_amdgcn_raw_buffer_store_b128(u4{sv[it][0], sv[it][1], sv[it][2], sv[it][3]}, rdx,
                                             obase + prow * (2u * FIX_CH * 2u), 0, kStoreAux);
    };
    auto sync_lds = [&]() {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));  // lgkmcnt(0), vmcnt unconstrained
      __builtin_amdgcn_s_barrier();
    };
#pragma unroll
    for (int st = 0; st < 32; st++) {
      const int g = st >> 3, j = (st >> 1) & 3, ks = st & 1, ph = st & 7;
      const int s1 = st + 1, g1 = s1 >> 3, j1 = (s1 >> 1) & 3, ks1 = s1 & 1;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        acc[q][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[j][ks][q], tb[st & 1], acc[q][g], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (q == 0) {
          if (s1 < 32 && g1 == 0 && ks1 == 0) {
            // tile KT-4+j1 (stage j1) complete: its loads are older than the
            // 8 (3 - j1) loads of the later tiles
            if (j1 == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
            if (j1 == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
            if (j1 == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __builtin_amdgcn_s_barrier();
          }
          if (g >= 2 && ph == 0) sync_lds();  // staging read out by every thread
          if (g >= 1 && ph == 4) {
            sync_lds();  // staging filled by every thread
            read_items();
          }
        }
        if (s1 < 32) {
          if (q == 0) tb[s1 & 1] = *(const bf16x8*)(smem + j1 * BBYTES + b_rd[g1][ks1]);
          if (g1 == 0) {
            lds_char* at = (lds_char*)smem + j1 * ABYTES;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(at + a_rd[q][ks1][0]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(at + a_rd[q][ks1][1]));
            ta[j1][ks1][q] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        if (g >= 1 && ph < 4) convert_part(g - 1, ph, q);
        // stores of the staged group: items 0, 1 at q = 2, 3 of the read
        // step, then two per step
        if (g >= 1 && ph == 4 && q >= 2) store_item(g - 1, q - 2);
        if (g >= 1 && ph > 4 && (q & 1) == 0) store_item(g - 1, 2 * (ph - 4) + (q >> 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    sync_lds();
#pragma unroll
    for (int bm = 0; bm < 4; bm++)
#pragma unroll
      for (int qq = 0; qq < 4; qq++) convert_part(3, bm, qq);
    sync_lds();
    read_items();
#pragma unroll
    for (int it = 0; it < 8; it++) store_item(3, it);
  };

  if constexpr (FIX) {
    // Tiles [0, KT-4) here; the last of them loads the W and dY parts of
    // tile KT-1 together (no loads past the end); tiles [KT-4, KT) in the
    // tail.
    static_assert(SKPT * STAPS % NSTAGE == 0 && SKPT * STAPS >= 2 * NSTAGE, "FIX: whole rounds of stages");
#pragma unroll 1
    for (int kt = 0; kt < KT - 2 * NSTAGE; kt += NSTAGE) {
      iter(kt, std::integral_constant<int, 0>());
      iter(kt + 1, std::integral_constant<int, 1>());
      iter(kt + 2, std::integral_constant<int, 2>());
      iter(kt + 3, std::integral_constant<int, 3>());
    }
    iter(KT - 8, std::integral_constant<int, 0>());
    iter(KT - 7, std::integral_constant<int, 1>());
    iter(KT - 6, std::integral_constant<int, 2>());
    {
      const int kt = KT - 5;
      constexpr int ST = 3;
      half(fa0, fb0, std::integral_constant<int, ST>(), 1, fa1, fb1, std::integral_constant<int, (ST + 3) & (NSTAGE - 1)>(),
           DMA_PER_TILE / 2, [&]() { advance_a(kb + kt + NSTAGE); }, std::integral_constant<int, 4>());
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((NSTAGE - 2) * DMA_PER_TILE));
      __builtin_amdgcn_s_barrier();
      half(fa1, fb1, std::integral_constant<int, 0>(), 0, fa0, fb0, std::integral_constant<int, ST>(), 0,
           [&]() { advance_b(kb + kt + NSTAGE); }, std::integral_constant<int, 8>());
    }
    tail_and_store();
    return;
  }
#pragma unroll 1
  for (int kt = 0; kt < KT; kt += NSTAGE) {
    iter(kt, std::integral_constant<int, 0>());
    if (kt + 1 < KT) iter(kt + 1, std::integral_constant<int, 1>());
    if (kt + 2 < KT) iter(kt + 2, std::integral_constant<int, 2>());
    if (kt + 3 < KT) iter(kt + 3, std::integral_constant<int, 3>());
  }

  // The loads past the last tile (zeros into free stages) must land before
  // the stages are reused for the C tile.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if constexpr (SPLIT) {
    // ---- split-K epilogue: the f32 partial tile goes to the workspace,
    // block t (256 KiB, [position row][256 channels]), for the finalising
    // kernel to sum.  Through LDS in two halves of 128 rows (the waves of
    // one position half at a time), 16-byte chunk q of row r stored at
    // chunk q ^ (r & 31); then 1 KiB rows out with 16-byte stores.
    char* const ws = (char*)a.ws + (size_t)t * (BM * BN * 4);
    const auto rws = dev::rsrc(ws, BM * BN * 4);
#pragma unroll
    for (int h = 0; h < 2; h++) {
      __syncthreads();
      if (wn == h) {
#pragma unroll
        for (int bn = 0; bn < 4; bn++) {
          const int prow = bn * 32 + (lane & 31);  // row within the half
          char* rowp = smem + prow * 1024;
#pragma unroll
          for (int bm = 0; bm < 4; bm++) {
#pragma unroll
            for (int qq = 0; qq < 4; qq++) {
              const int c = wm * 128 + bm * 32 + 8 * qq + 4 * (lane >> 5);
              const f32x4 v = {acc[bm][bn][4 * qq + 0], acc[bm][bn][4 * qq + 1],
                               acc[bm][bn][4 * qq + 2], acc[bm][bn][4 * qq + 3]};
              *(f32x4*)(rowp + (((c >> 2) ^ (prow & 31)) << 4)) = v;
            }
          }
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < 128 * 64 / THREADS; it++) {
        const int row = it * (THREADS / 64) + (tid >> 6), q = tid & 63;
        const u32x4 v = *(const u32x4*)(smem + row * 1024 + ((q ^ (row & 31)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(u4{v[0], v[1], v[2], v[3]}, rws,
                                               (uint32_t)((h * 128 + row) * 1024 + q * 16), 0, 0);
      }
    }
    return;
  }

  // ---- epilogue.  C tile [position row][256 channels] bf16 = 128 KiB over
  // the four stages, 16-byte chunk c/8 of row r stored at chunk
  // (c/8) ^ (r & 31).  In four column groups bn (positions 32 bn ... and
  // 128 + 32 bn ..., 64 rows): every wave converts its blocks of group bn,
  // a barrier, then 16-byte stores along the group's pixel rows; the stores
  // of one group drain while the next group is converted (distinct rows, so
  // no further barrier).
  __syncthreads();
  const int ch = tid & 31;
  const bool cv = m0 + 8 * ch < Cg;
#pragma unroll
  for (int bn = 0; bn < 4; bn++) {
    {
      const int prow = wn * 128 + bn * 32 + (lane & 31);
      char* rowp = smem + prow * 512;
#pragma unroll
      for (int bm = 0; bm < 4; bm++) {
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
          const int c = wm * 128 + bm * 32 + 8 * qq + 4 * (lane >> 5);
          u32x2 o;
          o[0] = dev::bf16_pack2(acc[bm][bn][4 * qq + 0], acc[bm][bn][4 * qq + 1]);
          o[1] = dev::bf16_pack2(acc[bm][bn][4 * qq + 2], acc[bm][bn][4 * qq + 3]);
          *(u32x2*)(rowp + (((c >> 3) ^ (prow & 31)) << 4) + ((c & 4) << 1)) = o;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 64 / (THREADS / 32); it++) {
      const int r = it * (THREADS / 32) + (tid >> 5);  // 0..63
      const int prow = (r & 32) * 4 + bn * 32 + (r & 31);
      const char* rowp = smem + prow * 512;
      const u32x4 v = *(const u32x4*)(rowp + ((ch ^ (prow & 31)) << 4));
      const uint32_t base = otab[prow];
      __builtin_amdgcn_raw_buffer_store_b128(u4{v[0], v[1], v[2], v[3]}, rdx,
                                             cv ? base + (uint32_t)ch * 16u : dev::kOOB, 0,
                                             kStoreAux);
    }
  }
}

// Finalising kernel of a split-K launch: dX = bf16(sum of the S partial
// tiles in the workspace, in split order).  Workgroup = 8 position rows of
// one tile; thread = 8 channels (two 16-byte loads per partial, one 16-byte
// store).
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const GemmArgs a) {
  const int S = a.ksplit;
  const int T = blockIdx.x / (BN / 8);  // tile (its workgroups in the main launch: T*S ...)
  const int row = (blockIdx.x % (BN / 8)) * 8 + (threadIdx.x >> 5);
  const int q = threadIdx.x & 31;
  const int t0 = T * S;
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
  const int p = n0 + row;
  const int c = m0 + 8 * q;
  if (p >= npos || c >= a.Cg) return;

  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const char* blk = (const char*)a.ws + (size_t)t0 * (BM * BN * 4) + row * 1024 + q * 32;
  for (int sp = 0; sp < S; sp++) {
    const f32x4 lo = *(const f32x4*)(blk + (size_t)sp * (BM * BN * 4));
    const f32x4 hi = *(const f32x4*)(blk + (size_t)sp * (BM * BN * 4) + 16);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[i] += lo[i];
      v[4 + i] += hi[i];
    }
  }
  const int n = p / npix_img;
  const int rr = p - n * npix_img;
  const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
  const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
  const uint32_t off = (uint32_t)(((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg + c) * 2u;
  const u4 o = {dev::bf16_pack2(v[0], v[1]), dev::bf16_pack2(v[2], v[3]), dev::bf16_pack2(v[4], v[5]),
                dev::bf16_pack2(v[6], v[7])};
  __builtin_amdgcn_raw_buffer_store_b128(o, dev::rsrc(a.dx, a.dx_bytes), off, 0, 0);
}

}  // namespace

int launch_splitk_finalize(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&splitk_finalize_kernel, dim3((unsigned)grid), dim3(256),
                              args, 0, (hipStream_t)stream);
}

int launch_nhwc_bf16(const GemmArgs& a, int64_t grid, void* stream) {
  const void* dy = a.dy;
  const void* w = a.w;
  void* dx = a.dx;
  uint32_t dyb = a.dy_bytes, wb = a.w_bytes, dxb = a.dx_bytes;
  int32_t npos = a.num_sub > 0 ? a.N * a.sub[0].pos_h * a.sub[0].pos_w : 0;
  int32_t tiles = a.total_tiles;
  void* args[] = {&dy, &w, &dx, &dyb, &wb, &dxb, &npos, &tiles, const_cast<GemmArgs*>(&a)};
  const void* k = a.ksplit > 1          ? (const void*)&igemm_nhwc_bf16_kernel<true, 0, 0, false>
                  : a.static_shape == 2 ? (const void*)&igemm_nhwc_bf16_kernel<false, 64, 1, true>
                  : a.static_shape == 1 ? (const void*)&igemm_nhwc_bf16_kernel<false, 64, 1, false>
                                        : (const void*)&igemm_nhwc_bf16_kernel<false, 0, 0, false>;
  return (int)hipLaunchKernel(k, dim3((unsigned)grid), dim3(THREADS), args, 0, (hipStream_t)stream);
}

}  // namespace cbd
