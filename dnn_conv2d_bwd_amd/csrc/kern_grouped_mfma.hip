// kern_grouped_mfma.hip -- grouped backward-data, bf16, C/G == K/G == 4,
// G in {32, 64}, on the 16-block 4x4x4 bf16 MFMA.
//
// Same row pipeline as kern_grouped_pipe.hip (a workgroup walks R output
// rows of one class and image; dY rows stream through an LDS ring of
// taps_h + 1 rows filled by LDS-DMA), over a block of CB positions of each
// row (the planner cuts wide rows so that several workgroups fit a compute
// unit's LDS), but the per-group 4x4 products run on
// the matrix cores: v_mfma_f32_4x4x4_16b_bf16 computes 16 independent
// 4x4x4 products, block b on lanes 4b..4b+3.  With
//   A_b = the group's filter tap transposed (4 output channels x 4 dY
//         channels; lane 4b+m holds row m, i.e. W[k = 0..3][c = m]),
//   B_b = dY at four positions (lane 4b+n holds dY[position n][k = 0..3],
//         the 8 bytes of the group at that pixel),
// D_b[m][n] lands in lane 4b+n, register m: the group's four dX channels at
// position n, stored as one 8-byte write.  A tap is one MFMA accumulating
// into D, so a quad of positions of 16 groups costs NT MFMAs (8 cycles
// each) where the dot-product kernel spends 8*NT v_dot2 per position pair.
//
// Lane layout: block b = group (set*16 + b), n = position within a quad of
// four consecutive class positions.  Waves split the G/16 group sets and
// the quads of a row.
//
// LDS bank conflicts: the four positions of a block sit one pixel (256 or
// 512 bytes) apart, i.e. on the same banks, so the copy XORs the 16-byte
// chunk index inside each pixel with 4*(column & 3): the 32 lanes of a
// half-wave then hit 64 distinct banks.
//
// dX goes out through LDS: each row's results are written (same swizzle)
// into an output row buffer after the ring, and the next row writes that
// buffer to dX as whole pixels, 16 bytes per lane, right after its opening
// barrier.  In the MFMA lane layout one store would cover only 128-byte
// halves of four pixels, which HBM absorbs at about 60% of the rate of
// whole-pixel stores; and issuing a row's stores one row late gives them a
// row of compute to drain before the wait at the next barrier (loads and
// stores share one counter).
#include "cbd_device.h"
#include "cbd_geo.h"
#include "cbd_internal.h"
#include "generic_shapes.h"

namespace cbd {
namespace {

// Cache policy of the dX stores: sc0 sc1 (bits 0 and 4 of the buffer_store
// cache-policy operand), written through instead of held dirty in L2.
// Measured on the 32-group 3x3 problems (graph / cold-cache us): stride 2
// 13.1 / 18.4 -> 11.7 / 17.1, stride 1 20.1 / 25.3 -> 19.0 / 24.8; the
// non-temporal hint alone, or with sc0 sc1, was slower cold on stride 1.
#ifndef CBD_GROUPED_STORE_AUX
#define CBD_GROUPED_STORE_AUX 17
#endif
constexpr int kStoreAux = CBD_GROUPED_STORE_AUX;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ s16x4 as_s16x4(uint32_t lo, uint32_t hi) {
  const u32x2 v = {lo, hi};
  return __builtin_bit_cast(s16x4, v);
}

template <int G, int NT, class Geo>
__device__ __forceinline__ void mfma_rows(const GemmArgs& a, const void* dy_p, const void* w_p, void* dx_p,
                                          const SubDesc& s, char* ring, int n, int th0, int th1, int tb,
                                          int seg) {
  constexpr int CG = 4, ES = 2;
  constexpr int PIXB = G * CG * ES;  // bytes per NHWC pixel: 256 or 512
  constexpr int PSHIFT = G == 32 ? 8 : 9;
  constexpr int NSETS = G / 16;      // sets of 16 groups
  constexpr int WPS = 4 / NSETS;     // waves per set
  static_assert(PIXB == 1 << PSHIFT && NSETS * WPS == 4, "G must be 32 or 64");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = wave % NSETS, wq = wave / NSETS;
  const int g = set * 16 + (lane >> 2);
  const int nn = lane & 3;

  const int Hi = Geo::Hi(a), Wi = Geo::Wi(a), Ho = Geo::Ho(a), Wo = Geo::Wo(a);
  const int Sh = Geo::Sh(a), Sw = Geo::Sw(a), Xf = Geo::X(a), delta_w = Geo::delta_w(a);
  const int span = delta_w * (s.taps_w - 1);
  const int col0 = s.beta_w - span + tb;  // dY column of staged column 0
  const int rowb = (seg + span) * PIXB;
  // Slots (whole KiB) also cover the 3 columns past the row that a partial
  // quad reads.
  const int ni = __builtin_amdgcn_readfirstlane((rowb + 3 * PIXB + 1023) >> 10);
  const int slotb = ni << 10;
  const int nslot = s.taps_h + 1;

  const i32x4 dyd = {(int)(uint32_t)(uintptr_t)dy_p, (int)(((uintptr_t)dy_p >> 32) & 0xffff),
                     (int)Geo::dy_bytes(a), 0x00020000};
  const auto rw = dev::rsrc(w_p, Geo::w_bytes(a));
  const auto rdx = dev::rsrc(dx_p, Geo::dx_bytes(a));
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  const int nquads = (seg + 3) >> 2;
  char* const out = ring + nslot * slotb;  // output row buffer: 4*nquads pixels
  constexpr int CPP = PIXB / 16;           // 16-byte chunks per pixel

  // Write the results of dX row `hrow` (class row) from the output buffer:
  // chunk j = pixel j / CPP, chunk j % CPP (stored at the swizzled place).
  auto flush_row = [&](int hrow) {
    const uint32_t xr = (uint32_t)((n * Hi + s.phase_h + Sh * hrow) * Wi) * (uint32_t)PIXB;
    const int nchunk = seg * CPP;
    for (int j = tid; j < nchunk; j += kGroupedThreads) {
      const int px = j / CPP, c = j - px * CPP;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = *(const u32x4*)(out + px * PIXB + ((c ^ ((px & 3) << 2)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, rdx, xr + ((uint32_t)(s.phase_w + Sw * (tb + px)) << PSHIFT) + (uint32_t)(c << 4), 0, kStoreAux);
    }
  };

  // Copy dY row ho into ring slot sl: LDS chunk lc of column col holds
  // global chunk lc ^ 4*(col & 3) of that pixel; zeros off dY's edge and
  // past the row.  ni KiB-instructions (64 lanes x 16 bytes), dealt to the
  // waves round-robin.
  auto copy_row = [&](int ho, int sl) {
    const bool hok = ho >= 0 && ho < Ho;
    const int rpix = (n * Ho + ho) * Wo;
    for (int i = wave; i < ni; i += 4) {
      const int b = (i << 10) + (lane << 4);
      const int col = b >> PSHIFT;
      const int wo = col0 + col;
      const int gc = ((b & (PIXB - 1)) >> 4) ^ ((col & 3) << 2);
      const bool ok = hok && b < rowb && wo >= 0 && wo < Wo;
      const uint32_t off = ok ? (uint32_t)(rpix + wo) * (uint32_t)PIXB + (uint32_t)(gc << 4) : dev::kOOB;
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(ring_base + (uint32_t)(sl * slotb + (i << 10)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                   :: "s"(m0v), "v"(off), "s"(dyd) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  int top = (th0 + s.beta_h) % nslot;  // slot of dY row th + beta_h
  if (top < 0) top += nslot;
  auto back = [&](int j) { return top - j < 0 ? top - j + nslot : top - j; };

  for (int jh = s.taps_h - 1; jh >= 0; jh--) copy_row(th0 + s.beta_h - jh, back(jh));

  // A operands: lane 4b+m holds W[g*4 + k][ty][tx][m], k = 0..3, per tap.
  const int YX = Geo::Y(a) * Xf;
  s16x4 wa[NT];
  int jhs[NT], cshift[NT];  // tap row; column shift span - delta_w*jw
#pragma unroll
  for (int tp = 0; tp < NT; tp++) {
    const int jh = tp / s.taps_w;
    const int jw = tp - jh * s.taps_w;
    const int ty = s.cls_h + Geo::tstep_h(a) * jh, tx = s.cls_w + Geo::tstep_w(a) * jw;
    jhs[tp] = jh;
    cshift[tp] = span - delta_w * jw;
    uint32_t e[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
      e[k] = __builtin_amdgcn_raw_buffer_load_b16(rw, (uint32_t)(((g * CG + k) * YX + ty * Xf + tx) * CG + nn) * ES, 0, 0);
    wa[tp] = as_s16x4(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
  }

  // The lane's first position and its per-tap LDS byte address within a
  // slot (quads further along the row add multiples of 4*WPS pixels, which
  // keep column & 3 and therefore the swizzle).
  const int tw0 = wq * 4 + nn;
  int lofs[NT];
#pragma unroll
  for (int tp = 0; tp < NT; tp++) {
    const int col = tw0 + cshift[tp];
    lofs[tp] = (col << PSHIFT) + ((((g >> 1) ^ ((col & 3) << 2))) << 4) + ((g & 1) << 3);
  }
  // The lane's byte in the output row buffer at its first position.
  const int oofs = (tw0 << PSHIFT) + (((g >> 1) ^ (nn << 2)) << 4) + ((g & 1) << 3);

  for (int th = th0; th < th1; th++) {
    // This wave's copies of row th + beta_h have landed and its LDS reads
    // and writes of row th-1 are done; the barrier extends both to the
    // workgroup.  (The wait also covers this wave's dX stores issued at the
    // start of row th-1: loads and stores share the counter.)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int next = top + 1 == nslot ? 0 : top + 1;
    if (th + 1 < th1) copy_row(th + 1 + s.beta_h, next);
    if (th > th0) flush_row(th - 1);
    const char* base[NT];
#pragma unroll
    for (int tp = 0; tp < NT; tp++) base[tp] = ring + back(jhs[tp]) * slotb + lofs[tp];
    // Every wave's reads of the output buffer (flush above) are done before
    // any wave overwrites it below.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // Two quads per pass; the second may lie past the row (uniform test).
    for (int qd = wq; qd < nquads; qd += 2 * WPS) {
      const bool two = qd + WPS < nquads;
      const int o0 = (qd - wq) * 4 * PIXB;
      const int o1 = two ? o0 + 4 * WPS * PIXB : o0;
      u32x2 v0[NT], v1[NT];
#pragma unroll
      for (int tp = 0; tp < NT; tp++) {
        v0[tp] = *(const u32x2*)(base[tp] + o0);
        v1[tp] = *(const u32x2*)(base[tp] + o1);
      }
      f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tp = 0; tp < NT; tp++) {
        d0 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(wa[tp], __builtin_bit_cast(s16x4, v0[tp]), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(wa[tp], __builtin_bit_cast(s16x4, v1[tp]), d1, 0, 0, 0);
      }
      const u32x2 p0 = {dev::bf16_pack2(d0[0], d0[1]), dev::bf16_pack2(d0[2], d0[3])};
      const u32x2 p1 = {dev::bf16_pack2(d1[0], d1[1]), dev::bf16_pack2(d1[2], d1[3])};
      *(u32x2*)(out + oofs + o0) = p0;
      if (two) *(u32x2*)(out + oofs + o1) = p1;
    }
    top = next;
  }
  // The last row: its results are in the buffer after this barrier.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  flush_row(th1 - 1);
}

template <int G, class Geo>
__global__ __launch_bounds__(kGroupedThreads) void grouped_mfma_kernel(const void* dy_p, const void* w_p,
                                                                      void* dx_p, const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  if constexpr (!Geo::kStatic) dev::prefetch_args(a);
  const int t = dev::chunked_block(blockIdx.x, Geo::total_tiles(a));
  const SubDesc s = Geo::sub(a, t);
  // (image, row block, column block), column blocks innermost
  const int R = Geo::grp_rows(a), CB = Geo::grp_cols(a);
  const int rblocks = (s.pos_h + R - 1) / R;
  const int cblocks = (s.pos_w + CB - 1) / CB;
  const int local = t - s.tile_begin;
  const int n = local / (rblocks * cblocks);
  const int rem = local - n * rblocks * cblocks;
  const int rb = rem / cblocks, cb = rem - (rem / cblocks) * cblocks;
  const int th0 = rb * R;
  const int th1 = th0 + R < s.pos_h ? th0 + R : s.pos_h;
  const int tb = cb * CB;
  const int seg = tb + CB < s.pos_w ? CB : s.pos_w - tb;
  static_assert(kGroupedMaxTaps == 9, "the switch below covers 1..9 taps");
  switch (s.taps_h * s.taps_w) {
    case 1: mfma_rows<G, 1, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 2: mfma_rows<G, 2, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 3: mfma_rows<G, 3, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 4: mfma_rows<G, 4, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 5: mfma_rows<G, 5, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 6: mfma_rows<G, 6, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 7: mfma_rows<G, 7, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    case 8: mfma_rows<G, 8, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
    default: mfma_rows<G, 9, Geo>(a, dy_p, w_p, dx_p, s, ring, n, th0, th1, tb, seg); break;
  }
}

// Merged phases (stride 2 x 2, each of the four phases a class, taps one dY
// row and column apart): a workgroup walks R class rows th of one image and a
// block of CB class columns, and for each computes all four phases, i.e. dX
// rows 2th and 2th+1 over dX columns 2tb ... 2(tb+seg)-1.  The ring holds the
// union of the dY rows the phases read (th + lo_h ... th + hi_h, one new row
// per class row) over the union of their columns, so every dY row is copied
// into LDS once instead of once per phase, and the output buffer holds two
// whole dX row segments, stored as contiguous 16-byte chunks.  Up to four taps
// per class (filters up to 4 x 4).  The products are the per-class kernel's
// (same MFMA, same tap order per class), so the bits are the same.
template <int G, class Geo>
__global__ __launch_bounds__(kGroupedThreads) void grouped_mfma_merged_kernel(const void* dy_p, const void* w_p,
                                                                             void* dx_p, const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  if constexpr (!Geo::kStatic) dev::prefetch_args(a);
  constexpr int CG = 4, ES = 2;
  constexpr int PIXB = G * CG * ES;  // bytes per NHWC pixel: 256 or 512
  constexpr int PSHIFT = G == 32 ? 8 : 9;
  constexpr int NSETS = G / 16;  // 16 groups per MFMA
  constexpr int WPS = 4 / NSETS;  // waves per group set
  constexpr int CPP = PIXB / 16;  // 16-byte chunks per pixel
  constexpr int CPPS = PSHIFT - 4;
  constexpr int NC = 4, NTM = 4;  // classes; taps per class at most
  static_assert(PIXB == 1 << PSHIFT && NSETS * WPS == 4, "G must be 32 or 64");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = wave % NSETS, wq = wave / NSETS;
  const int g = set * 16 + (lane >> 2);
  const int nn = lane & 3;

  const int Hi = Geo::Hi(a), Wi = Geo::Wi(a), Ho = Geo::Ho(a), Wo = Geo::Wo(a), Xf = Geo::X(a);
  const int YX = Geo::Y(a) * Xf;
  // The union of the classes' dY row and column offsets: class row th reads
  // dY rows th + beta_h - jh, class column tw reads dY columns tw + beta_w - jw.
  int lo_h = 1 << 30, hi_h = -(1 << 30), lo_w = 1 << 30, hi_w = -(1 << 30), PH = 0, PW = 0;
#pragma unroll
  for (int i = 0; i < NC; i++) {
    const SubDesc c = Geo::sub_at(a, i);
    lo_h = min(lo_h, c.beta_h - (c.taps_h - 1));
    hi_h = max(hi_h, c.beta_h);
    lo_w = min(lo_w, c.beta_w - (c.taps_w - 1));
    hi_w = max(hi_w, c.beta_w);
    PH = max(PH, c.pos_h);
    PW = max(PW, c.pos_w);
  }
  const int span_h = hi_h - lo_h, span_w = hi_w - lo_w;

  // (image, row block, column block), column blocks innermost
  const int R = Geo::grp_rows(a), CB = Geo::grp_cols(a);
  const int rblocks = (PH + R - 1) / R;
  const int cblocks = (PW + CB - 1) / CB;
  const int t = dev::chunked_block(blockIdx.x, Geo::total_tiles(a));
  const int n = t / (rblocks * cblocks);
  const int rem = t - n * rblocks * cblocks;
  const int rbk = rem / cblocks, cbk = rem - (rem / cblocks) * cblocks;
  const int th0 = rbk * R;
  const int th1 = th0 + R < PH ? th0 + R : PH;
  const int tb = cbk * CB;
  const int seg = tb + CB < PW ? CB : PW - tb;

  const int col0 = tb + lo_w;  // dY column of staged column 0
  const int rowb = (seg + span_w) * PIXB;
  // Slots (whole KiB) also cover the 3 columns past the row that a partial
  // quad reads.
  const int ni = __builtin_amdgcn_readfirstlane((rowb + 3 * PIXB + 1023) >> 10);
  const int slotb = ni << 10;
  const int nslot = span_h + 2;
  const int nquads = (seg + 3) >> 2;
  const int orow = 8 * nquads * PIXB;      // one dX row segment of the output buffer
  char* const out = ring + nslot * slotb;  // two of them: phases 0 and 1 along H

  const i32x4 dyd = {(int)(uint32_t)(uintptr_t)dy_p, (int)(((uintptr_t)dy_p >> 32) & 0xffff),
                     (int)Geo::dy_bytes(a), 0x00020000};
  const auto rw = dev::rsrc(w_p, Geo::w_bytes(a));
  const auto rdx = dev::rsrc(dx_p, Geo::dx_bytes(a));
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;

  // Write dX rows 2 thr and 2 thr + 1 (columns 2tb ...) from the output
  // buffer: pixel px of row r holds its chunk c at chunk c ^ 4*((px/2) & 3).
  const int rchunks = 2 * seg * CPP;
  auto flush_rows = [&](int thr) {
    for (int j = tid; j < 2 * rchunks; j += kGroupedThreads) {
      const int r = j >= rchunks ? 1 : 0;
      const int q = j - r * rchunks;
      const int px = q >> CPPS, c = q & (CPP - 1);
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 v = *(const u32x4*)(out + r * orow + px * PIXB + ((c ^ (((px >> 1) & 3) << 2)) << 4));
      const int hi = 2 * thr + r, wi = 2 * tb + px;
      const bool ok = hi < Hi && wi < Wi;
      __builtin_amdgcn_raw_buffer_store_b128(
          v, rdx, ok ? ((uint32_t)((n * Hi + hi) * Wi + wi) << PSHIFT) + (uint32_t)(c << 4) : dev::kOOB, 0,
          kStoreAux);
    }
  };

  // Copy dY row ho into ring slot sl (chunk swizzle as in mfma_rows).
  auto copy_row = [&](int ho, int sl) {
    const bool hok = ho >= 0 && ho < Ho;
    const int rpix = (n * Ho + ho) * Wo;
    for (int i = wave; i < ni; i += 4) {
      const int b = (i << 10) + (lane << 4);
      const int col = b >> PSHIFT;
      const int wo = col0 + col;
      const int gc = ((b & (PIXB - 1)) >> 4) ^ ((col & 3) << 2);
      const bool ok = hok && b < rowb && wo >= 0 && wo < Wo;
      const uint32_t off = ok ? (uint32_t)(rpix + wo) * (uint32_t)PIXB + (uint32_t)(gc << 4) : dev::kOOB;
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(ring_base + (uint32_t)(sl * slotb + (i << 10)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                   :: "s"(m0v), "v"(off), "s"(dyd) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  // Slot of dY row th + hi_h (the newest row a class row reads).
  int top = (th0 + hi_h) % nslot;
  if (top < 0) top += nslot;
  auto back = [&](int j) { return top - j < 0 ? top - j + nslot : top - j; };
  for (int j = span_h; j >= 0; j--) copy_row(th0 + hi_h - j, back(j));

  // Per class and tap: the A operand (lane 4b+m: W[g*4 + k][ty][tx][m]),
  // the tap's ring row (counted back from the newest) and the lane's LDS
  // byte offset within a slot at its first position; per class, the lane's
  // byte in the output buffer.
  s16x4 wa[NC][NTM];
  int rback[NC][NTM], lofs[NC][NTM], oofs[NC], ntap[NC];
  const int tw0 = wq * 4 + nn;
#pragma unroll
  for (int i = 0; i < NC; i++) {
    const SubDesc c = Geo::sub_at(a, i);
    ntap[i] = c.taps_h * c.taps_w;
    oofs[i] = c.phase_h * orow + ((2 * tw0 + c.phase_w) << PSHIFT) + (((g >> 1) ^ (nn << 2)) << 4) + ((g & 1) << 3);
#pragma unroll
    for (int tp = 0; tp < NTM; tp++) {
      const int jh = tp / c.taps_w, jw = tp - (tp / c.taps_w) * c.taps_w;
      const int ty = c.cls_h + Geo::tstep_h(a) * jh, tx = c.cls_w + Geo::tstep_w(a) * jw;
      rback[i][tp] = hi_h - (c.beta_h - jh);
      const int col = tw0 + c.beta_w - jw - lo_w;
      lofs[i][tp] = (col << PSHIFT) + ((((g >> 1) ^ ((col & 3) << 2))) << 4) + ((g & 1) << 3);
      uint32_t e[4] = {0u, 0u, 0u, 0u};
      if (tp < ntap[i]) {
#pragma unroll
        for (int k = 0; k < 4; k++)
          e[k] = __builtin_amdgcn_raw_buffer_load_b16(rw, (uint32_t)(((g * CG + k) * YX + ty * Xf + tx) * CG + nn) * ES,
                                                      0, 0);
      }
      wa[i][tp] = as_s16x4(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
    }
  }

  for (int th = th0; th < th1; th++) {
    // This wave's copies of row th + hi_h have landed and its LDS reads and
    // writes of class row th-1 are done; the barrier extends both to the
    // workgroup.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int next = top + 1 == nslot ? 0 : top + 1;
    if (th + 1 < th1) copy_row(th + 1 + hi_h, next);
    if (th > th0) flush_rows(th - 1);
    const char* base[NC][NTM];
#pragma unroll
    for (int i = 0; i < NC; i++)
#pragma unroll
      for (int tp = 0; tp < NTM; tp++) base[i][tp] = ring + back(rback[i][tp]) * slotb + lofs[i][tp];
    // Every wave's reads of the output buffer (flush above) are done before
    // any wave overwrites it below.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int qd = wq; qd < nquads; qd += WPS) {
      const int o = (qd - wq) * 4 * PIXB;
      f32x4 d[NC];
#pragma unroll
      for (int i = 0; i < NC; i++) d[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tp = 0; tp < NTM; tp++) {
#pragma unroll
        for (int i = 0; i < NC; i++) {
          if (tp < ntap[i]) {
            const u32x2 v = *(const u32x2*)(base[i][tp] + o);
            d[i] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(wa[i][tp], __builtin_bit_cast(s16x4, v), d[i], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NC; i++) {
        const u32x2 pk = {dev::bf16_pack2(d[i][0], d[i][1]), dev::bf16_pack2(d[i][2], d[i][3])};
        *(u32x2*)(out + oofs[i] + 2 * o) = pk;
      }
    }
    top = next;
  }
  // The last class row: its results are in the buffer after this barrier.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  flush_rows(th1 - 1);
}

template <int G, class Geo = DynGeo>
int launch_g(const GemmArgs& a, int64_t grid, void* stream) {
  const void* dy = a.dy;
  const void* w = a.w;
  void* dx = a.dx;
  void* args[] = {&dy, &w, &dx, const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_mfma_kernel<G, Geo>, dim3((unsigned)grid),
                              dim3(kGroupedThreads), args, (size_t)a.grp_lds, (hipStream_t)stream);
}

// A shape-specialised instance (StatGeo<T>, the group count from T).
int launch_static(const GemmArgs& a, int64_t grid, void* stream) {
  switch (a.static_id) {
#define CBD_CASE(i, T, name) \
  case i:                    \
    return launch_g<T::k.G, StatGeo<T>>(a, grid, stream);
    CBD_GROUPED_SHAPE_LIST(CBD_CASE)
#undef CBD_CASE
  }
  return (int)hipErrorInvalidValue;
}

template <int G, class Geo = DynGeo>
int launch_merged(const GemmArgs& a, int64_t grid, void* stream) {
  const void* dy = a.dy;
  const void* w = a.w;
  void* dx = a.dx;
  void* args[] = {&dy, &w, &dx, const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_mfma_merged_kernel<G, Geo>, dim3((unsigned)grid),
                              dim3(kGroupedThreads), args, (size_t)a.grp_lds, (hipStream_t)stream);
}

}  // namespace

int launch_grouped_mfma(const GemmArgs& a, int64_t grid, void* stream) {
  if (a.Cg != 4) return (int)hipErrorInvalidValue;
  if (a.grp_merged) {
    if (a.num_sub != 4) return (int)hipErrorInvalidValue;
    switch (a.G) {
      case 32: return launch_merged<32>(a, grid, stream);
      case 64: return launch_merged<64>(a, grid, stream);
      default: return (int)hipErrorInvalidValue;
    }
  }
  if (a.static_shape == 2) return launch_static(a, grid, stream);
  switch (a.G) {
    case 32: return launch_g<32>(a, grid, stream);
    case 64: return launch_g<64>(a, grid, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace cbd
