// kern_grouped_wide.hip -- grouped backward-data, bf16, C/G == K/G in
// {8, 16, 32}, on the 16x16x16 bf16 MFMA.
//
// Per group the class sum is a small GEMM: dX[c][position] = sum over taps
// and k of W[tap][k][c] * dY[position + tap][k], with c and k < C/G.  Here
// v_mfma_f32_16x16x16_bf16 takes A = the group's filter tap transposed
// (16 output channels x 16 dY channels; lane l holds A[l % 16][4(l/16) ..
// 4(l/16)+3]) and B = dY at 16 consecutive class positions (lane l holds
// B[4(l/16) .. +3][l % 16], i.e. 8 bytes of the group's channels at
// position l % 16); D[c][n] lands in lane n + 16 (c/4), register c % 4:
// four consecutive dX channels of one position.  C/G = 32 takes two
// channel halves times two k halves; C/G = 8 runs as C/G = 16 on pairs of
// adjacent groups (their 16 channels are contiguous in a pixel) with a
// block-diagonal A: the two groups' 8x8 taps on the diagonal, zeros off it.
// The lane layout was checked with a one-wave probe.
//
// Workgroup = (class, image, R output rows, a block of groups whose
// channels make a 256-byte slice of each pixel, a block of CB positions):
// 8 groups of 16 channels or 4 of 32, one or two per wave, so the filter
// taps stay in registers.  The row pipeline is that of kern_grouped_mfma.hip:
// dY rows of the slice stream through an LDS ring of taps_h + 1 rows filled
// by LDS-DMA, results go through an LDS row buffer and leave one row late
// as 256-byte slices, 16 bytes per lane.  Both LDS buffers XOR the 16-byte
// chunk index inside a pixel's slice with (column & 15): the 16 positions
// read by one MFMA operand are then on distinct banks.  Lanes whose
// position lies past the block read a valid column (clamped) and their
// results are never written out.
#include "cbd_device.h"
#include "cbd_internal.h"

// Cache policy of the dX stores: sc0 sc1 (written through instead of held
// dirty in L2), as in the 4-channel MFMA kernel.  Measured (graph us): 8
// channels per group at 56x56 stride 1 32.5 -> 31.0, 16 channels stride 2
// 27.5 -> 23.2, 32 channels 28x28 stride 1 34.7 -> 33.6.
#ifndef CBD_WIDE_STORE_AUX
#define CBD_WIDE_STORE_AUX 17
#endif

namespace cbd {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int SB = 256;  // bytes of a pixel's group slice handled by one workgroup

// CG: channels per (virtual) group, 16 or 32; PAIR8: the problem's groups
// have 8 channels and a virtual group is two of them.
template <int CG, bool PAIR8, int NT>
__device__ __forceinline__ void wide_rows(const GemmArgs& a, const SubDesc& s, char* ring, int n, int gb,
                                          int th0, int th1, int tb, int seg) {
  constexpr int ES = 2;
  constexpr int GB = SB / (CG * ES);  // groups per workgroup: 8 or 4
  constexpr int GPW = GB / 4;         // groups per wave: 2 or 1
  constexpr int H = CG / 16;          // channel (and k) halves
  static_assert(GB * CG * ES == SB && GPW * 4 == GB, "C/G must be 16 or 32");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 15, lq = lane >> 4;  // position within 16, channel quad

  const int pixb = a.C * ES;
  const int span = a.delta_w * (s.taps_w - 1);
  const int col0 = s.beta_w - span + tb;
  const int rowb = (seg + span) * SB;
  const int ni = __builtin_amdgcn_readfirstlane((rowb + 1023) >> 10);
  const int slotb = ni << 10;
  const int nslot = s.taps_h + 1;
  const int nchunks = (seg + 15) >> 4;
  char* const out = ring + nslot * slotb;  // output row buffer: 16*nchunks pixels

  const i32x4 dyd = {(int)(uint32_t)(uintptr_t)a.dy, (int)(((uintptr_t)a.dy >> 32) & 0xffff),
                     (int)a.dy_bytes, 0x00020000};
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
  const uint32_t slice = (uint32_t)(gb * SB);  // byte of the slice within a pixel

  // Copy dY row ho into ring slot sl: LDS chunk lc of column col holds the
  // slice's chunk lc ^ (col & 15); zeros off dY's edge.  KiB instructions
  // dealt to the waves round-robin.
  auto copy_row = [&](int ho, int sl) {
    const bool hok = ho >= 0 && ho < a.Ho;
    const int rpix = (n * a.Ho + ho) * a.Wo;
    for (int i = wave; i < ni; i += 4) {
      const int b = (i << 10) + (lane << 4);
      const int col = b >> 8;
      const int gc = ((b >> 4) & 15) ^ (col & 15);
      const int wo = col0 + col;
      const bool ok = hok && b < rowb && wo >= 0 && wo < a.Wo;
      const uint32_t off = ok ? (uint32_t)(rpix + wo) * (uint32_t)pixb + slice + (uint32_t)(gc << 4) : dev::kOOB;
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(ring_base + (uint32_t)(sl * slotb + (i << 10)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0"
                   :: "s"(m0v), "v"(off), "s"(dyd) : "memory", "m0");
#pragma clang diagnostic pop
    }
  };

  // dX row hrow of the block from the output buffer: 256-byte slices.
  auto flush_row = [&](int hrow) {
    const uint32_t xr = (uint32_t)((n * a.Hi + s.phase_h + a.Sh * hrow) * a.Wi);
    for (int j = tid; j < seg * 16; j += kGroupedThreads) {
      const int px = j >> 4, c = j & 15;
      const u32x4 v = *(const u32x4*)(out + px * SB + ((c ^ (px & 15)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(
          v, rdx, (xr + (uint32_t)(s.phase_w + a.Sw * (tb + px))) * (uint32_t)pixb + slice + (uint32_t)(c << 4),
          0, CBD_WIDE_STORE_AUX);
    }
  };

  int top = (th0 + s.beta_h) % nslot;  // slot of dY row th + beta_h
  if (top < 0) top += nslot;
  auto back = [&](int j) { return top - j < 0 ? top - j + nslot : top - j; };

  for (int jh = s.taps_h - 1; jh >= 0; jh--) copy_row(th0 + s.beta_h - jh, back(jh));

  // A operands: group gl = wave*GPW + j (global gb*GB + gl); lane l holds
  // W[g*CG + 16 kh + 4 lq + e][ty][tx][16 ch + ln], e = 0..3 (paired groups
  // of 8: the entry of real group 2g + ln/8 where k and c fall in the same
  // group, 0 elsewhere).  W is c-contiguous; for the paired groups of 8 the
  // lanes of a pair (ln even, ln + 1) each read two 4-byte words, channels
  // (ln & ~1, +1) of k rows 2 (ln & 1) + {0, 1}, and swap them (DPP): the
  // even lane keeps the low halves of all four rows, the odd lane the high
  // halves, with half the loads of one 2-byte gather per element (8
  // channels per group, N = 32: 7x7 7.0 -> 6.3 us, 28x28 14.3 -> 13.1).
  const int YX = a.Y * a.X;
  const int odd = ln & 1, hsh = 16 * odd;
  s16x4 wa[GPW][NT][H][H];
  int jhs[NT], cshift[NT];
#pragma unroll
  for (int tp = 0; tp < NT; tp++) {
    const int jh = tp / s.taps_w;
    jhs[tp] = jh;
    cshift[tp] = span - a.delta_w * (tp - jh * s.taps_w);
  }
  // The words of tap tp: k rows 4 lq + 2 odd + i, channels (ln & ~1, +1).
  // Taps are pipelined one deep (tap tp + 1's loads in flight while tap
  // tp's are swapped and packed), which keeps the registers this takes to
  // two taps' words.
  typedef uint32_t TapWords[GPW][H][H][2];
  auto load_tap = [&](int tp, TapWords& wl) {
    const int jh = tp / s.taps_w;
    const int jw = tp - jh * s.taps_w;
    const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
#pragma unroll
    for (int j = 0; j < GPW; j++) {
      const int g = gb * GB + wave * GPW + j;
#pragma unroll
      for (int kh = 0; kh < H; kh++)
#pragma unroll
        for (int ch = 0; ch < H; ch++)
#pragma unroll
          for (int i = 0; i < 2; i++) {
            const int q = 2 * odd + i;
            const int k = 4 * lq + q;  // 0..15 within the pair; k / 8 == lq / 2 for all four rows
            const bool on = (k >> 3) == (ln >> 3);
            const int rg = 2 * g + (ln >> 3);
            wl[j][kh][ch][i] = __builtin_amdgcn_raw_buffer_load_b32(
                rw, on ? (uint32_t)(((rg * 8 + (k & 7)) * YX + ty * a.X + tx) * 8 + (ln & 6)) * ES : dev::kOOB,
                0, 0);
          }
    }
  };
  // Partner's words (lane ^ 1, DPP quad_perm [1, 0, 3, 2]); the even lane
  // takes the low halves (its channel) of rows 0, 1 (its own words) and 2, 3
  // (the partner's), the odd lane the high halves of rows 0, 1 (the
  // partner's) and 2, 3 (its own).
  auto half2 = [&](uint32_t x0, uint32_t x1) {
    return ((x0 >> hsh) & 0xffffu) | (((x1 >> hsh) & 0xffffu) << 16);
  };
  auto pack_tap = [&](int tp, const TapWords& wl) {
#pragma unroll
    for (int j = 0; j < GPW; j++)
#pragma unroll
      for (int kh = 0; kh < H; kh++)
#pragma unroll
        for (int ch = 0; ch < H; ch++) {
          const uint32_t w0 = wl[j][kh][ch][0], w1 = wl[j][kh][ch][1];
          const uint32_t p0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w0, 0xB1, 0xf, 0xf, false);
          const uint32_t p1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w1, 0xB1, 0xf, 0xf, false);
          const uint32_t a0 = odd ? p0 : w0, a1 = odd ? p1 : w1;  // rows 0, 1
          const uint32_t b0 = odd ? w0 : p0, b1 = odd ? w1 : p1;  // rows 2, 3
          const u32x2 v = {half2(a0, a1), half2(b0, b1)};
          wa[j][tp][kh][ch] = __builtin_bit_cast(s16x4, v);
        }
  };
  if constexpr (PAIR8) {
    TapWords wbuf[2];
    load_tap(0, wbuf[0]);
#pragma unroll
    for (int tp = 0; tp < NT; tp++) {
      if (tp + 1 < NT) load_tap(tp + 1, wbuf[(tp + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      pack_tap(tp, wbuf[tp & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // 16 or 32 channels: one 2-byte gather per element (the paired words
    // measured slower here: at 32 channels the kernel's registers rise
    // past what four waves per SIMD allow).
#pragma unroll
    for (int tp = 0; tp < NT; tp++) {
      const int jh = tp / s.taps_w;
      const int jw = tp - jh * s.taps_w;
      const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
#pragma unroll
      for (int j = 0; j < GPW; j++) {
        const int g = gb * GB + wave * GPW + j;
#pragma unroll
        for (int kh = 0; kh < H; kh++)
#pragma unroll
          for (int ch = 0; ch < H; ch++) {
            uint32_t e[4];
#pragma unroll
            for (int q = 0; q < 4; q++)
              e[q] = __builtin_amdgcn_raw_buffer_load_b16(
                  rw, (uint32_t)(((g * CG + 16 * kh + 4 * lq + q) * YX + ty * a.X + tx) * CG + 16 * ch + ln) * ES, 0,
                  0);
            const u32x2 v = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            wa[j][tp][kh][ch] = __builtin_bit_cast(s16x4, v);
          }
      }
    }
  }

  // Byte of (group j, k half kh, channel quad lq) in a pixel's slice.
  auto sbyte = [&](int j, int kh) { return (wave * GPW + j) * CG * ES + kh * 32 + lq * 8; };

  for (int th = th0; th < th1; th++) {
    // Copies of row th + beta_h landed and LDS reads/writes of row th-1
    // done (this wave), then for the workgroup.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int next = top + 1 == nslot ? 0 : top + 1;
    if (th + 1 < th1) copy_row(th + 1 + s.beta_h, next);
    if (th > th0) flush_row(th - 1);
    int sbase[NT];
#pragma unroll
    for (int tp = 0; tp < NT; tp++) sbase[tp] = back(jhs[tp]) * slotb;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int ck = 0; ck < nchunks; ck++) {
      const int tl = (ck << 4) + ln;             // local position of this lane
      const int tc = tl < seg ? tl : seg - 1;    // clamped for reads
#pragma unroll
      for (int j = 0; j < GPW; j++) {
        u32x2 bv[NT][H];
#pragma unroll
        for (int tp = 0; tp < NT; tp++) {
          const int col = tc + cshift[tp];
#pragma unroll
          for (int kh = 0; kh < H; kh++) {
            const int sb = sbyte(j, kh);
            bv[tp][kh] = *(const u32x2*)(ring + sbase[tp] + col * SB + ((((sb >> 4) ^ (col & 15))) << 4) + (sb & 15));
          }
        }
        f32x4 d[H];
#pragma unroll
        for (int ch = 0; ch < H; ch++) d[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tp = 0; tp < NT; tp++)
#pragma unroll
          for (int kh = 0; kh < H; kh++)
#pragma unroll
            for (int ch = 0; ch < H; ch++)
              d[ch] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wa[j][tp][kh][ch],
                                                                 __builtin_bit_cast(s16x4, bv[tp][kh]), d[ch], 0, 0, 0);
#pragma unroll
        for (int ch = 0; ch < H; ch++) {
          const int sb = sbyte(j, ch);  // channels 16 ch + 4 lq .. +3 of group j
          const u32x2 p = {dev::bf16_pack2(d[ch][0], d[ch][1]), dev::bf16_pack2(d[ch][2], d[ch][3])};
          *(u32x2*)(out + tl * SB + ((((sb >> 4) ^ (tl & 15))) << 4) + (sb & 15)) = p;
        }
      }
    }
    top = next;
  }
  // The last row: its results are in the buffer after this barrier.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  flush_row(th1 - 1);
}

// 32 channels per group: at most 128 VGPRs (four waves per SIMD, as many
// workgroups as LDS holds where the ring is small; the compiler's own choice
// was 133): 28x28 stride 2 22.5 -> 17.2 us, 14x14 stride 2 13.1 -> 10.5,
// 28x28 stride 1 33.4 -> 30.6 (N = 32), no spills.
template <int CG, bool PAIR8>
__global__ __launch_bounds__(kGroupedThreads, CG == 32 ? 4 : 1) void grouped_wide_kernel(const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char ring[];
  constexpr int GB = SB / ((PAIR8 ? 8 : CG) * 2);  // the problem's groups per workgroup
  dev::prefetch_args(a);
  const int t = dev::chunked_block(blockIdx.x, a.total_tiles);
  const SubDesc s = a.sub[dev::find_class(a, t)];
  // (image, row block, group block, column block), column blocks innermost
  const int R = a.grp_rows, CB = a.grp_cols;
  const int rblocks = (s.pos_h + R - 1) / R;
  const int gblocks = a.G / GB;
  const int cblocks = (s.pos_w + CB - 1) / CB;
  const int per_img = rblocks * gblocks * cblocks;
  const int local = t - s.tile_begin;
  const int n = local / per_img;
  int rem = local - n * per_img;
  const int rb = rem / (gblocks * cblocks);
  rem -= rb * gblocks * cblocks;
  const int gb = rem / cblocks, cb = rem - (rem / cblocks) * cblocks;
  const int th0 = rb * R;
  const int th1 = th0 + R < s.pos_h ? th0 + R : s.pos_h;
  const int tb = cb * CB;
  const int seg = tb + CB < s.pos_w ? CB : s.pos_w - tb;
  static_assert(kGroupedMaxTaps == 9, "the switch below covers 1..9 taps");
  switch (s.taps_h * s.taps_w) {
    case 1: wide_rows<CG, PAIR8, 1>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 2: wide_rows<CG, PAIR8, 2>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 3: wide_rows<CG, PAIR8, 3>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 4: wide_rows<CG, PAIR8, 4>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 5: wide_rows<CG, PAIR8, 5>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 6: wide_rows<CG, PAIR8, 6>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 7: wide_rows<CG, PAIR8, 7>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    case 8: wide_rows<CG, PAIR8, 8>(a, s, ring, n, gb, th0, th1, tb, seg); break;
    default: wide_rows<CG, PAIR8, 9>(a, s, ring, n, gb, th0, th1, tb, seg); break;
  }
}

template <int CG, bool PAIR8>
int launch_cg(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&grouped_wide_kernel<CG, PAIR8>, dim3((unsigned)grid),
                              dim3(kGroupedThreads), args, (size_t)a.grp_lds, (hipStream_t)stream);
}

}  // namespace

int launch_grouped_wide(const GemmArgs& a, int64_t grid, void* stream) {
  switch (a.Cg) {
    case 8: return launch_cg<16, true>(a, grid, stream);
    case 16: return launch_cg<16, false>(a, grid, stream);
    case 32: return launch_cg<32, false>(a, grid, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace cbd
