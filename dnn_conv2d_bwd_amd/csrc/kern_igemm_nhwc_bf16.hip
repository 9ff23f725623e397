// kern_igemm_nhwc_bf16.hip -- the large-problem family: NHWC dX / NHWK dY /
// KYXC W in bf16, f32 accumulation, bf16 result (the dtype contract of the
// BOO listing in fusilli issue #101: extf to f32, mulf/addf, truncf).
//
// Same per-residue-class GEMM as the generic family (kern_igemm_generic.hip),
// specialised for C/G % 8 == 0 and K/G % 64 == 0, laid out for gfx950:
//   * 256(M = c) x 256(N = positions) workgroup tiles, 32-wide k tiles;
//     512 threads = 8 waves in 2(M) x 4(N), each wave 128x64 = 4x2 blocks of
//     v_mfma_f32_32x32x16_bf16; two waves share each SIMD, so one wave's
//     memory-instruction stalls are covered by the other's MFMAs;
//   * both operands travel global -> LDS by buffer_load ... lds (no VGPR
//     staging, no VALU, no ds_write): lane l of an instruction fills 16 bytes
//     at slot l of a 1 KiB LDS block, so the row swizzle is applied by
//     choosing which global chunk each lane fetches;
//   * dY rows (position, 32 k = 64 B) are k-contiguous and feed the MFMA B
//     operand with ds_read_b128; W rows (k, 256 c = 512 B) stay c-contiguous
//     and ds_read_b64_tr_b16 transposes 4x4 bf16 blocks on the way out, giving
//     each lane the k-vector of one channel (MFMA A operand);
//   * XOR swizzles: dY chunk ^ ((row>>1 ^ row>>3) & 3), W chunk ^ 2*(row & 3),
//     so fragment reads hit every bank once;
//   * four 32 KiB LDS stages, loads three k tiles ahead; each wave's four
//     load instructions of a tile are spread between its MFMAs; one barrier
//     per k tile (explicit vmcnt waits: the only vector-memory ops in the loop
//     are these loads);
//   * per-tap dY gather offsets (position -> byte offset, or out of range for
//     taps off dY's edge and ragged tiles) and per-position dX offsets are
//     built once per workgroup into small LDS tables;
//   * epilogue: accumulators -> bf16 (nearest-even, v_cvt_pk_bf16_f32) -> LDS
//     ([position][c], chunk ^ (row & 31)) -> 16-byte coalesced stores along
//     each dX pixel row.
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
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int BM = kFastBM, BN = kFastBN, BK = kFastBK;  // 256, 256, 32
constexpr int THREADS = kFastThreads;                    // 512
constexpr int NSTAGE = 4;
constexpr int AROW = BM * 2;                             // 512 B: one k row of the W tile
constexpr int BROW = BK * 2;                             // 64 B: one position row of the dY tile
constexpr int ABYTES = BK * AROW;                        // 16 KiB
constexpr int STAGE = ABYTES + BN * BROW;                // 32 KiB
constexpr int MAX_TAPS = kFastMaxTaps;                   // gather-table capacity (taps per class)
constexpr int DMA_PER_TILE = 4;                          // per wave: 2 W + 2 dY instructions
static_assert(THREADS / 64 * DMA_PER_TILE * 1024 == STAGE, "one stage = all waves' loads of a tile");
static_assert(THREADS >= BN, "one thread per position row builds the tables");

// s_waitcnt immediate: vmcnt <= n, other counters unconstrained (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ inline int swz_w(int row) { return 2 * (row & 3); }                  // 32 chunks/row
__device__ inline int swz_y(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }  // 4 chunks/row

__global__ __launch_bounds__(THREADS, 1) void igemm_nhwc_bf16_kernel(const GemmArgs a) {
  // Stages as distinct objects: the compiler can then see that fragment reads
  // of one stage do not alias the loads in flight into another.
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage2[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage3[STAGE];
  __shared__ uint32_t gtab[MAX_TAPS * BN];  // dY byte offset of (tap, position row), channel g*Kg
  __shared__ uint32_t otab[BN];             // dX byte offset of position row, channel g*Cg + m0
  auto stage_ptr = [&](int st) -> char* {
    return st == 0 ? stage0 : st == 1 ? stage1 : st == 2 ? stage2 : stage3;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // wm: 128-channel half, wn: 64-position quarter

  const int t = dev::logical_tile(blockIdx.x, a.total_tiles, a.xcd_remap);
  const SubDesc s = a.sub[dev::find_class(a, t)];
  const int npix_img = s.pos_h * s.pos_w;
  const int npos = a.N * npix_img;
  const int tiles_n = (npos + BN - 1) / BN;
  const int per_group = a.tiles_m * tiles_n;
  const int local = t - s.tile_begin;
  const int g = local / per_group;
  const int rem = local - g * per_group;
  const int m0 = (rem % a.tiles_m) * BM;
  const int n0 = (rem / a.tiles_m) * BN;
  const int ntaps = s.taps_h * s.taps_w;

  const auto rdy = dev::rsrc(a.dy, a.dy_bytes);
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);

  // ---- per-workgroup tables (threads 0..255: one position row each)
  if (tid < BN) {
    const int p = n0 + tid;
    const bool pv = p < npos;
    const int pp = pv ? p : 0;
    const int n = pp / npix_img;
    const int rr = pp - n * npix_img;
    const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
    for (int tap = 0; tap < ntaps; tap++) {
      const int jh = tap / s.taps_w, jw = tap - (tap / s.taps_w) * s.taps_w;
      const int ho = th + s.beta_h - a.delta_h * jh, wo = tw + s.beta_w - a.delta_w * jw;
      const bool ok = pv && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
      gtab[tap * BN + tid] = ok ? (uint32_t)(((n * a.Ho + ho) * a.Wo + wo) * a.K + g * a.Kg) * 2u : dev::kOOB;
    }
    const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
    otab[tid] = pv ? (uint32_t)(((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg + m0) * 2u : dev::kOOB;
  }
  __syncthreads();

  const int YX = a.Y * a.X;
  const uint32_t wrow = (uint32_t)(YX * a.Cg) * 2u;  // bytes between consecutive k rows of W
  const int kpt = a.Kg / BK;
  const int KT = ntaps * kpt;

  // ---- load roles.  W: instruction i (0, 1) of wave w fills k rows
  // 4w + 2i + (lane >> 5), 16-byte slot lane & 31 holding channel chunk
  // (lane & 31) ^ swz_w(row).  dY: instruction i fills position rows
  // 16*(2w + i) + (lane >> 2), slot lane & 3 holding k chunk (lane & 3) ^ swz_y(row).
  uint32_t a_lane[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int row = 4 * wave + 2 * i + (lane >> 5);
    const int c = m0 + 8 * ((lane & 31) ^ swz_w(row));
    a_lane[i] = c < a.Cg ? (uint32_t)row * wrow + (uint32_t)c * 2u : dev::kOOB;
  }
  int b_row[2];
  uint32_t b_chunk[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    b_row[i] = 16 * (2 * wave + i) + (lane >> 2);
    b_chunk[i] = (uint32_t)(((lane & 3) ^ swz_y(b_row[i])) * 16);
  }

  uint32_t dma_off[DMA_PER_TILE];
  lds_char* dma_st = (lds_char*)stage0;
  int cur_tap = -1;
  uint32_t a_tap = 0, b_tap[2] = {0, 0};  // per-tap bases, refreshed when the tap changes
  auto prepare_dma = [&](int kt) {
    const int tap = kt / kpt;
    const int k0 = (kt - tap * kpt) * BK;
    if (tap != cur_tap) {  // uniform branch, taken once per tap
      cur_tap = tap;
      const int jh = tap / s.taps_w, jw = tap - (tap / s.taps_w) * s.taps_w;
      const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
      a_tap = (uint32_t)(((g * a.Kg) * YX + ty * a.X + tx) * a.Cg) * 2u;
#pragma unroll
      for (int i = 0; i < 2; i++) b_tap[i] = gtab[tap * BN + b_row[i]] + b_chunk[i];
    }
    dma_st = (lds_char*)stage_ptr(kt % NSTAGE);
    // Whole offsets go in the per-lane operand, so the record-count check
    // sees every byte a lane touches.
#pragma unroll
    for (int i = 0; i < 2; i++) dma_off[i] = a_lane[i] + a_tap + (uint32_t)k0 * wrow;
#pragma unroll
    for (int i = 0; i < 2; i++) dma_off[2 + i] = b_tap[i] + (uint32_t)k0 * 2u;
  };
  auto issue_one = [&](int j) {
    if (j < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dma_st + (2 * wave + j) * 1024), 16,
                                               dma_off[j], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rdy, (lds_void*)(dma_st + ABYTES + (2 * wave + j - 2) * 1024),
                                               16, dma_off[j], 0, 0, 0);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
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
  // B: lane reads chunk 2*ks + (lane >> 5) of position row wn*64 + 32*bn + (lane & 31).
  int b_rd[2][2];
#pragma unroll
  for (int bn = 0; bn < 2; bn++) {
    const int row = wn * 64 + bn * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
      b_rd[bn][ks] = ABYTES + row * BROW + (((2 * ks + (lane >> 5)) ^ swz_y(row)) << 4);
  }

  // One k tile: 2 k steps x (4 A fragments, 2 B fragments, 8 MFMAs); the
  // wave's 4 load instructions for a future tile go after MFMA pairs.
  auto compute = [&](auto stc, bool dma) {
    constexpr int ST = decltype(stc)::value;
    lds_char* st = (lds_char*)(ST == 0 ? stage0 : ST == 1 ? stage1 : ST == 2 ? stage2 : stage3);
    const char* sb = ST == 0 ? stage0 : ST == 1 ? stage1 : ST == 2 ? stage2 : stage3;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int bm = 0; bm < 4; bm++) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(st + a_rd[bm][ks][0]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(st + a_rd[bm][ks][1]));
        fa[bm] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int bn = 0; bn < 2; bn++) fb[bn] = *(const bf16x8*)(sb + b_rd[bn][ks]);
#pragma unroll
      for (int bm = 0; bm < 4; bm++) {
#pragma unroll
        for (int bn = 0; bn < 2; bn++)
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[bm], fb[bn], acc[bm][bn], 0, 0, 0);
        if (dma && (bm & 1)) issue_one(2 * ks + (bm >> 1));
      }
    }
  };

  // ---- main loop: tiles kt+1, kt+2 in flight while tile kt computes.
#pragma unroll
  for (int s0 = 0; s0 < NSTAGE - 1; s0++)
    if (s0 < KT) {
      prepare_dma(s0);
#pragma unroll
      for (int j = 0; j < DMA_PER_TILE; j++) issue_one(j);
    }
  auto step = [&](int kt, auto stc) {
    // This wave's loads of tile kt have landed once at most `later` newer
    // tiles' loads are outstanding; the barrier extends that to every wave
    // and guarantees nobody still reads tile kt-1's stage.
    const int later = (KT - 1 - kt) < (NSTAGE - 2) ? (KT - 1 - kt) : (NSTAGE - 2);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * DMA_PER_TILE));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_PER_TILE));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    const bool dma = kt + NSTAGE - 1 < KT;
    if (dma) prepare_dma(kt + NSTAGE - 1);  // into the stage of tile kt-1
    compute(stc, dma);
  };
  for (int kt = 0; kt < KT; kt += NSTAGE) {
    step(kt, std::integral_constant<int, 0>());
    if (kt + 1 < KT) step(kt + 1, std::integral_constant<int, 1>());
    if (kt + 2 < KT) step(kt + 2, std::integral_constant<int, 2>());
    if (kt + 3 < KT) step(kt + 3, std::integral_constant<int, 3>());
  }

  // ---- epilogue.  C tile [position row][256 channels] bf16 = 128 KiB over
  // the four stages (64 rows each), 16-byte chunk c/8 of row r stored at
  // chunk (c/8) ^ (r & 31).
  __syncthreads();
#pragma unroll
  for (int bn = 0; bn < 2; bn++) {
    const int prow = wn * 64 + bn * 32 + (lane & 31);
    char* rowp = stage_ptr(prow >> 6) + (prow & 63) * 512;
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
  {
    const int ch = tid & 31;
    const bool cv = m0 + 8 * ch < a.Cg;
#pragma unroll 4
    for (int it = 0; it < BN / (THREADS / 32); it++) {
      const int prow = it * (THREADS / 32) + (tid >> 5);
      const char* rowp = stage_ptr(prow >> 6) + (prow & 63) * 512;
      const u32x4 v = *(const u32x4*)(rowp + ((ch ^ (prow & 31)) << 4));
      const uint32_t base = otab[prow];
      __builtin_amdgcn_raw_buffer_store_b128(u4{v[0], v[1], v[2], v[3]}, rdx,
                                             cv ? base + (uint32_t)ch * 16u : dev::kOOB, 0, 0);
    }
  }
}

}  // namespace

int launch_nhwc_bf16(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&igemm_nhwc_bf16_kernel, dim3((unsigned)grid),
                              dim3(THREADS), args, 0, (hipStream_t)stream);
}

}  // namespace cbd
