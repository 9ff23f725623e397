// kern_igemm_nhwc_bf16.hip -- the large-problem family: NHWC dX / NHWK dY /
// KYXC W in bf16, f32 accumulation, bf16 result (the dtype contract of the
// BOO listing in fusilli issue #101: extf to f32, mulf/addf, truncf).
//
// Same per-residue-class GEMM as the generic family (see
// kern_igemm_generic.hip), specialised for C/G % 8 == 0 and K/G % 64 == 0:
//   * 256(M = c) x 256(N = positions) x 64(K = k) tiles, 256 threads = 4
//     waves in 2x2, each wave 128x128 = 4x4 blocks of
//     v_mfma_f32_32x32x16_bf16 (256 f32 accumulators per lane);
//   * dY rows are k-contiguous: 16-byte buffer loads go to LDS as they are
//     (row = position, 128-byte row of 64 k);
//   * W rows are c-contiguous: each thread loads an 8(k) x 8(c) block with
//     eight 16-byte loads and transposes it in registers, so LDS holds
//     row = c, 64 k contiguous -- the k-vector each MFMA lane consumes;
//   * LDS rows of 8 16-byte chunks are XOR-swizzled (chunk ^ ((row ^
//     row>>3) & 7)) so both the transposed writes and the MFMA fragment
//     reads spread over all banks;
//   * two LDS stages (2 x 64 KiB) and register fragments one k step ahead:
//     global loads run two k tiles ahead of the MFMAs, LDS writes one;
//   * taps off dY's edge and ragged M/N tiles read zeros through buffer
//     record bounds; stores outside dX's class lattice are dropped the same
//     way; the f32 -> bf16 rounding (nearest-even) is fused in the epilogue.
#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int BM = kFastBM, BN = kFastBN, BK = kFastBK;
constexpr int ROWB = BK * 2;            // bytes per LDS row (64 bf16)
constexpr int ABYTES = BM * ROWB;       // 32 KiB
constexpr int BBYTES = BN * ROWB;       // 32 KiB
constexpr int STAGE = ABYTES + BBYTES;  // 64 KiB

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

__global__ __launch_bounds__(kFastThreads, 1) void igemm_nhwc_bf16_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

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

  const auto rdy = dev::rsrc(a.dy, a.dy_bytes);
  const auto rw = dev::rsrc(a.w, a.w_bytes);
  const auto rdx = dev::rsrc(a.dx, a.dx_bytes);

  const int YX = a.Y * a.X;
  // W block of this thread: c chunk cq (8 channels), k rows 8*kr .. 8*kr+7.
  const int cq = tid & 31, kr = tid >> 5;
  const int a_c = m0 + 8 * cq;
  const bool a_ok = a_c < a.Cg;
  const uint32_t a_row = (uint32_t)(YX * a.Cg) * 2u;  // bytes between k rows
  // dY chunk of this thread: k chunk q (8 channels) of positions pr + 32*i.
  const int q = tid & 7, pr = tid >> 3;

  // LDS addresses (bytes) this thread writes.
  uint32_t a_st[8], b_st[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int row = 8 * cq + e;
    a_st[e] = row * ROWB + ((kr ^ swz(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int row = pr + 32 * i;
    b_st[i] = ABYTES + row * ROWB + ((q ^ swz(row)) << 4);
  }

  const int kpt = a.Kg / BK;  // k tiles per tap
  const int KT = s.taps_h * s.taps_w * kpt;

  int cur_tap = -1;
  uint32_t a_off0 = 0;
  uint32_t b_off[8];
  u32x4 ra[8], rb[8];

  auto issue_loads = [&](int kt) {
    const int tap = kt / kpt;
    const int k0 = (kt - tap * kpt) * BK;
    if (tap != cur_tap) {
      cur_tap = tap;
      const int jh = tap / s.taps_w, jw = tap - (tap / s.taps_w) * s.taps_w;
      const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
      const int dho = s.beta_h - a.delta_h * jh, dwo = s.beta_w - a.delta_w * jw;
      a_off0 = a_ok ? (uint32_t)((((g * a.Kg + 8 * kr) * YX + ty * a.X + tx) * a.Cg + a_c)) * 2u
                    : dev::kOOB;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int p = n0 + pr + 32 * i;
        const bool pv = p < npos;
        const int pp = pv ? p : 0;
        const int n = pp / npix_img;
        const int rr = pp - n * npix_img;
        const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
        const int ho = th + dho, wo = tw + dwo;
        const bool ok = pv && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
        b_off[i] = ok ? (uint32_t)(((n * a.Ho + ho) * a.Wo + wo) * a.K + g * a.Kg + 8 * q) * 2u
                      : dev::kOOB;
      }
    }
    const uint32_t ao = a_off0 + (uint32_t)k0 * a_row;
#pragma unroll
    for (int i = 0; i < 8; i++)
      ra[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, ao + i * a_row, 0, 0));
#pragma unroll
    for (int i = 0; i < 8; i++)
      rb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdy, b_off[i] + (uint32_t)k0 * 2u, 0, 0));
  };

  auto store_stage = [&](int stage) {
    char* base = smem + stage * STAGE;
    // W: ra[i] = 8 channels of k row i; LDS row c = 8*cq+e takes k 0..7 of column e.
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int w = e >> 1;
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t lo = ra[2 * j][w], hi = ra[2 * j + 1][w];
        o[j] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *(u32x4*)(base + a_st[e]) = o;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) *(u32x4*)(base + b_st[i]) = rb[i];
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

  // Fragment rows (A: channel, B: position) of this lane; the 16-byte chunk
  // for k step ks is 2*ks + (lane >> 5), XOR-ed with the row swizzle.
  int a_row_of[4], b_row_of[4];
#pragma unroll
  for (int b = 0; b < 4; b++) {
    a_row_of[b] = wm * 128 + b * 32 + (lane & 31);
    b_row_of[b] = wn * 128 + b * 32 + (lane & 31);
  }
  bf16x8 fa[2][4], fb[2][4];
  auto load_frags = [&](int buf, const char* base, int ks) {
    const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int ra_ = a_row_of[b], rb_ = b_row_of[b];
      fa[buf][b] = *(const bf16x8*)(base + ra_ * ROWB + ((chunk ^ swz(ra_)) << 4));
      fb[buf][b] = *(const bf16x8*)(base + ABYTES + rb_ * ROWB + ((chunk ^ swz(rb_)) << 4));
    }
  };
  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int bm = 0; bm < 4; bm++)
#pragma unroll
      for (int bn = 0; bn < 4; bn++)
        acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][bm], fb[buf][bn],
                                                              acc[bm][bn], 0, 0, 0);
  };

  // Software pipeline.  During k tile kt: LDS stage kt&1 feeds the MFMAs
  // (fragments double-buffered in registers, one k step ahead); tile kt+1,
  // loaded into registers during tile kt-1, is written to the other stage
  // halfway through; then the global loads of tile kt+2 are issued.
  issue_loads(0);
  store_stage(0);
  if (KT > 1) issue_loads(1);
  __syncthreads();
  load_frags(0, smem, 0);

  for (int kt = 0; kt < KT; kt++) {
    const int cur = kt & 1;
    const char* base = smem + cur * STAGE;
    load_frags(1, base, 1);
    mfma_step(0);
    load_frags(0, base, 2);
    mfma_step(1);
    if (kt + 1 < KT) store_stage(cur ^ 1);
    if (kt + 2 < KT) issue_loads(kt + 2);
    load_frags(1, base, 3);
    mfma_step(0);
    mfma_step(1);
    __syncthreads();
    if (kt + 1 < KT) load_frags(0, smem + (cur ^ 1) * STAGE, 0);
  }

  // Epilogue.  Lane holds, per 32x32 block, rows 8*(v>>2) + 4*(lane>>5) + (v&3)
  // (four consecutive channels per v>>2) of column lane&31 (one position).
#pragma unroll
  for (int bn = 0; bn < 4; bn++) {
    const int p = n0 + wn * 128 + bn * 32 + (lane & 31);
    const bool pv = p < npos;
    const int pp = pv ? p : 0;
    const int n = pp / npix_img;
    const int rr = pp - n * npix_img;
    const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
    const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
    const int pbase = ((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg;
#pragma unroll
    for (int bm = 0; bm < 4; bm++) {
#pragma unroll
      for (int qq = 0; qq < 4; qq++) {
        const int c = m0 + wm * 128 + bm * 32 + 8 * qq + 4 * (lane >> 5);
        const bool ok = pv && c < a.Cg;
        u32x2 o;
        o[0] = dev::bf16_rne(acc[bm][bn][4 * qq + 0]) | (dev::bf16_rne(acc[bm][bn][4 * qq + 1]) << 16);
        o[1] = dev::bf16_rne(acc[bm][bn][4 * qq + 2]) | (dev::bf16_rne(acc[bm][bn][4 * qq + 3]) << 16);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), rdx,
                                              ok ? (uint32_t)(pbase + c) * 2u : dev::kOOB, 0, 0);
      }
    }
  }
}

}  // namespace

int launch_nhwc_bf16(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&igemm_nhwc_bf16_kernel, dim3((unsigned)grid),
                              dim3(kFastThreads), args, 0, (hipStream_t)stream);
}

}  // namespace cbd
