// kern_igemm_generic.hip -- implicit-GEMM backward-data for any layout and
// dtype (the fallback family).  One launch covers every stride-residue class:
// each workgroup decodes (class, group, M-tile, N-tile) from its id.
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
// Tiles 64(M) x 64(N) x 16(K), 256 threads = 4 waves in 2x2, each wave
// 32x32 via v_mfma_f32_16x16x4_f32.  Operands are gathered element-wise with
// buffer loads (out-of-range -> 0: padding, ragged tiles, taps off dY's
// edge), converted to f32 and staged in LDS.  bf16 products are exact in
// f32, so this matches a bf16 MFMA's arithmetic up to summation order.
#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

template <int DT>
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  if constexpr (DT == 0) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
  } else {
    return dev::bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0));
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

template <int DT, int LAYOUT>
__global__ __launch_bounds__(kGenericThreads) void igemm_generic_kernel(const GemmArgs a) {
  constexpr int BM = kGenericBM, BN = kGenericBN, BK = kGenericBK;
  constexpr uint32_t ES = DT == 0 ? 4 : 2;
  constexpr int NPIX = LAYOUT == 0 ? 1 : 4;  // dY positions each thread gathers
  __shared__ float As[BK][BM];
  __shared__ float Bs[BK][BN];

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
  const int HoWo = a.Ho * a.Wo;

  // A (filter) gather: column m = tid & 63, rows kk = (tid >> 6) + 4*i.
  const int am = tid & 63;
  const int ac = m0 + am;
  const bool ac_ok = ac < a.Cg;
  // B (dY) gather: NCHW walks positions across lanes (w is contiguous),
  // NHWC walks k across lanes (channels are contiguous).
  int pn[NPIX], pth[NPIX], ptw[NPIX];
  bool pok[NPIX];
#pragma unroll
  for (int j = 0; j < NPIX; j++) {
    const int p = n0 + (LAYOUT == 0 ? (tid & 63) : (tid >> 4) + 16 * j);
    pok[j] = p < npos;
    const int pp = pok[j] ? p : 0;
    pn[j] = pp / npix_img;
    const int rr = pp - pn[j] * npix_img;
    pth[j] = rr / s.pos_w;
    ptw[j] = rr - pth[j] * s.pos_w;
  }

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int jh = 0; jh < s.taps_h; jh++) {
    for (int jw = 0; jw < s.taps_w; jw++) {
      const int ty = s.cls_h + a.tstep_h * jh, tx = s.cls_w + a.tstep_w * jw;
      const int dho = s.beta_h - a.delta_h * jh, dwo = s.beta_w - a.delta_w * jw;
      // dY element offset of channel g*Kg (k added per element), or -1.
      int boff[NPIX];
#pragma unroll
      for (int j = 0; j < NPIX; j++) {
        const int ho = pth[j] + dho, wo = ptw[j] + dwo;
        const bool ok = pok[j] && ho >= 0 && ho < a.Ho && wo >= 0 && wo < a.Wo;
        const int o = LAYOUT == 0 ? ((pn[j] * a.K + g * a.Kg) * a.Ho + ho) * a.Wo + wo
                                  : ((pn[j] * a.Ho + ho) * a.Wo + wo) * a.K + g * a.Kg;
        boff[j] = ok ? o : -1;
      }
      for (int k0 = 0; k0 < a.Kg; k0 += BK) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int k = k0 + (tid >> 6) + 4 * i;
          const int o = LAYOUT == 0 ? ((g * a.Kg + k) * a.Cg + ac) * YX + ty * a.X + tx
                                    : ((g * a.Kg + k) * YX + ty * a.X + tx) * a.Cg + ac;
          av[i] = load_elem<DT>(rw, (ac_ok && k < a.Kg) ? (uint32_t)o * ES : dev::kOOB);
        }
        if constexpr (LAYOUT == 0) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int k = k0 + (tid >> 6) + 4 * i;
            const bool ok = boff[0] >= 0 && k < a.Kg;
            bv[i] = load_elem<DT>(rdy, ok ? (uint32_t)(boff[0] + k * HoWo) * ES : dev::kOOB);
          }
        } else {
          const int k = k0 + (tid & 15);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const bool ok = boff[j] >= 0 && k < a.Kg;
            bv[j] = load_elem<DT>(rdy, ok ? (uint32_t)(boff[j] + k) * ES : dev::kOOB);
          }
        }
        __syncthreads();  // previous tile's MFMAs are done with LDS
#pragma unroll
        for (int i = 0; i < 4; i++) As[(tid >> 6) + 4 * i][am] = av[i];
        if constexpr (LAYOUT == 0) {
#pragma unroll
          for (int i = 0; i < 4; i++) Bs[(tid >> 6) + 4 * i][tid & 63] = bv[i];
        } else {
#pragma unroll
          for (int j = 0; j < 4; j++) Bs[tid & 15][(tid >> 4) + 16 * j] = bv[j];
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 4; ks++) {
          const int kr = 4 * ks + (lane >> 4);
#pragma unroll
          for (int bm = 0; bm < 2; bm++) {
            const float x = As[kr][wm * 32 + bm * 16 + (lane & 15)];
#pragma unroll
            for (int bn = 0; bn < 2; bn++) {
              const float y = Bs[kr][wn * 32 + bn * 16 + (lane & 15)];
              acc[bm][bn] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc[bm][bn], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // Epilogue: lane holds rows 4*(lane>>4)+v, column lane&15 of each 16x16 block.
#pragma unroll
  for (int bn = 0; bn < 2; bn++) {
    const int p = n0 + wn * 32 + bn * 16 + (lane & 15);
    const bool pv = p < npos;
    const int pp = pv ? p : 0;
    const int n = pp / npix_img;
    const int rr = pp - n * npix_img;
    const int th = rr / s.pos_w, tw = rr - (rr / s.pos_w) * s.pos_w;
    const int hi = s.phase_h + a.Sh * th, wi = s.phase_w + a.Sw * tw;
    const int pbase = LAYOUT == 0 ? (n * a.C + g * a.Cg) * a.Hi * a.Wi + hi * a.Wi + wi
                                  : ((n * a.Hi + hi) * a.Wi + wi) * a.C + g * a.Cg;
    const int cstride = LAYOUT == 0 ? a.Hi * a.Wi : 1;
#pragma unroll
    for (int bm = 0; bm < 2; bm++) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int c = m0 + wm * 32 + bm * 16 + 4 * (lane >> 4) + v;
        const bool ok = pv && c < a.Cg;
        store_elem<DT>(rdx, ok ? (uint32_t)(pbase + c * cstride) * ES : dev::kOOB,
                       acc[bm][bn][v]);
      }
    }
  }
}

template <int DT, int LAYOUT>
int launch_one(const GemmArgs& a, int64_t grid, void* stream) {
  void* args[] = {const_cast<GemmArgs*>(&a)};
  return (int)hipLaunchKernel((const void*)&igemm_generic_kernel<DT, LAYOUT>,
                              dim3((unsigned)grid), dim3(kGenericThreads), args, 0,
                              (hipStream_t)stream);
}

}  // namespace

int launch_generic(const GemmArgs& a, int layout, int dtype, int64_t grid, void* stream) {
  if (dtype == CBD_F32)
    return layout == CBD_LAYOUT_NCHW ? launch_one<0, 0>(a, grid, stream)
                                     : launch_one<0, 1>(a, grid, stream);
  return layout == CBD_LAYOUT_NCHW ? launch_one<1, 0>(a, grid, stream)
                                   : launch_one<1, 1>(a, grid, stream);
}

}  // namespace cbd
