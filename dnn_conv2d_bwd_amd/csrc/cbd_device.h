// cbd_device.h -- small gfx950 device helpers shared by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cbd_kernarg.h"

namespace cbd {
namespace dev {

// Buffer resource over one tensor.  Record count = tensor bytes, so a load
// at an offset past the end returns zeros and a store there is dropped:
// predication costs one out-of-range offset instead of a branch.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data format for the gfx9 family.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // > every record count (tensors < 2 GiB)

// f32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two f32 -> packed bf16 (lo in bits 0-15), round to nearest even; gfx950
// does this in one instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16_pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Logical tile of hardware workgroup b.  Workgroups are dealt round-robin to
// the 8 XCDs (each with its own L2); with remap on, XCD x receives the
// contiguous logical range [x*q + min(x, r), ...), so neighbouring tiles --
// which share operand panels -- meet in one L2.
__device__ inline int logical_tile(int b, int total, int remap) {
  const int q = total >> 3, r = total & 7, x = b & 7, idx = b >> 3;
  return remap ? x * q + (x < r ? x : r) + idx : b;
}

// Logical block of hardware workgroup b for the grouped row kernels:
// workgroups go round-robin to the 8 XCDs, and XCD x gets logical blocks
// 64r + 8x .. 64r + 8x + 7, so neighbouring row blocks of one image (which
// share dY rows) meet in one L2.  Blocks past the last multiple of 64 map to
// themselves.
__device__ inline int chunked_block(int b, int total) {
  const int full = total & ~63;
  if (b >= full) return b;
  const int r = b >> 6, i = b & 63;
  return (r << 6) + ((i & 7) << 3) + (i >> 3);
}

// dY index read by tap j of class position t along one axis.  Residue split:
// t + beta - delta*j.  Zero-insertion form (no_split): t is the dX index
// itself and the term exists only where t + pad - j*dil is a non-negative
// multiple of the stride; otherwise -1 (out of range: the load reads 0).
__device__ inline int dy_index(int no_split, int t, int beta, int delta, int j, int pad, int dil,
                               int str) {
  if (!no_split) return t + beta - delta * j;
  const int num = t + pad - j * dil;
  return (num >= 0 && num % str == 0) ? num / str : -1;
}

// x / d for 32-bit x, with mag = ceil(2^32 / d) (0 for d = 1): the
// multiply-high estimate is the quotient or one more, and one compare fixes it.
__device__ inline uint32_t fdiv(uint32_t x, uint32_t d, uint32_t mag) {
  const uint32_t q = __umulhi(x, mag);
  return d == 1u ? x : (q * d > x ? q - 1u : q);
}

// Zero-fill work item `item` (regions reg[0..nreg), item_begin ascending):
// one element (NCHW, or NHWC rows not a multiple of 16 bytes) or one
// 16-byte chunk of an NHWC pixel row of an unreached dX phase lattice.
// Item counts stay below 2^32 and dX below 2^31 bytes (the planner's
// limits), so the arithmetic is 32-bit.
__device__ inline void zero_item(__amdgpu_buffer_rsrc_t rdx, int layout, int esize, int chunk, int C,
                                 int Hi, int Wi, int Sh, int Sw, const ZeroDesc* reg, int nreg,
                                 uint32_t item) {
  int r = 0;
  for (int i = 1; i < nreg; i++)
    if ((uint32_t)reg[i].item_begin <= item) r = i;
  const ZeroDesc& d = reg[r];
  uint32_t li = item - (uint32_t)d.item_begin;
  uint32_t off;
  uint32_t cidx = 0;
  if (layout == 1) {
    const uint32_t pos = fdiv(li, d.per_pos, d.mag_pp);
    cidx = li - pos * d.per_pos;
    li = pos;
  }
  const uint32_t q = fdiv(li, (uint32_t)d.pos_w, d.mag_w);
  const uint32_t b = li - q * (uint32_t)d.pos_w;
  const uint32_t nc = fdiv(q, (uint32_t)d.pos_h, d.mag_h);  // n (NHWC) or n*C + c (NCHW)
  const uint32_t a = q - nc * (uint32_t)d.pos_h;
  const uint32_t hi = (uint32_t)d.phase_h + (uint32_t)Sh * a, wi = (uint32_t)d.phase_w + (uint32_t)Sw * b;
  if (layout == 1)
    off = (((nc * (uint32_t)Hi + hi) * (uint32_t)Wi + wi) * (uint32_t)C) * (uint32_t)esize + cidx * (uint32_t)chunk;
  else
    off = ((nc * (uint32_t)Hi + hi) * (uint32_t)Wi + wi) * (uint32_t)esize;
  if (chunk == 16) {
    typedef uint32_t u4z __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(u4z{0u, 0u, 0u, 0u}, rdx, off, 0, 0);
  } else if (chunk == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(0u, rdx, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rdx, off, 0, 0);
  }
}

// Touch every 64-byte line of the kernel arguments that a GEMM workgroup
// reads (the header lines, the class table and the first two class
// descriptors) in one batch at entry.  The first access to each line misses
// the scalar cache; fetched at their first uses, which depend on one
// another (tile -> class -> descriptor), the misses would be paid one round
// trip at a time.
__device__ inline void prefetch_args(const GemmArgs& a) {
  const int h0 = a.N, h1 = a.num_sub, h2 = a.class_begin[1], h3 = a.class_begin[15];
  const int h4 = a.sub[0].phase_h, h5 = a.sub[1].tile_begin;
  const void* p0 = a.dy;
  const void* p1 = a.dx;
  asm volatile("" ::"s"(h0), "s"(h1), "s"(h2), "s"(h3), "s"(h4), "s"(h5), "s"(p0), "s"(p1));
}

// Class owning logical tile t (class_begin ascends with the class index):
// the number of classes after the first that begin at or before t.  The
// first 16 entries are read unconditionally (one batch of scalar loads).
__device__ inline int find_class(const GemmArgs& a, int t) {
  const int ns = a.num_sub;
  int r = 0;
#pragma unroll
  for (int i = 1; i < 16; i++) r += (i < ns && a.class_begin[i] <= t) ? 1 : 0;
  for (int i = 16; i < ns; i++) r += a.class_begin[i] <= t ? 1 : 0;
  return r;
}

}  // namespace dev
}  // namespace cbd
