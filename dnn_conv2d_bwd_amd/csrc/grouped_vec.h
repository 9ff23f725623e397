// grouped_vec.h -- small helpers shared by the grouped kernels: one group's
// channels at one pixel as a vector of 2, 4, 8 or a multiple of 16 bytes
// (LDS read up to 16 bytes, buffer load, buffer store).
#pragma once
#include "cbd_device.h"

namespace cbd {
namespace grp {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int BYTES>
struct Vec {
  static constexpr int W = BYTES >= 4 ? BYTES / 4 : 1;
  uint32_t w[W];
};

// p is aligned to BYTES (a group's channels start at a multiple of their
// size inside a 16-byte-aligned pixel row), so 8 and 16 bytes are single
// ds_read_b64 / ds_read_b128.
template <int BYTES>
__device__ inline Vec<BYTES> lds_vec(const char* p) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  Vec<BYTES> v;
  if constexpr (BYTES == 2) {
    v.w[0] = *(const uint16_t*)p;
  } else if constexpr (BYTES == 4) {
    v.w[0] = *(const uint32_t*)p;
  } else if constexpr (BYTES == 8) {
    const u2 x = *(const u2*)p;
    v.w[0] = x[0];
    v.w[1] = x[1];
  } else {
    const u4 x = *(const u4*)p;
#pragma unroll
    for (int i = 0; i < 4; i++) v.w[i] = x[i];
  }
  return v;
}

template <int BYTES>
__device__ inline Vec<BYTES> load_vec(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Vec<BYTES> v;
  if constexpr (BYTES == 2) {
    v.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (BYTES == 4) {
    v.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (BYTES == 8) {
    auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    v.w[0] = x[0];
    v.w[1] = x[1];
  } else {
    static_assert(BYTES % 16 == 0, "2, 4, 8 or a multiple of 16 bytes");
#pragma unroll
    for (int h = 0; h < BYTES / 16; h++) {
      auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; j++) v.w[4 * h + j] = x[j];
    }
  }
  return v;
}

template <int BYTES>
__device__ inline void store_vec(__amdgpu_buffer_rsrc_t r, uint32_t off, const Vec<BYTES>& v) {
  if constexpr (BYTES == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v.w[0], r, off, 0, 0);
  } else if constexpr (BYTES == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(v.w[0], r, off, 0, 0);
  } else if constexpr (BYTES == 8) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    u2 x = {v.w[0], v.w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, 0);
  } else {
    static_assert(BYTES % 16 == 0, "2, 4, 8 or a multiple of 16 bytes");
#pragma unroll
    for (int h = 0; h < BYTES / 16; h++) {
      u4 x = {v.w[4 * h], v.w[4 * h + 1], v.w[4 * h + 2], v.w[4 * h + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(x, r, off + 16 * h, 0, 0);
    }
  }
}

}  // namespace grp
}  // namespace cbd
