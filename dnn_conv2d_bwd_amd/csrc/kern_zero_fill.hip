// kern_zero_fill.hip -- writes +0 to the dX phase lattices that no filter tap
// reaches.  Along one axis a dX position hi is reached only if
// hi + pad - tap*dil is a non-negative multiple of the stride for some tap;
// with gcd(stride, dil) > 1, or with fewer taps than stride classes, whole
// phases hi = phase + S*a are never reached (1x1 filters at stride 2 leave
// three of four phases).  The zero-inserted dY of fusilli issue #101's BOO
// listing shows the same holes as explicit zeros; here they are never
// materialised, only the dX lattice is cleared.
//
// One work item = one element (NCHW, or NHWC rows whose byte size is not a
// multiple of 16) or one 16-byte chunk of an NHWC pixel row.
#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

__global__ __launch_bounds__(kZeroThreads) void zero_fill_kernel(const ZeroArgs z) {
  const int64_t item = (int64_t)blockIdx.x * kZeroThreads + threadIdx.x;
  if (item >= z.total_items) return;
  int r = 0;
  for (int i = 1; i < z.num_regions; i++)
    if (z.reg[i].item_begin <= item) r = i;
  const ZeroDesc d = z.reg[r];
  int64_t li = item - d.item_begin;
  const auto rdx = dev::rsrc(z.dx, z.dx_bytes);
  uint32_t off;
  if (z.layout == 1) {
    const int64_t per_pos = (int64_t)z.C * z.esize / z.chunk;
    const int64_t cidx = li % per_pos;
    int64_t pos = li / per_pos;
    const int64_t b = pos % d.pos_w;
    pos /= d.pos_w;
    const int64_t a = pos % d.pos_h;
    const int64_t n = pos / d.pos_h;
    const int64_t hi = d.phase_h + (int64_t)z.Sh * a, wi = d.phase_w + (int64_t)z.Sw * b;
    off = (uint32_t)((((n * z.Hi + hi) * z.Wi + wi) * z.C) * z.esize + cidx * z.chunk);
  } else {
    const int64_t b = li % d.pos_w;
    li /= d.pos_w;
    const int64_t a = li % d.pos_h;
    const int64_t nc = li / d.pos_h;
    const int64_t hi = d.phase_h + (int64_t)z.Sh * a, wi = d.phase_w + (int64_t)z.Sw * b;
    off = (uint32_t)(((nc * z.Hi + hi) * z.Wi + wi) * z.esize);
  }
  if (z.chunk == 16) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(u4{0u, 0u, 0u, 0u}, rdx, off, 0, 0);
  } else if (z.chunk == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(0u, rdx, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rdx, off, 0, 0);
  }
}

}  // namespace

int launch_zero_fill(const ZeroArgs& z, int64_t grid, void* stream) {
  void* args[] = {const_cast<ZeroArgs*>(&z)};
  return (int)hipLaunchKernel((const void*)&zero_fill_kernel, dim3((unsigned)grid),
                              dim3(kZeroThreads), args, 0, (hipStream_t)stream);
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace cbd
