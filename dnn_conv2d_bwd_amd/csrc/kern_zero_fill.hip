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
// multiple of 16) or one 16-byte chunk of an NHWC pixel row; a thread takes
// kZeroItemsPerThread items, kZeroThreads apart (each store instruction of a
// wave covers 64 consecutive items).
#include "cbd_device.h"
#include "cbd_internal.h"

namespace cbd {
namespace {

__global__ __launch_bounds__(kZeroThreads) void zero_fill_kernel(const ZeroArgs z) {
  const auto rdx = dev::rsrc(z.dx, z.dx_bytes);
  const uint32_t base = (uint32_t)blockIdx.x * (kZeroThreads * kZeroItemsPerThread) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kZeroItemsPerThread; i++) {
    const uint32_t item = base + (uint32_t)(i * kZeroThreads);
    if ((int64_t)item < z.total_items)
      dev::zero_item(rdx, z.layout, z.esize, z.chunk, z.C, z.Hi, z.Wi, z.Sh, z.Sw, z.reg,
                     z.num_regions, item);
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
