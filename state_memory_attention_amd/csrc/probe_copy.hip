// Measurement helper, not part of the DART path: a plain device copy of a
// known number of bytes (16-byte vector loads and stores, grid-stride), used
// to calibrate the hardware memory-traffic counters against kernels that
// access memory the same way.  Built as its own library, libdart_probe.so.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {
__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}
}  // namespace

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`.
// Returns 0, or -1 on bad arguments, or -5 if the launch failed.
extern "C" int dart_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || (bytes & 15) || (((uintptr_t)src | (uintptr_t)dst) & 15)) return -1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  copy16_kernel<<<dim3(4096), dim3(256), 0, (hipStream_t)stream>>>((const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
