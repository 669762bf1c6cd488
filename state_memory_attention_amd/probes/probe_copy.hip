// Measurement helpers, not part of the DART path, built as their own library
// (libdart_probe.so):
//   * a plain device copy of a known number of bytes (16-byte vector loads and
//     stores, grid-stride), used to calibrate the hardware memory-traffic
//     counters against kernels that access memory the same way;
//   * a streaming read (16-byte non-temporal vector loads, eight in flight
//     per lane, 8192 blocks, grid-stride: the fastest of a sweep over 4-16
//     loads in flight, 2048-65536 blocks, plain or non-temporal), the
//     yardstick for what a read-only kernel can draw from HBM on this device;
//   * a plain matrix-core loop (v_mfma_f32_32x32x16_bf16 on operands held in
//     registers, two waves per SIMD, the forward's burst shape), the yardstick
//     for what dense bf16 work sustains on this device at the clock it holds
//     under that load with the given operand values.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 probe_bf16x8_t;
typedef float probe_f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int probe_u32x4_t __attribute__((ext_vector_type(4)));

namespace {
__global__ __launch_bounds__(256) void copy16_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}
// The loaded words are folded into one value per lane, written only if it
// equals an impossible pattern, so that the loads are not optimised away.
__global__ __launch_bounds__(256) void read16_kernel(const probe_u32x4_t* __restrict__ src, size_t n16,
                                                     unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    probe_u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i).x;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}
// Each wave: 16 operand registers (8 A, 8 B) read once from `ops`, then
// `iters` bursts of 32 MFMAs (8 k-steps x 4 accumulators, two A and two B
// operands per k-step, as in the forward's per-chunk burst).  The
// accumulators are folded and written only if the fold equals an impossible
// value, so that the work is not optimised away.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_kernel(const uint4* __restrict__ ops, int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  probe_bf16x8_t a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = __builtin_bit_cast(probe_bf16x8_t, ops[64 * k + lane]);
    b[k] = __builtin_bit_cast(probe_bf16x8_t, ops[512 + 64 * k + lane]);
  }
  probe_f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const probe_bf16x8_t a0 = a[ks], a1 = a[(ks + 1) & 7];
      w0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[ks], w0, 0, 0, 0);
      w1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[ks], w1, 0, 0, 0);
      v0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[(ks + 3) & 7], v0, 0, 0, 0);
      v1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[(ks + 3) & 7], v1, 0, 0, 0);
    }
  }
  float f = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) f += w0[r] + w1[r] + v0[r] + v1[r];
  if (f == 1234.5f) sink[blockIdx.x * blockDim.x + threadIdx.x] = f;
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

// Reads `bytes` (a multiple of 16; `src` 16-byte aligned) on `stream`;
// `sink` (4 bytes, device) is written only in the impossible case above.
// Returns 0, or -1 on bad arguments, or -5 if the launch failed.
extern "C" int dart_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || (bytes & 15) || ((uintptr_t)src & 15)) return -1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  read16_kernel<<<dim3(8192), dim3(256), 0, (hipStream_t)stream>>>((const probe_u32x4_t*)src, n16,
                                                                  (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Runs `blocks` blocks of 4 waves, each wave `iters` bursts of 32
// v_mfma_f32_32x32x16_bf16 (32768 flop each) on operands from `ops` (16 KB,
// 16-byte aligned: 512 pieces of A then 512 of B).  `sink` holds one float
// per thread and is written only in the impossible case above.  Returns 0,
// or -1 on bad arguments, or -5 if the launch failed.
extern "C" int dart_probe_mfma(const void* ops, int blocks, int iters, void* sink, void* stream) {
  if (!ops || !sink || blocks <= 0 || iters < 0 || ((uintptr_t)ops & 15)) return -1;
  mfma_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((const uint4*)ops, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
