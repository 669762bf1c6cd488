// Device helpers shared by the DART kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dart {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;  // MFMA operand
typedef float f32x16_t __attribute__((ext_vector_type(16)));                   // 32x32 MFMA acc
typedef float f32x4_t __attribute__((ext_vector_type(4)));                     // 16x16 MFMA acc

// log2(e): the kernels run the softmax in base 2 (exp2/log2 are the native
// transcendental instructions), so logits are pre-multiplied by log2(e).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest even: the native conversion
// (v_cvt_pk_bf16_f32 on gfx950 converts two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Native base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float ld(const float* p, int64_t i) { return p[i]; }
  __device__ static void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static float ld(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static void st(bf16_t* p, int64_t i, float v) { p[i] = (bf16_t)f32_to_bf16(v); }
};
// float16 storage (the score memory of bfloat16 inputs): round to nearest even
template <> struct Elem<_Float16> {
  __device__ static float ld(const _Float16* p, int64_t i) { return (float)p[i]; }
  __device__ static void st(_Float16* p, int64_t i, float v) { p[i] = (_Float16)v; }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace dart
