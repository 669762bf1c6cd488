// Decode-side cache maintenance: the in-progress chunk memory of every
// (batch row, head) absorbs one new token, and a chunk that the token closes
// is appended to the chunk-memory cache (with its inverse RMS along the value
// axis when the normalised score branch is in use, App. B.1 Eq. 26).
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032).  The cache holds one
// memory per complete chunk [§4 "Inference Cache"]; the memory of chunk c is
// the chunk's zero-initial-state contribution dH_[c] [§3 Eq. 5; App. A
// Eq. 20], which is the step recurrence of §2 Eq. 2 restarted from zero at
// the chunk's first token:
//     state <- a_t state + B_t^T X_t,
// so after the chunk's last token the state equals dH_[c].
//
// Memory bound: the float32 state (N x P per head) is read and written once
// per token, the dtype cache row is written only when a chunk closes.  One
// block per (b, h), the token's B and x rows staged in LDS; every thread owns
// 8 consecutive entries (one 32-byte vector) of rows p of the [P][N] state
// at a time, and issues the loads of four such steps together.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_update_kernel(
    int64_t H, int64_t G, int N, int P, int64_t S, int64_t max_chunks, const T* __restrict__ x,
    const T* __restrict__ B, const float* __restrict__ a, float* __restrict__ state,
    const int32_t* __restrict__ pos, T* __restrict__ cache, int32_t* __restrict__ n_chunks,
    float* __restrict__ r_cache, float eps) {
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H, h = bh % H, g = h / (H / G);
  const int64_t t = pos[b];
  if (t < 0) return;  // padding row: untouched
  const int64_t c = t / S;
  const bool closes = (t % S) == S - 1;
  if (h == 0 && threadIdx.x == 0 && n_chunks) {
    const int64_t done = (t + 1) / S;
    n_chunks[b] = (int32_t)(done < max_chunks ? done : max_chunks);
  }
  const float at = a[bh];
  float* st = state + bh * (int64_t)P * N;
  T* dst = (closes && c < max_chunks) ? cache + (bh * max_chunks + c) * (int64_t)P * N : nullptr;
  const int total = P * N;  // N, P <= 256
  // the token's B row and x row, as float32, shared by the whole block
  __shared__ __attribute__((aligned(16))) float s_b[256];
  __shared__ float s_x[256];
  const T* br = B + (b * G + g) * N;
  const T* xr = x + bh * P;
  for (int i = threadIdx.x; i < N; i += kThreads) s_b[i] = Elem<T>::ld(br, i);
  for (int i = threadIdx.x; i < P; i += kThreads) s_x[i] = Elem<T>::ld(xr, i);
  __syncthreads();
  if ((N & 7) == 0) {
    // 8 entries of one row per step (state as 2 float4, cache as 8
    // elements); the state loads of kSteps steps are issued together
    constexpr int kSteps = 4;
    for (int i0 = threadIdx.x * 8; i0 < total; i0 += kThreads * 8 * kSteps) {
      float4 sv[kSteps][2];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int i = i0 + u * kThreads * 8;
        if (i < total) {
          sv[u][0] = *(const float4*)(st + i);
          sv[u][1] = *(const float4*)(st + i + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int i = i0 + u * kThreads * 8;
        if (i >= total) break;
        const int p = i / N, n = i - p * N;
        const float xp = s_x[p];
        const float4 b0 = *(const float4*)(s_b + n), b1 = *(const float4*)(s_b + n + 4);
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        float v[8] = {sv[u][0].x, sv[u][0].y, sv[u][0].z, sv[u][0].w,
                      sv[u][1].x, sv[u][1].y, sv[u][1].z, sv[u][1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = fmaf(at, v[k], bv[k] * xp);
        if (closes) {
          if (dst)
#pragma unroll
            for (int k = 0; k < 8; ++k) Elem<T>::st(dst, i + k, v[k]);
          *(float4*)(st + i) = make_float4(0.f, 0.f, 0.f, 0.f);
          *(float4*)(st + i + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
          *(float4*)(st + i) = make_float4(v[0], v[1], v[2], v[3]);
          *(float4*)(st + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < total; i += kThreads) {
      const int p = i / N, n = i - p * N;
      const float v = fmaf(at, st[i], s_b[n] * s_x[p]);
      if (closes) {
        if (dst) Elem<T>::st(dst, i, v);
        st[i] = 0.f;
      } else {
        st[i] = v;
      }
    }
  }
  // Inverse RMS of the memory just closed, along the value axis, from the
  // values as cached [App. B.1 Eq. 26]: read back after the block's stores.
  if (r_cache && dst) {
    __syncthreads();
    for (int n = threadIdx.x; n < N; n += kThreads) {
      float ss = 0.f;
      for (int p = 0; p < P; ++p) {
        const float v = Elem<T>::ld(dst, (int64_t)p * N + n);
        ss = fmaf(v, v, ss);
      }
      r_cache[(bh * max_chunks + c) * N + n] = 1.f / sqrtf(ss / (float)P + eps);
    }
  }
}

}  // namespace

hipError_t launch_decode_update(const Shape& s, bool bf16, int64_t max_chunks, const void* x,
                                const void* B, const float* a, float* state, const int32_t* pos,
                                void* cache, int32_t* n_chunks, float* r_cache, float eps,
                                hipStream_t st) {
  const int64_t blocks = s.b * s.H;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    decode_update_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s.H, s.G, (int)s.N, (int)s.P, s.S, max_chunks, (const bf16_t*)x, (const bf16_t*)B, a, state,
        pos, (bf16_t*)cache, n_chunks, r_cache, eps);
  else
    decode_update_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s.H, s.G, (int)s.N, (int)s.P, s.S, max_chunks, (const float*)x, (const float*)B, a, state, pos,
        (float*)cache, n_chunks, r_cache, eps);
  return hipGetLastError();
}

}  // namespace dart
