// RMS-normalised score branch, general kernels (any N, P <= 256; float32 or
// bfloat16 inputs).
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §3 text after Eq. 10
// and App. B.1 Eq. 25-27.  The logit of token t and chunk c becomes
//     l = RMSNorm(Q_t) . (r_c * (dH_c RMSNorm(E_t))) / sqrt(N),
//     r_c[n] = (mean_p dH_c[n][p]^2 + eps)^(-1/2)                  (Eq. 26)
// with RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w (optional per-channel
// weight w); the values V = C_t dH_c, the softmax and the residual are those
// of the plain branch.
//
// Everything that depends only on the chunk is applied once per chunk: the
// chunk-state side produces r_c and the score memory
//     dHs_c[p][n] = w_e[p] dH_c[p][n] r_c[n] w_q[n]
// (float16 for bfloat16 inputs, float32 otherwise), so the forward pass
// contracts the score memory exactly like the plain branch contracts dH_c
// and applies the per-token factors 1/rms(Q_t) and 1/rms(E_t) to the logit.
// Decode reads r_c from the cache and scales q by r_c w_q per chunk instead
// (a cache of r costs N floats per chunk, a cached score memory N P).
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kThreads = 256;

// r_c and the score memory of one chunk memory: block per (b, h, chunk),
// thread per key index n (N <= 256); both are computed from dH as stored.
template <typename T, typename TS>
__global__ __launch_bounds__(kThreads) void chunk_rms_kernel(
    int64_t n_mem, int N, int P, float eps, const T* __restrict__ dH, const float* __restrict__ wq,
    const float* __restrict__ we, float* __restrict__ r, TS* __restrict__ dHs) {
  const int64_t c = blockIdx.x;
  const int n = threadIdx.x;
  if (c >= n_mem || n >= N) return;
  const T* mem = dH + c * (int64_t)P * N;
  float ss = 0.f;
  for (int p = 0; p < P; ++p) {
    const float x = Elem<T>::ld(mem, (int64_t)p * N + n);
    ss = fmaf(x, x, ss);
  }
  const float rn = 1.f / sqrtf(ss / (float)P + eps);  // [Eq. 26]
  if (r) r[c * N + n] = rn;
  if (dHs) {
    const float rq = rn * (wq ? wq[n] : 1.f);
    TS* out = dHs + c * (int64_t)P * N;
    for (int p = 0; p < P; ++p) {
      const float x = Elem<T>::ld(mem, (int64_t)p * N + n) * rq;
      Elem<TS>::st(out, (int64_t)p * N + n, we ? x * we[p] : x);
    }
  }
}

// One token against `n_hist` chunk memories, one wave, with the normalised
// score branch.  Lane owns p = lane + 64 k.  Exactly one of `smem` (score
// memories, forward) and `rmem` (r_c per chunk, decode; then wq and we are
// the RMSNorm weights) supplies the scaling along n.
template <typename T, typename TS>
__device__ void token_sma_rms_wave(const T* __restrict__ q, const T* __restrict__ c,
                                   const T* __restrict__ e, const T* __restrict__ mem,
                                   const TS* __restrict__ smem, const float* __restrict__ rmem,
                                   const float* __restrict__ wq, const float* __restrict__ we,
                                   int64_t n_hist, int N, int P, float eps, float* sq, float* sc,
                                   float r[4], float& lse) {
  const int lane = threadIdx.x & 63;
  // RMSNorm of the query and of the key readout vector [Eq. 25]
  float ssq = 0.f, sse = 0.f;
  for (int i = lane; i < N; i += 64) {
    const float x = Elem<T>::ld(q, i);
    ssq = fmaf(x, x, ssq);
  }
  for (int i = lane; i < P; i += 64) {
    const float x = Elem<T>::ld(e, i);
    sse = fmaf(x, x, sse);
  }
  const float inv_q = 1.f / sqrtf(wave_sum(ssq) / (float)N + eps);
  const float inv_e = 1.f / sqrtf(wave_sum(sse) / (float)P + eps);
  for (int i = lane; i < N; i += 64) {
    const float x = Elem<T>::ld(q, i) * inv_q;
    sq[i] = wq ? x * wq[i] : x;
    sc[i] = Elem<T>::ld(c, i);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float scale = kLog2e / sqrtf((float)N) * inv_e;
  float ev[4], o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    float x = p < P ? Elem<T>::ld(e, p) * scale : 0.f;
    if (we && p < P) x *= we[p];
    ev[k] = x;
    o[k] = 0.f;
  }
  float m = -INFINITY, d = 0.f;
  for (int64_t j = 0; j < n_hist; ++j) {
    const T* dj = mem + j * (int64_t)P * N;
    const TS* sj = smem ? smem + j * (int64_t)P * N : nullptr;
    const float* rj = rmem ? rmem + j * (int64_t)N : nullptr;
    float v[4], part = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = lane + 64 * k;
      float ws = 0.f, vs = 0.f;
      if (p < P) {
        const T* row = dj + (int64_t)p * N;
        if (sj) {
          const TS* srow = sj + (int64_t)p * N;
          for (int i = 0; i < N; ++i) {
            ws = fmaf(sq[i], Elem<TS>::ld(srow, i), ws);
            vs = fmaf(sc[i], Elem<T>::ld(row, i), vs);
          }
        } else {
          for (int i = 0; i < N; ++i) {
            const float x = Elem<T>::ld(row, i);
            ws = fmaf(sq[i] * rj[i], x, ws);
            vs = fmaf(sc[i], x, vs);
          }
        }
      }
      v[k] = vs;
      part = fmaf(ws, ev[k], part);
    }
    const float l2 = wave_sum(part);
    const float mn = fmaxf(m, l2);
    const float alpha = fast_exp2(m - mn);  // m = -inf on the first chunk -> 0
    const float pj = fast_exp2(l2 - mn);
    d = fmaf(alpha, d, pj);
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = fmaf(alpha, o[k], pj * v[k]);
    m = mn;
  }
  const float inv = d > 0.f ? 1.f / d : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = o[k] * inv;
  lse = d > 0.f ? (m + fast_log2(d)) * kLn2 : -INFINITY;
}

// Gated residual epilogue for one token-head row [§3 Eq. 11].
template <typename T>
__device__ void write_row_rms(const T* __restrict__ Y, const T* __restrict__ gate, int gate_pc,
                              T* __restrict__ out, float* __restrict__ Rout, int64_t row, int P,
                              const float r[4]) {
  const int lane = threadIdx.x & 63;
  const float gs = gate_pc ? 0.f : Elem<T>::ld(gate, row);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    if (p < P) {
      const int64_t i = row * P + p;
      const float g = gate_pc ? Elem<T>::ld(gate, i) : gs;
      Elem<T>::st(out, i, fmaf(g, r[k], Elem<T>::ld(Y, i)));
      if (Rout) Rout[i] = r[k];
    }
  }
}

// Forward, one wave per token, 4 tokens per block.
template <typename T, typename TS>
__global__ __launch_bounds__(kThreads) void sma_fwd_rms_general_kernel(
    Shape s, float eps, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const T* __restrict__ dH, const TS* __restrict__ dHs, const T* __restrict__ Y,
    const T* __restrict__ gate, int gate_pc, T* __restrict__ out, float* __restrict__ R,
    float* __restrict__ lse, int64_t groups_per_head) {
  __shared__ float s_q[4][256];
  __shared__ float s_c[4][256];
  const int wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.x / groups_per_head;
  const int64_t t = (blockIdx.x % groups_per_head) * 4 + wave;
  if (t >= s.L) return;  // no block-level barrier below
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tok = b * s.L + t;
  const int64_t n_hist = t / s.S;
  const int64_t base = bh * s.M * (int64_t)P * N;
  float r[4], l;
  token_sma_rms_wave<T, TS>(Q + (tok * s.G + g) * N, C + (tok * s.G + g) * N,
                            E + (tok * s.G + g) * P, dH + base, dHs + base, nullptr, nullptr,
                            nullptr, n_hist, N, P, eps, s_q[wave], s_c[wave], r, l);
  write_row_rms<T>(Y, gate, gate_pc, out, R, tok * s.H + h, P, r);
  if (lse && (threadIdx.x & 63) == 0) lse[bh * s.L + t] = l;
}

// Decode, one wave per (b, h), 4 per block.
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_decode_rms_general_kernel(
    Shape s, int64_t max_chunks, float eps, const T* __restrict__ q, const T* __restrict__ c,
    const T* __restrict__ e, const T* __restrict__ cache, const float* __restrict__ r_cache,
    const int32_t* __restrict__ n_chunks, const float* __restrict__ wq,
    const float* __restrict__ we, const T* __restrict__ y, const T* __restrict__ gate, int gate_pc,
    T* __restrict__ out, float* __restrict__ R, float* __restrict__ lse) {
  __shared__ float s_q[4][256];
  __shared__ float s_c[4][256];
  const int wave = threadIdx.x >> 6;
  const int64_t bh = (int64_t)blockIdx.x * 4 + wave;
  if (bh >= s.b * s.H) return;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  int64_t nb = n_chunks ? (int64_t)n_chunks[b] : max_chunks;
  nb = nb < 0 ? 0 : (nb > max_chunks ? max_chunks : nb);
  float r[4], l;
  token_sma_rms_wave<T, float>(q + (b * s.G + g) * N, c + (b * s.G + g) * N, e + (b * s.G + g) * P,
                               cache + bh * max_chunks * (int64_t)P * N, nullptr,
                               r_cache + bh * max_chunks * (int64_t)N, wq, we, nb, N, P, eps,
                               s_q[wave], s_c[wave], r, l);
  write_row_rms<T>(y, gate, gate_pc, out, R, bh, P, r);
  if (lse && (threadIdx.x & 63) == 0) lse[bh] = l;
}

}  // namespace

hipError_t launch_chunk_rms(const Shape& s, bool bf16, float eps, const void* dH, const float* wq,
                            const float* we, float* r, void* dHs, hipStream_t st) {
  const int64_t n_mem = s.b * s.H * s.M;
  if (n_mem == 0) return hipSuccess;
  if (bf16)
    chunk_rms_kernel<bf16_t, _Float16><<<dim3((unsigned)n_mem), dim3(kThreads), 0, st>>>(
        n_mem, (int)s.N, (int)s.P, eps, (const bf16_t*)dH, wq, we, r, (_Float16*)dHs);
  else
    chunk_rms_kernel<float, float><<<dim3((unsigned)n_mem), dim3(kThreads), 0, st>>>(
        n_mem, (int)s.N, (int)s.P, eps, (const float*)dH, wq, we, r, (float*)dHs);
  return hipGetLastError();
}

hipError_t launch_sma_fwd_rms_general(const Shape& s, bool bf16, float eps, const void* Q,
                                      const void* C, const void* E, const void* dH, const void* dHs,
                                      const void* Y, const void* gate, int gate_pc, void* out,
                                      float* R, float* lse, hipStream_t st) {
  const int64_t gph = (s.L + 3) / 4;
  const int64_t blocks = s.b * s.H * gph;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    sma_fwd_rms_general_kernel<bf16_t, _Float16><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, eps, (const bf16_t*)Q, (const bf16_t*)C, (const bf16_t*)E, (const bf16_t*)dH,
        (const _Float16*)dHs, (const bf16_t*)Y, (const bf16_t*)gate, gate_pc, (bf16_t*)out, R, lse,
        gph);
  else
    sma_fwd_rms_general_kernel<float, float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, eps, (const float*)Q, (const float*)C, (const float*)E, (const float*)dH,
        (const float*)dHs, (const float*)Y, (const float*)gate, gate_pc, (float*)out, R, lse, gph);
  return hipGetLastError();
}

hipError_t launch_sma_decode_rms_general(const Shape& s, bool bf16, int64_t max_chunks, float eps,
                                         const void* q, const void* c, const void* e,
                                         const void* cache, const float* r_cache,
                                         const int32_t* n_chunks, const float* wq, const float* we,
                                         const void* y, const void* gate, int gate_pc, void* out,
                                         float* R, float* lse, hipStream_t st) {
  const int64_t blocks = (s.b * s.H + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    sma_decode_rms_general_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, max_chunks, eps, (const bf16_t*)q, (const bf16_t*)c, (const bf16_t*)e,
        (const bf16_t*)cache, r_cache, n_chunks, wq, we, (const bf16_t*)y, (const bf16_t*)gate,
        gate_pc, (bf16_t*)out, R, lse);
  else
    sma_decode_rms_general_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, max_chunks, eps, (const float*)q, (const float*)c, (const float*)e, (const float*)cache,
        r_cache, n_chunks, wq, we, (const float*)y, (const float*)gate, gate_pc, (float*)out, R,
        lse);
  return hipGetLastError();
}

}  // namespace dart
