// General DART kernels: any state size N <= 256, head dim P <= 256, any chunk
// size S, float32 or bfloat16 storage, float32 arithmetic.  They cover every
// shape the MFMA kernels do not, and serve as a second GPU implementation to
// cross-check them.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032).
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kThreads = 256;
constexpr int kSub = 8;  // tokens staged per step in the chunk-state kernel

// ---------------------------------------------------------------------------
// Chunk state memories [§3 Eq. 5]: dH_[c] = sum_s w_s B_s^T X_s with
// w_s = prod_{k=s+1}^{e(c)} a_k.  One block per (b, h, chunk, 256-entry tile
// of the N x P output); each thread owns one output entry (p, n).
// The chunk is walked from its end in 256-token segments; a block-wide
// suffix product gives w inside a segment and `carry` holds the product of
// the decays of all later segments.
template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_states_general_kernel(
    Shape s, const T* __restrict__ X, const T* __restrict__ B, const float* __restrict__ A,
    T* __restrict__ dH, int out_tiles) {
  __shared__ float s_scan[kThreads];
  __shared__ float s_w[kThreads];
  __shared__ float s_x[kSub][256];
  __shared__ float s_b[kSub][256];

  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int tile = (int)(blk % out_tiles);
  const int64_t rest = blk / out_tiles;
  const int64_t c = rest % s.M;
  const int64_t bh = rest / s.M;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int idx = tile * kThreads + tid;
  const bool active = idx < N * P;
  const int p = active ? idx / N : 0;
  const int n = active ? idx % N : 0;

  const int64_t s0 = c * s.S;
  const int64_t s1 = (s0 + s.S < s.L) ? s0 + s.S : s.L;

  float acc = 0.f;
  float carry = 1.f;  // prod of a_k over tokens after the current segment
  for (int64_t seg_end = s1; seg_end > s0; seg_end -= kThreads) {
    const int64_t seg_start = (seg_end - kThreads > s0) ? seg_end - kThreads : s0;
    const int cnt = (int)(seg_end - seg_start);
    s_scan[tid] = tid < cnt ? A[(b * s.L + seg_start + tid) * s.H + h] : 1.f;
    __syncthreads();
    // inclusive suffix product: s_scan[k] = prod_{j >= k} a_j (padding is 1)
    for (int off = 1; off < kThreads; off <<= 1) {
      const float v = s_scan[tid] * (tid + off < kThreads ? s_scan[tid + off] : 1.f);
      __syncthreads();
      s_scan[tid] = v;
      __syncthreads();
    }
    s_w[tid] = carry * (tid + 1 < kThreads ? s_scan[tid + 1] : 1.f);
    const float seg_prod = s_scan[0];
    __syncthreads();
    carry *= seg_prod;

    for (int k0 = 0; k0 < cnt; k0 += kSub) {
      for (int e = tid; e < kSub * P; e += kThreads) {
        const int kk = e / P, pp = e % P;
        float v = 0.f;
        if (k0 + kk < cnt)
          v = Elem<T>::ld(X, ((b * s.L + seg_start + k0 + kk) * s.H + h) * P + pp) * s_w[k0 + kk];
        s_x[kk][pp] = v;
      }
      for (int e = tid; e < kSub * N; e += kThreads) {
        const int kk = e / N, nn = e % N;
        float v = 0.f;
        if (k0 + kk < cnt) v = Elem<T>::ld(B, ((b * s.L + seg_start + k0 + kk) * s.G + g) * N + nn);
        s_b[kk][nn] = v;
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int kk = 0; kk < kSub; ++kk) acc = fmaf(s_b[kk][n], s_x[kk][p], acc);
      }
      __syncthreads();
    }
  }
  if (active) Elem<T>::st(dH, ((bh * s.M + c) * P + p) * (int64_t)N + n, acc);
}

// ---------------------------------------------------------------------------
// One token against `n_hist` chunk memories, one wave [§3 Eq. 8-10; App. C
// Eq. 29-31].  Lane owns p = lane + 64k.  q and c are staged in the wave's
// LDS slice.  The softmax runs in base 2 (logit * log2 e).
// Returns R in r[] (lane's p values) and the natural-log lse.
template <typename T>
__device__ void token_sma_wave(const T* __restrict__ q, const T* __restrict__ c,
                               const T* __restrict__ e, const T* __restrict__ mem, int64_t n_hist,
                               int N, int P, float* sq, float* sc, float r[4], float& lse) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < N; i += 64) {
    sq[i] = Elem<T>::ld(q, i);
    sc[i] = Elem<T>::ld(c, i);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float scale = kLog2e / sqrtf((float)N);
  float ev[4], o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    ev[k] = p < P ? Elem<T>::ld(e, p) * scale : 0.f;
    o[k] = 0.f;
  }
  float m = -INFINITY, d = 0.f;
  for (int64_t j = 0; j < n_hist; ++j) {
    const T* dj = mem + j * (int64_t)P * N;
    float w[4], v[4], part = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = lane + 64 * k;
      float ws = 0.f, vs = 0.f;
      if (p < P) {
        const T* row = dj + (int64_t)p * N;
        for (int i = 0; i < N; ++i) {
          const float x = Elem<T>::ld(row, i);
          ws = fmaf(sq[i], x, ws);
          vs = fmaf(sc[i], x, vs);
        }
      }
      w[k] = ws;
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
__device__ void write_row(const T* __restrict__ Y, const T* __restrict__ gate, int gate_pc,
                          T* __restrict__ out, float* __restrict__ Rout, int64_t row, int64_t grow,
                          int P, const float r[4]) {
  const int lane = threadIdx.x & 63;
  const float gs = gate_pc ? 0.f : Elem<T>::ld(gate, grow);
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

// SMA forward, one wave per token, 4 tokens per block.
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_fwd_general_kernel(
    Shape s, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const T* __restrict__ dH, const T* __restrict__ Y, const T* __restrict__ gate, int gate_pc,
    T* __restrict__ out, float* __restrict__ R, float* __restrict__ lse, int64_t groups_per_head) {
  __shared__ float s_q[4][256];
  __shared__ float s_c[4][256];
  const int wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.x / groups_per_head;
  const int64_t t = (blockIdx.x % groups_per_head) * 4 + wave;
  if (t >= s.L) return;  // no block-level barrier below
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tok = b * s.L + t;
  const int64_t n_hist = t / s.S;  // chunks 0 .. chunk(t)-1 are visible
  float r[4], l;
  token_sma_wave<T>(Q + (tok * s.G + g) * N, C + (tok * s.G + g) * N, E + (tok * s.G + g) * P,
                    dH + bh * s.M * (int64_t)P * N, n_hist, N, P, s_q[wave], s_c[wave], r, l);
  write_row<T>(Y, gate, gate_pc, out, R, tok * s.H + h, tok * s.H + h, P, r);
  if (lse && (threadIdx.x & 63) == 0) lse[bh * s.L + t] = l;
}

// Decode, one wave per (b, h), 4 per block.
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_decode_general_kernel(
    Shape s, int64_t max_chunks, const T* __restrict__ q, const T* __restrict__ c,
    const T* __restrict__ e, const T* __restrict__ cache, const int32_t* __restrict__ n_chunks,
    const T* __restrict__ y, const T* __restrict__ gate, int gate_pc, T* __restrict__ out,
    float* __restrict__ R, float* __restrict__ lse) {
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
  token_sma_wave<T>(q + (b * s.G + g) * N, c + (b * s.G + g) * N, e + (b * s.G + g) * P,
                    cache + bh * max_chunks * (int64_t)P * N, nb, N, P, s_q[wave], s_c[wave], r, l);
  write_row<T>(y, gate, gate_pc, out, R, bh, bh, P, r);
  if (lse && (threadIdx.x & 63) == 0) lse[bh] = l;
}

}  // namespace

hipError_t launch_chunk_states_general(const Shape& s, bool bf16, const void* X, const void* B,
                                       const float* A, void* dH, hipStream_t st) {
  const int out_tiles = (int)((s.N * s.P + kThreads - 1) / kThreads);
  const int64_t blocks = s.b * s.H * s.M * out_tiles;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    chunk_states_general_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)X, (const bf16_t*)B, A, (bf16_t*)dH, out_tiles);
  else
    chunk_states_general_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, (const float*)X, (const float*)B, A, (float*)dH, out_tiles);
  return hipGetLastError();
}

hipError_t launch_sma_fwd_general(const Shape& s, bool bf16, const void* Q, const void* C,
                                  const void* E, const void* dH, const void* Y, const void* gate,
                                  int gate_pc, void* out, float* R, float* lse, hipStream_t st) {
  const int64_t gph = (s.L + 3) / 4;
  const int64_t blocks = s.b * s.H * gph;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    sma_fwd_general_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)Q, (const bf16_t*)C, (const bf16_t*)E, (const bf16_t*)dH,
        (const bf16_t*)Y, (const bf16_t*)gate, gate_pc, (bf16_t*)out, R, lse, gph);
  else
    sma_fwd_general_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, (const float*)Q, (const float*)C, (const float*)E, (const float*)dH, (const float*)Y,
        (const float*)gate, gate_pc, (float*)out, R, lse, gph);
  return hipGetLastError();
}

hipError_t launch_sma_decode_general(const Shape& s, bool bf16, int64_t max_chunks, const void* q,
                                     const void* c, const void* e, const void* cache,
                                     const int32_t* n_chunks, const void* y, const void* gate,
                                     int gate_pc, void* out, float* R, float* lse, hipStream_t st) {
  const int64_t blocks = (s.b * s.H + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (bf16)
    sma_decode_general_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, max_chunks, (const bf16_t*)q, (const bf16_t*)c, (const bf16_t*)e,
        (const bf16_t*)cache, n_chunks, (const bf16_t*)y, (const bf16_t*)gate, gate_pc,
        (bf16_t*)out, R, lse);
  else
    sma_decode_general_kernel<float><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        s, max_chunks, (const float*)q, (const float*)c, (const float*)e, (const float*)cache,
        n_chunks, (const float*)y, (const float*)gate, gate_pc, (float*)out, R, lse);
  return hipGetLastError();
}

}  // namespace dart
