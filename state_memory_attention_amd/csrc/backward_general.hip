// Backward pass, general kernels (any N, P <= 256; float32 or bfloat16 inputs,
// float32 arithmetic and float32 gradients).
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032).  The forward keeps only
// R and lse; the backward recomputes every logit and recovers the chunk
// weights as p = exp(l - lse) [§4 "Efficient Training"; App. C "Recomputation",
// Eq. 33-35], then applies the chain rule through §3 Eq. 8-11 and Eq. 5:
//
//   dR_t = g_t * dout_t,  D_t = dR_t . R_t,  V_tc = C_t dH_c,  W_tc = Q_t dH_c,
//   l_tc = W_tc . E_t / sqrt(N),  p_tc = exp(l_tc - lse_t),
//   dl_tc = p_tc (dR_t . V_tc - D_t),
//   dQ_t = sum_c dl_tc dH_c E_t / sqrt(N),   dE_t = sum_c dl_tc W_tc / sqrt(N),
//   dC_t = sum_c p_tc dH_c dR_t,
//   d_dH_c = sum_{t: chunk(t) > c} p_tc C_t^T dR_t + dl_tc Q_t^T E_t / sqrt(N),
//   dX_s = w_s B_s d_dH_c,  dB_s = w_s d_dH_c X_s^T,  dw_s = B_s d_dH_c X_s^T,
//   dA_k = w_k u_k,  u_{s0} = 0,  u_{k+1} = a_k u_k + dw_k   (within a chunk),
// the last line being sum_{s<k} dw_s dw_s/da_k written as a forward recurrence
// (no division by a_k, which may be 0).
//
// Kernels: (1) one wave per (token, head) recomputes the token's logits chunk
// by chunk, accumulates dQ, dC, dE and stores (p, dl) per (chunk, token) in
// the workspace; (2) one block per (chunk, head, 256 entries of d_dH) sums the
// rank-1 terms over the later tokens; (3) chunk-state backward, one block per
// (chunk, head); (4) the decay recurrence, one thread per (chunk, head);
// (5) sums over the heads of a projection group.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kThreads = 256;

// dR = g * dout for p = lane + 64 k.
template <typename T>
__device__ void load_dr(const T* dout, const T* gate, int gate_pc, int64_t row, int64_t grow, int P,
                        float dr[4]) {
  const int lane = threadIdx.x & 63;
  const float gs = gate_pc ? 0.f : Elem<T>::ld(gate, grow);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    dr[k] = 0.f;
    if (p < P) dr[k] = (gate_pc ? Elem<T>::ld(gate, row * P + p) : gs) * Elem<T>::ld(dout, row * P + p);
  }
}

// (1) Token kernel: one wave per (token, head), 4 per block.  Lanes own
// p = lane + 64k for the P-side sums (W, V, dE) and n = lane + 64k for the
// N-side sums (dQ, dC).
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_bwd_token_kernel(
    Shape s, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const T* __restrict__ dH, const T* __restrict__ gate, int gate_pc, const float* __restrict__ R,
    const float* __restrict__ lse, const T* __restrict__ dout, float* __restrict__ dq_out,
    float* __restrict__ dc_out, float* __restrict__ de_out, int64_t head_stride_out,
    float* __restrict__ dgate, float* __restrict__ pd, int64_t groups_per_head) {
  __shared__ float s_q[4][256], s_c[4][256], s_e[4][256], s_r[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / groups_per_head;
  const int64_t t = (blockIdx.x % groups_per_head) * 4 + wave;
  if (t >= s.L) return;  // no block-level barrier below
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tok = b * s.L + t;
  const int64_t row = tok * s.H + h;  // [b][L][H] row
  const int64_t n_hist = t / s.S;
  const float scale = 1.f / sqrtf((float)N);

  float* sq = s_q[wave];
  float* sc = s_c[wave];
  float* se = s_e[wave];
  float* sr = s_r[wave];  // dR
  for (int i = lane; i < N; i += 64) {
    sq[i] = Elem<T>::ld(Q + (tok * s.G + g) * N, i);
    sc[i] = Elem<T>::ld(C + (tok * s.G + g) * N, i);
  }
  float dr[4], rr[4], part = 0.f;
  load_dr<T>(dout, gate, gate_pc, row, row, P, dr);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    rr[k] = p < P ? R[row * P + p] : 0.f;
    if (p < P) {
      se[p] = Elem<T>::ld(E + (tok * s.G + g) * P, p);
      sr[p] = dr[k];
    }
    part = fmaf(dr[k], rr[k], part);
  }
  const float D = wave_sum(part);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float lse_t = lse[bh * s.L + t];
  float dq[4] = {0.f, 0.f, 0.f, 0.f}, dc[4] = {0.f, 0.f, 0.f, 0.f}, de[4] = {0.f, 0.f, 0.f, 0.f};
  const T* mem = dH + bh * s.M * (int64_t)P * N;
  for (int64_t j = 0; j < n_hist; ++j) {
    const T* dj = mem + j * (int64_t)P * N;
    float w[4], lp = 0.f, vp = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = lane + 64 * k;
      float ws = 0.f, vs = 0.f;
      if (p < P) {
        const T* rowp = dj + (int64_t)p * N;
        for (int i = 0; i < N; ++i) {
          const float x = Elem<T>::ld(rowp, i);
          ws = fmaf(sq[i], x, ws);
          vs = fmaf(sc[i], x, vs);
        }
        lp = fmaf(ws, se[p], lp);
        vp = fmaf(vs, dr[k], vp);
      }
      w[k] = ws;
    }
    const float l = wave_sum(lp) * scale;
    const float dp = wave_sum(vp);
    const float pj = expf(l - lse_t);
    const float dl = pj * (dp - D);
#pragma unroll
    for (int k = 0; k < 4; ++k) de[k] = fmaf(dl * scale, w[k], de[k]);
    // N side: sum_p dH[p][n] E_p and sum_p dH[p][n] dR_p, lanes over n
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = lane + 64 * k;
      if (n < N) {
        float ke = 0.f, kr = 0.f;
        for (int p = 0; p < P; ++p) {
          const float x = Elem<T>::ld(dj, (int64_t)p * N + n);
          ke = fmaf(x, se[p], ke);
          kr = fmaf(x, sr[p], kr);
        }
        dq[k] = fmaf(dl * scale, ke, dq[k]);
        dc[k] = fmaf(pj, kr, dc[k]);
      }
    }
    if (lane == 0) {
      const int64_t i = (bh * s.M + j) * s.L + t;
      pd[2 * i] = pj;
      pd[2 * i + 1] = dl;
    }
  }
  // per-head results: [b][L][Hout][...] with Hout = G (written directly) or H
  const int64_t orow = tok * head_stride_out + (head_stride_out == s.H ? h : g);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = lane + 64 * k, p = n;
    if (n < N) {
      dq_out[orow * N + n] = dq[k];
      dc_out[orow * N + n] = dc[k];
    }
    if (p < P) de_out[orow * P + p] = de[k];
  }
  if (dgate) {
    float gp = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = lane + 64 * k;
      if (p < P) {
        const float v = Elem<T>::ld(dout, row * P + p) * rr[k];
        if (gate_pc) dgate[row * P + p] = v;
        gp += v;
      }
    }
    gp = wave_sum(gp);
    if (!gate_pc && lane == 0) dgate[row] = gp;
  }
}

// (2) d_dH_c[p][n] = sum_{t >= (c+1)S} p_tc C_t[n] dR_t[p] + dl_tc Q_t[n] E_t[p] / sqrt(N);
// one thread per entry, one block per (b, h, c, 256 entries).
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_bwd_ddh_kernel(
    Shape s, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const T* __restrict__ gate, int gate_pc, const T* __restrict__ dout, const float* __restrict__ pd,
    float* __restrict__ ddh, int tiles) {
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tile = blockIdx.x % tiles;
  const int64_t c = (blockIdx.x / tiles) % s.M;
  const int64_t bh = blockIdx.x / tiles / s.M;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int64_t idx = tile * kThreads + threadIdx.x;  // p * N + n
  if (idx >= (int64_t)N * P) return;
  const int p = (int)(idx / N), n = (int)(idx % N);
  const float scale = 1.f / sqrtf((float)N);
  float acc = 0.f;
  const float* pdc = pd + 2 * (bh * s.M + c) * s.L;
  for (int64_t t = (c + 1) * s.S; t < s.L; ++t) {
    const int64_t tok = b * s.L + t;
    const int64_t row = tok * s.H + h;
    const float pj = pdc[2 * t], dl = pdc[2 * t + 1];
    const float gv = gate_pc ? Elem<T>::ld(gate, row * P + p) : Elem<T>::ld(gate, row);
    const float drp = gv * Elem<T>::ld(dout, row * P + p);
    const float cn = Elem<T>::ld(C, (tok * s.G + g) * N + n);
    const float qn = Elem<T>::ld(Q, (tok * s.G + g) * N + n);
    const float ep = Elem<T>::ld(E, (tok * s.G + g) * P + p);
    acc = fmaf(pj * cn, drp, acc);
    acc = fmaf(dl * scale * qn, ep, acc);
  }
  ddh[(bh * s.M + c) * (int64_t)P * N + idx] = acc;
}

// Sum over the heads of each group: out[r][g][k] = sum_{h in g} in[r][h][k].
__global__ __launch_bounds__(kThreads) void group_sum_kernel(const float* __restrict__ in,
                                                             float* __restrict__ out, int64_t rows,
                                                             int64_t G, int64_t hpg, int64_t K) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // over rows * G * K
  if (i >= rows * G * K) return;
  const int64_t k = i % K, gg = (i / K) % G, r = i / K / G;
  float acc = 0.f;
  for (int64_t j = 0; j < hpg; ++j) acc += in[((r * G + gg) * hpg + j) * K + k];
  out[i] = acc;
}

// (3) Chunk-state backward, one block per (b, h, c).  Token segments of 256
// are visited from the chunk end; the block forms the segment's weights with
// a suffix scan (carry = product of the later decays), then, token by token,
// dX_s[p] = w_s t_p with t_p = sum_n B_s[n] G[p][n], dw_s = sum_p X_s[p] t_p and
// dB_s[n] = w_s sum_p G[p][n] X_s[p].  w_s and dw_s go to the workspace.
template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_states_bwd_kernel(
    Shape s, const T* __restrict__ X, const T* __restrict__ B, const float* __restrict__ A,
    const float* __restrict__ ddh, float* __restrict__ dX, float* __restrict__ db_out,
    int64_t db_heads, float* __restrict__ wsw, float* __restrict__ wsdw) {
  __shared__ float s_scan[kThreads];
  __shared__ float s_x[256], s_b[256], s_red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = blockIdx.x % s.M, bh = blockIdx.x / s.M;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int64_t s0 = c * s.S, s1 = (s0 + s.S < s.L) ? s0 + s.S : s.L;
  const float* G = ddh + (bh * s.M + c) * (int64_t)P * N;
  float carry = 1.f;
  for (int64_t seg_end = s1; seg_end > s0; seg_end -= kThreads) {
    const int64_t seg0 = seg_end - kThreads > s0 ? seg_end - kThreads : s0;
    const int cnt = (int)(seg_end - seg0);
    // inclusive suffix product of a over the segment (Hillis-Steele)
    float v = tid < cnt ? A[(b * s.L + seg0 + tid) * s.H + h] : 1.f;
    s_scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const float u = tid + off < kThreads ? s_scan[tid + off] : 1.f;
      __syncthreads();
      v *= u;
      s_scan[tid] = v;
      __syncthreads();
    }
    const float w_self = carry * (tid + 1 < kThreads ? s_scan[tid + 1] : 1.f);
    const float seg_prod = s_scan[0];
    __syncthreads();
    s_scan[tid] = w_self;  // w of token seg0 + tid
    __syncthreads();
    for (int i = 0; i < cnt; ++i) {
      const int64_t sidx = seg0 + i;
      const int64_t tok = b * s.L + sidx;
      const float w = s_scan[i];
      for (int k = tid; k < P; k += kThreads) s_x[k] = Elem<T>::ld(X, (tok * s.H + h) * P + k);
      for (int k = tid; k < N; k += kThreads) s_b[k] = Elem<T>::ld(B, (tok * s.G + g) * N + k);
      __syncthreads();
      float part = 0.f;
      for (int p = tid; p < P; p += kThreads) {
        float tp = 0.f;
        for (int n = 0; n < N; ++n) tp = fmaf(s_b[n], G[(int64_t)p * N + n], tp);
        dX[(tok * s.H + h) * P + p] = w * tp;
        part = fmaf(s_x[p], tp, part);
      }
      for (int n = tid; n < N; n += kThreads) {
        float acc = 0.f;
        for (int p = 0; p < P; ++p) acc = fmaf(G[(int64_t)p * N + n], s_x[p], acc);
        db_out[(tok * db_heads + (db_heads == s.H ? h : g)) * N + n] = w * acc;
      }
      part = wave_sum(part);
      if (lane == 0) s_red[wave] = part;
      __syncthreads();
      if (tid == 0) {
        wsw[bh * s.L + sidx] = w;
        wsdw[bh * s.L + sidx] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
      }
      __syncthreads();
    }
    carry *= seg_prod;
  }
}

// (4) dA_k = w_k u_k with u_{s0} = 0, u_{k+1} = a_k u_k + dw_k: one wave per
// (b, h, c).  The recurrence is affine in u, so a chunk is scanned 256 tokens
// at a time: every lane composes the maps u -> a_k u + dw_k of its 4 tokens,
// a wave scan (log2 64 steps of lane shuffles) composes the lanes before it,
// and each lane then replays its own tokens from the u it starts with.  Only
// products and sums: exact where a_k = 0.
constexpr int kScanLanes = 64;

__global__ __launch_bounds__(kScanLanes) void decay_grad_kernel(Shape s, const float* __restrict__ A,
                                                                const float* __restrict__ wsw,
                                                                const float* __restrict__ wsdw,
                                                                float* __restrict__ dA) {
  const int64_t i = blockIdx.x;  // (b, h, c)
  const int64_t c = i % s.M, bh = i / s.M, b = bh / s.H, h = bh % s.H;
  const int64_t s0 = c * s.S, s1 = (s0 + s.S < s.L) ? s0 + s.S : s.L;
  const int lane = threadIdx.x;
  float carry = 0.f;  // u at the start of the current 256-token segment
  for (int64_t seg = s0; seg < s1; seg += 4 * kScanLanes) {
    float av[4], dw[4], wv[4];
    float al = 1.f, be = 0.f;  // this lane's map u -> al u + be
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = seg + 4 * lane + k;
      const bool ok = t < s1;
      av[k] = ok ? A[(b * s.L + t) * s.H + h] : 1.f;
      dw[k] = ok ? wsdw[bh * s.L + t] : 0.f;
      wv[k] = ok ? wsw[bh * s.L + t] : 0.f;
      be = fmaf(av[k], be, dw[k]);
      al *= av[k];
    }
    // inclusive scan of the maps over lanes: (al, be) <- (al, be) o (al', be')
#pragma unroll
    for (int d = 1; d < kScanLanes; d <<= 1) {
      const float pa = __shfl_up(al, d), pb = __shfl_up(be, d);
      if (lane >= d) {
        be = fmaf(al, pb, be);
        al *= pa;
      }
    }
    // exclusive: the lanes before this one applied to the segment's carry
    float ea = __shfl_up(al, 1), eb = __shfl_up(be, 1);
    if (lane == 0) {
      ea = 1.f;
      eb = 0.f;
    }
    float u = fmaf(ea, carry, eb);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = seg + 4 * lane + k;
      if (t < s1) dA[(b * s.L + t) * s.H + h] = wv[k] * u;
      u = fmaf(av[k], u, dw[k]);
    }
    carry = __shfl(u, kScanLanes - 1);
  }
}

inline unsigned grid1(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_group_sum(const float* in, float* out, int64_t rows, int64_t G, int64_t hpg,
                            int64_t K, hipStream_t st) {
  group_sum_kernel<<<grid1(rows * G * K), dim3(kThreads), 0, st>>>(in, out, rows, G, hpg, K);
  return hipGetLastError();
}

size_t sma_bwd_workspace_bytes(const Shape& s) {
  const int64_t pd = 2 * s.b * s.H * s.M * s.L;
  const int64_t heads = (s.H != s.G) ? s.b * s.L * s.H * (2 * s.N + s.P) : 0;
  return (size_t)(pd + heads) * sizeof(float);
}

hipError_t launch_sma_bwd_general(const Shape& s, bool bf16, const void* Q, const void* C,
                                  const void* E, const void* dH, const void* gate, int gate_pc,
                                  const float* R, const float* lse, const void* dout, float* dQ,
                                  float* dC, float* dE, float* ddH, float* dgate, float* ws,
                                  hipStream_t st) {
  float* pd = ws;
  const bool grouped = s.H != s.G;
  float* hq = grouped ? ws + 2 * s.b * s.H * s.M * s.L : dQ;
  float* hc = grouped ? hq + s.b * s.L * s.H * s.N : dC;
  float* he = grouped ? hc + s.b * s.L * s.H * s.N : dE;
  const int64_t hs = grouped ? s.H : s.G;
  const int64_t gph = (s.L + 3) / 4;
  const int tiles = (int)((s.N * s.P + kThreads - 1) / kThreads);
  // pd rows of chunks no token reads (and of the last chunk) are never
  // written; the d_dH kernel only reads entries of tokens in later chunks.
  if (bf16) {
    sma_bwd_token_kernel<bf16_t><<<dim3((unsigned)(s.b * s.H * gph)), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)Q, (const bf16_t*)C, (const bf16_t*)E, (const bf16_t*)dH,
        (const bf16_t*)gate, gate_pc, R, lse, (const bf16_t*)dout, hq, hc, he, hs, dgate, pd, gph);
    sma_bwd_ddh_kernel<bf16_t><<<dim3((unsigned)(s.b * s.H * s.M * tiles)), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)Q, (const bf16_t*)C, (const bf16_t*)E, (const bf16_t*)gate, gate_pc,
        (const bf16_t*)dout, pd, ddH, tiles);
  } else {
    sma_bwd_token_kernel<float><<<dim3((unsigned)(s.b * s.H * gph)), dim3(kThreads), 0, st>>>(
        s, (const float*)Q, (const float*)C, (const float*)E, (const float*)dH, (const float*)gate,
        gate_pc, R, lse, (const float*)dout, hq, hc, he, hs, dgate, pd, gph);
    sma_bwd_ddh_kernel<float><<<dim3((unsigned)(s.b * s.H * s.M * tiles)), dim3(kThreads), 0, st>>>(
        s, (const float*)Q, (const float*)C, (const float*)E, (const float*)gate, gate_pc,
        (const float*)dout, pd, ddH, tiles);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !grouped) return e;
  const int64_t rows = s.b * s.L, hpg = s.H / s.G;
  group_sum_kernel<<<grid1(rows * s.G * s.N), dim3(kThreads), 0, st>>>(hq, dQ, rows, s.G, hpg, s.N);
  group_sum_kernel<<<grid1(rows * s.G * s.N), dim3(kThreads), 0, st>>>(hc, dC, rows, s.G, hpg, s.N);
  group_sum_kernel<<<grid1(rows * s.G * s.P), dim3(kThreads), 0, st>>>(he, dE, rows, s.G, hpg, s.P);
  return hipGetLastError();
}

// Workspace of the chunk-state backward: w_s and dw_s [b][H][L] float32 each,
// then (grouped heads) per-head dB [b][L][H][N] float32 from the next
// 256-byte boundary (the matrix-core kernel writes it with 16-byte stores).
static int64_t cs_bwd_heads_offset(const Shape& s) { return (2 * s.b * s.H * s.L + 63) / 64 * 64; }

size_t chunk_states_bwd_workspace_bytes(const Shape& s) {
  const int64_t heads = (s.H != s.G) ? s.b * s.L * s.H * s.N : 0;
  return (size_t)(cs_bwd_heads_offset(s) + heads) * sizeof(float);
}

hipError_t launch_chunk_states_bwd_general(const Shape& s, bool bf16, bool mfma, const void* X,
                                           const void* B, const float* A, const float* ddH, float* dX,
                                           float* dB, float* dA, float* ws, hipStream_t st) {
  float* wsw = ws;
  float* wsdw = ws + s.b * s.H * s.L;
  const bool grouped = s.H != s.G;
  float* hb = grouped ? ws + cs_bwd_heads_offset(s) : dB;
  const int64_t hs = grouped ? s.H : s.G;
  const unsigned blocks = (unsigned)(s.b * s.H * s.M);
  if (mfma) {
    hipError_t e = launch_chunk_states_bwd_mfma(s, X, B, A, ddH, dX, hb, (int)hs, wsw, wsdw, st);
    if (e != hipSuccess) return e;
  } else if (bf16)
    chunk_states_bwd_kernel<bf16_t><<<dim3(blocks), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)X, (const bf16_t*)B, A, ddH, dX, hb, hs, wsw, wsdw);
  else
    chunk_states_bwd_kernel<float><<<dim3(blocks), dim3(kThreads), 0, st>>>(
        s, (const float*)X, (const float*)B, A, ddH, dX, hb, hs, wsw, wsdw);
  decay_grad_kernel<<<dim3((unsigned)(s.b * s.H * s.M)), dim3(kScanLanes), 0, st>>>(s, A, wsw, wsdw, dA);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !grouped) return e;
  const int64_t rows = s.b * s.L;
  group_sum_kernel<<<grid1(rows * s.G * s.N), dim3(kThreads), 0, st>>>(hb, dB, rows, s.G, s.H / s.G,
                                                                        s.N);
  return hipGetLastError();
}

}  // namespace dart
