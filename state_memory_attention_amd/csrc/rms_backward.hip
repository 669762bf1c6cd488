// Backward of the RMS-normalised score branch, general kernels (any N, P <= 256;
// float32 or bfloat16 inputs, float32 arithmetic and float32 gradients).
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), App. B.1 Eq. 25-27
// differentiated, with the recomputation of §4 "Efficient Training" and
// App. C Eq. 33-35.  Forward, per token t and earlier chunk c:
//   zq = Q_t rho_q, rho_q = (mean Q_t^2 + eps)^(-1/2), qn = zq * w_q   (ze, en from E_t, w_e)
//   r_c[n] = (mean_p dH_c[p][n]^2 + eps)^(-1/2)
//   l_tc = sum_{n,p} qn[n] r_c[n] dH_c[p][n] en[p] / sqrt(N),   V_tc = C_t dH_c
// and the plain branch's softmax and readout.  Backward, with p_tc = exp(l_tc - lse_t)
// recomputed from the score memory dHs_c[p][n] = w_e[p] dH_c[p][n] r_c[n] w_q[n]
// exactly as the forward formed the logits:
//   dl_tc  = p_tc (dR_t . V_tc - dR_t . R_t)
//   dqn_t  = sum_c dl_tc r_c * (dH_c en_t) / sqrt(N)          (gradient of qn)
//   den_t  = sum_c dl_tc dH_c^T (r_c * qn_t) / sqrt(N)        (gradient of en)
//   dC_t   = sum_c p_tc dH_c dR_t
//   dS_c   = sum_t dl_tc qn_t en_t^T / sqrt(N)                (gradient of diag(r_c) dH_c)
//   d_dH_c = sum_t p_tc C_t^T dR_t + r_c * dS_c
//            - (r_c^3 / P) * dH_c * sum_p (dS_c * dH_c)       (through r_c)
//   dQ_t   = rho_q dzq - rho_q^3 Q_t (Q_t . dzq) / N,  dzq = w_q * sum_{heads} dqn_t
//   dw_q   = sum over tokens and groups of zq * sum_{heads} dqn_t       (E alike)
//
// Kernels: (1) one wave per (token, head): logits, weights, dqn, den, dC and
// (p, dl) per (chunk, token); (2) one thread per entry of each chunk memory:
// the readout term of d_dH and dS; (3) one thread per key row n of each chunk
// memory: r_c and the chain through r_c; (4) one wave per (token, group): the
// sums over the group's heads and the RMSNorm backward of Q_t and E_t, plus
// the per-row terms of dw_q, dw_e; (5) column sums of those terms in a fixed
// order (two passes), so every result is deterministic.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workspace regions, float32, each starting on a 256-byte boundary.
struct RmsBwdWs {
  int64_t pd, hq, he, hc, rho, ds, wpq, wpe, part, total;
};

RmsBwdWs rms_bwd_layout(const Shape& s) {
  auto up = [](int64_t n) { return (n + 63) / 64 * 64; };
  RmsBwdWs w;
  int64_t o = 0;
  w.pd = o;  o += up(2 * s.b * s.H * s.M * s.L);
  w.hq = o;  o += up(s.b * s.L * s.H * s.N);
  w.he = o;  o += up(s.b * s.L * s.H * s.P);
  w.hc = o;  o += (s.H != s.G) ? up(s.b * s.L * s.H * s.N) : 0;
  w.rho = o; o += up(2 * s.b * s.L * s.G);
  w.ds = o;  o += up(s.b * s.H * s.M * s.P * s.N);
  w.wpq = o; o += up(s.b * s.L * s.G * s.N);
  w.wpe = o; o += up(s.b * s.L * s.G * s.P);
  w.part = o; o += up(col_sum_split(s.b * s.L * s.G) * (s.N + s.P));
  w.total = o;
  return w;
}

// (1) Token kernel.  Lanes own n = lane + 64 k for the key-side sums (r_c,
// dH_c en, dH_c dR) and p = lane + 64 k for the value-side sums (logit, V,
// dH_c^T (r qn)).
template <typename T, typename TS>
__global__ __launch_bounds__(kThreads) void sma_bwd_rms_token_kernel(
    Shape s, float eps, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const T* __restrict__ dH, const TS* __restrict__ dHs, const float* __restrict__ wq,
    const float* __restrict__ we, const T* __restrict__ gate, int gate_pc,
    const float* __restrict__ R, const float* __restrict__ lse, const T* __restrict__ dout,
    float* __restrict__ hq, float* __restrict__ he, float* __restrict__ dc_out,
    int64_t dc_heads, float* __restrict__ rho, float* __restrict__ dgate, float* __restrict__ pd,
    int64_t groups_per_head) {
  __shared__ float s_zq[4][256], s_qn[4][256], s_c[4][256], s_en[4][256], s_dr[4][256], s_r[4][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / groups_per_head;
  const int64_t t = (blockIdx.x % groups_per_head) * 4 + wave;
  if (t >= s.L) return;  // no block-level barrier below
  const int64_t hpg = s.H / s.G;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / hpg;
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tok = b * s.L + t;
  const int64_t row = tok * s.H + h;  // [b][L][H] row
  const int64_t n_hist = t / s.S;
  const float scale = 1.f / sqrtf((float)N);
  const T* q = Q + (tok * s.G + g) * N;
  const T* c = C + (tok * s.G + g) * N;
  const T* e = E + (tok * s.G + g) * P;

  float* zq = s_zq[wave];
  float* qn = s_qn[wave];
  float* sc = s_c[wave];
  float* en = s_en[wave];
  float* sdr = s_dr[wave];
  float* sr = s_r[wave];

  // RMSNorm of Q_t and E_t [Eq. 25]
  float ssq = 0.f, sse = 0.f;
  for (int i = lane; i < N; i += 64) {
    const float x = Elem<T>::ld(q, i);
    ssq = fmaf(x, x, ssq);
  }
  for (int i = lane; i < P; i += 64) {
    const float x = Elem<T>::ld(e, i);
    sse = fmaf(x, x, sse);
  }
  const float rq = 1.f / sqrtf(wave_sum(ssq) / (float)N + eps);
  const float re = 1.f / sqrtf(wave_sum(sse) / (float)P + eps);
  for (int i = lane; i < N; i += 64) {
    const float z = Elem<T>::ld(q, i) * rq;
    zq[i] = z;
    qn[i] = wq ? z * wq[i] : z;
    sc[i] = Elem<T>::ld(c, i);
  }
  const float gs = gate_pc ? 0.f : Elem<T>::ld(gate, row);
  float ze[4], dr[4], rr[4], part = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    ze[k] = dr[k] = rr[k] = 0.f;
    if (p < P) {
      ze[k] = Elem<T>::ld(e, p) * re;
      en[p] = we ? ze[k] * we[p] : ze[k];
      dr[k] = (gate_pc ? Elem<T>::ld(gate, row * P + p) : gs) * Elem<T>::ld(dout, row * P + p);
      sdr[p] = dr[k];
      rr[k] = R[row * P + p];
    }
    part = fmaf(dr[k], rr[k], part);
  }
  const float D = wave_sum(part);
  if (lane == 0 && h % hpg == 0) {  // one head of the group stores the token's factors
    rho[2 * (tok * s.G + g)] = rq;
    rho[2 * (tok * s.G + g) + 1] = re;
  }
  wave_sync();

  const float lse_t = lse[bh * s.L + t];
  float dqn[4] = {0.f, 0.f, 0.f, 0.f}, dc[4] = {0.f, 0.f, 0.f, 0.f}, den[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t mem_off = bh * s.M * (int64_t)P * N;
  for (int64_t j = 0; j < n_hist; ++j) {
    const T* dj = dH + mem_off + j * (int64_t)P * N;
    const TS* sj = dHs + mem_off + j * (int64_t)P * N;
    // key side: r_c[n], sum_p dH[p][n] en[p], sum_p dH[p][n] dR[p]
    float ke[4], kr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = lane + 64 * k;
      ke[k] = kr[k] = 0.f;
      if (n < N) {
        float ss = 0.f, a = 0.f, bsum = 0.f;
        for (int p = 0; p < P; ++p) {
          const float x = Elem<T>::ld(dj, (int64_t)p * N + n);
          ss = fmaf(x, x, ss);
          a = fmaf(x, en[p], a);
          bsum = fmaf(x, sdr[p], bsum);
        }
        const float rn = 1.f / sqrtf(ss / (float)P + eps);  // [Eq. 26]
        sr[n] = rn;
        ke[k] = rn * a;
        kr[k] = bsum;
      }
    }
    wave_sync();
    // value side: the logit from the score memory (as the forward), V, dH^T (r qn)
    float wr[4], lp = 0.f, vp = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = lane + 64 * k;
      float ws = 0.f, vs = 0.f, us = 0.f;
      if (p < P) {
        const T* rowp = dj + (int64_t)p * N;
        const TS* srow = sj + (int64_t)p * N;
        for (int i = 0; i < N; ++i) {
          const float x = Elem<T>::ld(rowp, i);
          ws = fmaf(zq[i], Elem<TS>::ld(srow, i), ws);
          vs = fmaf(sc[i], x, vs);
          us = fmaf(qn[i] * sr[i], x, us);
        }
      }
      lp = fmaf(ws, ze[k], lp);
      vp = fmaf(vs, dr[k], vp);
      wr[k] = us;
    }
    const float l = wave_sum(lp) * scale;
    const float dp = wave_sum(vp);
    const float pj = expf(l - lse_t);
    const float dl = pj * (dp - D);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      den[k] = fmaf(dl * scale, wr[k], den[k]);
      dqn[k] = fmaf(dl * scale, ke[k], dqn[k]);
      dc[k] = fmaf(pj, kr[k], dc[k]);
    }
    if (lane == 0) {
      const int64_t i = (bh * s.M + j) * s.L + t;
      pd[2 * i] = pj;
      pd[2 * i + 1] = dl;
    }
    wave_sync();  // sr is rewritten by the next chunk
  }
  const int64_t orow = tok * dc_heads + (dc_heads == s.H ? h : g);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = lane + 64 * k, p = n;
    if (n < N) {
      hq[row * N + n] = dqn[k];
      dc_out[orow * N + n] = dc[k];
    }
    if (p < P) he[row * P + p] = den[k];
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

// (2) Per entry (p, n) of chunk memory c, over the tokens of later chunks:
//   ddh = sum_t p_tc C_t[n] dR_t[p],   ds = sum_t dl_tc qn_t[n] en_t[p] / sqrt(N).
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_bwd_rms_ddh_kernel(
    Shape s, const T* __restrict__ Q, const T* __restrict__ C, const T* __restrict__ E,
    const float* __restrict__ wq, const float* __restrict__ we, const T* __restrict__ gate,
    int gate_pc, const T* __restrict__ dout, const float* __restrict__ pd,
    const float* __restrict__ rho, float* __restrict__ ddh, float* __restrict__ ds, int tiles) {
  const int N = (int)s.N, P = (int)s.P;
  const int64_t tile = blockIdx.x % tiles;
  const int64_t c = (blockIdx.x / tiles) % s.M;
  const int64_t bh = blockIdx.x / tiles / s.M;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int64_t idx = tile * kThreads + threadIdx.x;  // p * N + n
  if (idx >= (int64_t)N * P) return;
  const int p = (int)(idx / N), n = (int)(idx % N);
  const float scale = 1.f / sqrtf((float)N);
  const float wqn = wq ? wq[n] : 1.f, wep = we ? we[p] : 1.f;
  float acc_v = 0.f, acc_s = 0.f;
  const float* pdc = pd + 2 * (bh * s.M + c) * s.L;
  for (int64_t t = (c + 1) * s.S; t < s.L; ++t) {
    const int64_t tok = b * s.L + t;
    const int64_t row = tok * s.H + h;
    const int64_t tg = tok * s.G + g;
    const float pj = pdc[2 * t], dl = pdc[2 * t + 1];
    const float gv = gate_pc ? Elem<T>::ld(gate, row * P + p) : Elem<T>::ld(gate, row);
    const float drp = gv * Elem<T>::ld(dout, row * P + p);
    const float cn = Elem<T>::ld(C, tg * N + n);
    const float qv = Elem<T>::ld(Q, tg * N + n) * rho[2 * tg] * wqn;
    const float ev = Elem<T>::ld(E, tg * P + p) * rho[2 * tg + 1] * wep;
    acc_v = fmaf(pj * cn, drp, acc_v);
    acc_s = fmaf(dl * qv, ev, acc_s);
  }
  const int64_t o = (bh * s.M + c) * (int64_t)P * N + idx;
  ddh[o] = acc_v;
  ds[o] = acc_s * scale;
}

// (3) Through S_c = diag(r_c) dH_c: per key row n of chunk memory c,
//   ddh[p][n] += r dS[p][n] - (r^3 / P) dH[p][n] sum_p' dS[p'][n] dH[p'][n].
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_bwd_rms_chain_kernel(
    int64_t n_rows, int N, int P, float eps, const T* __restrict__ dH, const float* __restrict__ ds,
    float* __restrict__ ddh) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // over (memory, n)
  if (i >= n_rows) return;
  const int64_t mem = i / N;
  const int n = (int)(i % N);
  const int64_t base = mem * (int64_t)P * N + n;
  float ss = 0.f, tdot = 0.f;
  for (int p = 0; p < P; ++p) {
    const float x = Elem<T>::ld(dH, base + (int64_t)p * N);
    ss = fmaf(x, x, ss);
    tdot = fmaf(ds[base + (int64_t)p * N], x, tdot);
  }
  const float r = 1.f / sqrtf(ss / (float)P + eps);
  const float k3 = r * r * r / (float)P * tdot;
  for (int p = 0; p < P; ++p) {
    const int64_t o = base + (int64_t)p * N;
    const float x = Elem<T>::ld(dH, o);
    ddh[o] = fmaf(r, ds[o], fmaf(-k3, x, ddh[o]));
  }
}

// (4) One wave per (token, group): sums of dqn, den over the group's heads,
// RMSNorm backward of Q_t and E_t, and the per-row weight-gradient terms.
template <typename T>
__global__ __launch_bounds__(kThreads) void sma_bwd_rms_norm_kernel(
    Shape s, const T* __restrict__ Q, const T* __restrict__ E, const float* __restrict__ wq,
    const float* __restrict__ we, const float* __restrict__ hq, const float* __restrict__ he,
    const float* __restrict__ rho, float* __restrict__ dQ, float* __restrict__ dE,
    float* __restrict__ wpq, float* __restrict__ wpe) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tg = (int64_t)blockIdx.x * 4 + wave;  // (b, t, g)
  if (tg >= s.b * s.L * s.G) return;
  const int64_t hpg = s.H / s.G;
  const int64_t tok = tg / s.G, g = tg % s.G;
  const int64_t h0 = tok * s.H + g * hpg;  // first [b][L][H] row of the group
  const int N = (int)s.N, P = (int)s.P;
  for (int side = 0; side < 2; ++side) {
    const int K = side ? P : N;
    const T* x = side ? E + tg * P : Q + tg * N;
    const float* w = side ? we : wq;
    const float* hsrc = side ? he : hq;
    const float r = rho[2 * tg + side];
    float dz[4], xv[4], part = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = lane + 64 * k;
      dz[k] = xv[k] = 0.f;
      if (i < K) {
        float acc = 0.f;
        for (int64_t j = 0; j < hpg; ++j) acc += hsrc[(h0 + j) * K + i];
        xv[k] = Elem<T>::ld(x, i);
        float* wp = side ? wpe : wpq;
        if (wp) wp[tg * K + i] = acc * xv[k] * r;  // d w_i = d(normalised)_i * z_i
        dz[k] = w ? acc * w[i] : acc;
        part = fmaf(xv[k], dz[k], part);
      }
    }
    const float dot = wave_sum(part);
    const float c3 = r * r * r * dot / (float)K;
    float* out = side ? dE + tg * P : dQ + tg * N;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = lane + 64 * k;
      if (i < K) out[i] = fmaf(r, dz[k], -c3 * xv[k]);
    }
  }
}

// (5) out[split][k] = sum of in[row][k] over rows split*chunk .. +chunk, in
// row order per wave, then over the block's four waves in order.
__global__ __launch_bounds__(kThreads) void col_sum_kernel(const float* __restrict__ in,
                                                           float* __restrict__ out, int64_t rows,
                                                           int K, int64_t chunk) {
  __shared__ float s_red[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = (int)blockIdx.x * 64 + lane;
  const int64_t split = blockIdx.y;
  const int64_t r0 = split * chunk;
  const int64_t r1 = r0 + chunk < rows ? r0 + chunk : rows;
  float acc = 0.f;
  if (k < K)
    for (int64_t r = r0 + wave; r < r1; r += 4) acc += in[r * K + k];
  s_red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && k < K) out[split * K + k] = ((s_red[0][lane] + s_red[1][lane]) + s_red[2][lane]) + s_red[3][lane];
}

template <typename T, typename TS>
hipError_t launch_rms_bwd(const Shape& s, float eps, const void* Qv, const void* Cv, const void* Ev,
                          const void* dHv, const void* dHsv, const float* wq, const float* we,
                          const void* gatev, int gate_pc, const float* R, const float* lse,
                          const void* doutv, float* dQ, float* dC, float* dE, float* ddH,
                          float* dgate, float* dwq, float* dwe, float* ws, hipStream_t st) {
  const T* Q = (const T*)Qv;
  const T* C = (const T*)Cv;
  const T* E = (const T*)Ev;
  const T* dH = (const T*)dHv;
  const TS* dHs = (const TS*)dHsv;
  const T* gate = (const T*)gatev;
  const T* dout = (const T*)doutv;
  const RmsBwdWs w = rms_bwd_layout(s);
  const bool grouped = s.H != s.G;
  float* hc = grouped ? ws + w.hc : dC;
  const int64_t gph = (s.L + 3) / 4;
  sma_bwd_rms_token_kernel<T, TS><<<dim3((unsigned)(s.b * s.H * gph)), dim3(kThreads), 0, st>>>(
      s, eps, Q, C, E, dH, dHs, wq, we, gate, gate_pc, R, lse, dout, ws + w.hq, ws + w.he, hc,
      grouped ? s.H : s.G, ws + w.rho, dgate, ws + w.pd, gph);
  const int tiles = (int)((s.N * s.P + kThreads - 1) / kThreads);
  sma_bwd_rms_ddh_kernel<T><<<dim3((unsigned)(s.b * s.H * s.M * tiles)), dim3(kThreads), 0, st>>>(
      s, Q, C, E, wq, we, gate, gate_pc, dout, ws + w.pd, ws + w.rho, ddH, ws + w.ds, tiles);
  const int64_t n_rows = s.b * s.H * s.M * s.N;
  sma_bwd_rms_chain_kernel<T><<<dim3((unsigned)((n_rows + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                                st>>>(n_rows, (int)s.N, (int)s.P, eps, dH, ws + w.ds, ddH);
  const int64_t tgs = s.b * s.L * s.G;
  sma_bwd_rms_norm_kernel<T><<<dim3((unsigned)((tgs + 3) / 4)), dim3(kThreads), 0, st>>>(
      s, Q, E, wq, we, ws + w.hq, ws + w.he, ws + w.rho, dQ, dE, dwq ? ws + w.wpq : nullptr,
      dwe ? ws + w.wpe : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dwq && (e = launch_col_sum(ws + w.wpq, ws + w.part, dwq, tgs, (int)s.N, st)) != hipSuccess) return e;
  if (dwe && (e = launch_col_sum(ws + w.wpe, ws + w.part, dwe, tgs, (int)s.P, st)) != hipSuccess) return e;
  if (grouped) return launch_group_sum(hc, dC, s.b * s.L, s.G, s.H / s.G, s.N, st);
  return hipSuccess;
}

}  // namespace

int64_t col_sum_split(int64_t rows) {
  const int64_t n = (rows + 63) / 64;  // parts of 64 rows (16 per wave), at most 1024
  return n < 1 ? 1 : (n > 1024 ? 1024 : n);
}

hipError_t launch_col_sum(const float* in, float* part, float* out, int64_t rows, int K, hipStream_t st) {
  const int64_t split = col_sum_split(rows);
  const int64_t chunk = (rows + split - 1) / split;
  const unsigned cols = (unsigned)((K + 63) / 64);
  col_sum_kernel<<<dim3(cols, (unsigned)split), dim3(kThreads), 0, st>>>(in, part, rows, K, chunk);
  col_sum_kernel<<<dim3(cols, 1), dim3(kThreads), 0, st>>>(part, out, split, K, split);
  return hipGetLastError();
}

size_t sma_bwd_rms_workspace_bytes(const Shape& s) { return (size_t)rms_bwd_layout(s).total * sizeof(float); }

hipError_t launch_sma_bwd_rms_general(const Shape& s, bool bf16, float eps, const void* Q, const void* C,
                                      const void* E, const void* dH, const void* dHs, const float* wq,
                                      const float* we, const void* gate, int gate_pc, const float* R,
                                      const float* lse, const void* dout, float* dQ, float* dC, float* dE,
                                      float* ddH, float* dgate, float* dwq, float* dwe, float* ws,
                                      hipStream_t st) {
  if (bf16)
    return launch_rms_bwd<bf16_t, _Float16>(s, eps, Q, C, E, dH, dHs, wq, we, gate, gate_pc, R, lse, dout, dQ,
                                            dC, dE, ddH, dgate, dwq, dwe, ws, st);
  return launch_rms_bwd<float, float>(s, eps, Q, C, E, dH, dHs, wq, we, gate, gate_pc, R, lse, dout, dQ, dC,
                                      dE, ddH, dgate, dwq, dwe, ws, st);
}

}  // namespace dart
