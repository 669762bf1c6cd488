// State-memory attention decode on gfx950: one new token per (b, h) against a
// cache of chunk memories, bfloat16 storage, N = 128, P = 64.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §4 "Inference Cache"
// (one chunk memory per chunk is the persistent cache) and §3 Eq. 8-11.
//
// The call reads every cached memory once (2 flop per byte), so it is bound
// by HBM.  Design:
//   * the chunk axis of each (b, h) is split into ranges; a block of 4 waves
//     owns one range and each wave streams every 4th chunk of it;
//   * per chunk a wave issues its sixteen 16-byte loads (the whole 16 KB
//     memory) straight into MFMA B-operand registers and runs 16
//     v_mfma_f32_16x16x32_bf16 with A = [q; c; 0 ...], so lanes 0..15 receive
//     W = q dH and V = c dH for 16 values of p each -- the matrix core does the
//     dot products and the VALU only runs the row-dot with e and the softmax;
//   * the 4 waves merge their (max, sum, O) states through LDS and write one
//     partial per range to the workspace; a second kernel merges the ranges
//     of each (b, h) in a fixed order (deterministic) and applies the gate.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kThreads = 256;
constexpr int kMemBytes = kP * kN * 2;
constexpr float kTau = 8.f;

struct DecArgs {
  const bf16_t* q;
  const bf16_t* c;
  const bf16_t* e;
  const bf16_t* cache;
  const int32_t* n_chunks;
  float* ws;
  int64_t max_chunks;
  int H, G, hpg, splits, cps;
  float e_scale;
};

__device__ __forceinline__ int64_t valid_chunks(const DecArgs& a, int b) {
  int64_t nb = a.n_chunks ? (int64_t)a.n_chunks[b] : a.max_chunks;
  return nb < 0 ? 0 : (nb > a.max_chunks ? a.max_chunks : nb);
}

__global__ __launch_bounds__(kThreads) void sma_decode_partial_kernel(DecArgs a) {
  __shared__ float s_m[4], s_d[4];
  __shared__ float s_o[4][kP];

  const int split = blockIdx.x % a.splits;
  const int bh = blockIdx.x / a.splits;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int64_t nb = valid_chunks(a, b);
  const int64_t c_begin = (int64_t)split * a.cps;
  if (c_begin >= nb) return;  // whole block: this range holds no valid chunk
  const int64_t c_end = (c_begin + a.cps < nb) ? c_begin + a.cps : nb;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = lane & 15, kg = lane >> 4;

  // A operand rows: 0 = q, 1 = c, others zero; lane holds n = 32 kb + 8 kg + 0..7
  bf16x8_t af[4];
  {
    const bf16_t* src = row == 0 ? a.q : a.c;
    const int64_t base = ((int64_t)b * a.G + g) * kN + 8 * kg;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < 2) v = *(const uint4*)(src + base + 32 * kb);
      af[kb] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  float ev[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
    ev[pb] = lane < 16 ? bf16_to_f32(a.e[((int64_t)b * a.G + g) * kP + 16 * pb + lane]) * a.e_scale
                       : 0.f;

  float m = -INFINITY, d = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* head = (const uint8_t*)(a.cache + (int64_t)bh * a.max_chunks * (kP * kN));
  // B operand: lane holds p = 16 pb + row, n = 32 kb + 8 kg + 0..7
  const int lofs = row * (kN * 2) + kg * 16;
  for (int64_t j = c_begin + wave; j < c_end; j += 4) {
    const uint8_t* cj = head + j * kMemBytes + lofs;
    bf16x8_t bf[4][4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        bf[pb][kb] = *(const bf16x8_t*)(cj + pb * 16 * (kN * 2) + kb * 64);
    float part = 0.f;
    f32x4_t acc[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      acc[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kb], bf[pb][kb], acc[pb], 0, 0, 0);
      part = fmaf(acc[pb][0], ev[pb], part);  // lanes 0..15: W[16 pb + lane] * e'
    }
    // row-dot over the 16 lanes of each lane group (only lanes 0..15 matter)
    part += __shfl_xor(part, 8);
    part += __shfl_xor(part, 4);
    part += __shfl_xor(part, 2);
    part += __shfl_xor(part, 1);
    const float l2 = part;
    const float mn = (l2 > m + kTau) ? l2 : m;
    if (__any(mn != m)) {
      const float alpha = (mn == m) ? 1.f : fast_exp2(m - mn);
      d *= alpha;
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) o[pb] *= alpha;
      m = mn;
    }
    const float pj = fast_exp2(l2 - m);
    d += pj;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) o[pb] = fmaf(pj, acc[pb][1], o[pb]);  // V[16 pb + lane]
  }

  // merge the 4 waves of the block
  if (lane < 16) {
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) s_o[wave][16 * pb + lane] = o[pb];
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_d[wave] = d;
  }
  __syncthreads();
  if (tid < kP) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_d[w] > 0.f) M = fmaxf(M, s_m[w]);
    float D = 0.f, Ov = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_d[w] > 0.f) {
        const float f = fast_exp2(s_m[w] - M);
        D = fmaf(s_d[w], f, D);
        Ov = fmaf(s_o[w][tid], f, Ov);
      }
    float* dst = a.ws + ((int64_t)bh * a.splits + split) * (kP + 2);
    if (tid == 0) {
      dst[0] = M;
      dst[1] = D;
    }
    dst[2 + tid] = Ov;
  }
}

// Merge the chunk ranges of one (b, h) in range order; gate and write.
__global__ __launch_bounds__(kP) void sma_decode_combine_kernel(
    DecArgs a, const bf16_t* __restrict__ y, const bf16_t* __restrict__ gate, int gate_pc,
    bf16_t* __restrict__ out, float* __restrict__ R, float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / a.H;
  const int p = threadIdx.x;
  const int64_t nb = valid_chunks(a, b);
  const int nsplit = (int)((nb + a.cps - 1) / a.cps);
  const float* src = a.ws + (int64_t)bh * a.splits * (kP + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    if (src[s * (kP + 2) + 1] > 0.f) M = fmaxf(M, src[s * (kP + 2)]);
  float D = 0.f, Ov = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ps = src + s * (kP + 2);
    if (ps[1] > 0.f) {
      const float f = fast_exp2(ps[0] - M);
      D = fmaf(ps[1], f, D);
      Ov = fmaf(ps[2 + p], f, Ov);
    }
  }
  const float r = D > 0.f ? Ov / D : 0.f;
  const int64_t i = (int64_t)bh * kP + p;
  const float gv = bf16_to_f32(gate_pc ? gate[i] : gate[bh]);
  out[i] = (bf16_t)f32_to_bf16(fmaf(gv, r, bf16_to_f32(y[i])));
  if (R) R[i] = r;
  if (lse && p == 0) lse[bh] = D > 0.f ? (M + fast_log2(D)) * kLn2 : -INFINITY;
}

}  // namespace

DecodePlan decode_plan(int64_t b, int64_t H, int64_t P, int64_t max_chunks) {
  DecodePlan plan;
  const int64_t bh = b * H;
  const int64_t target_blocks = 2048;
  int64_t splits = bh > 0 ? (target_blocks + bh - 1) / bh : 1;
  const int64_t max_splits = max_chunks > 4 ? (max_chunks + 3) / 4 : 1;  // >= 4 chunks a range
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t cps = max_chunks > 0 ? (max_chunks + splits - 1) / splits : 1;
  splits = max_chunks > 0 ? (max_chunks + cps - 1) / cps : 1;
  plan.splits = splits;
  plan.chunks_per_split = cps;
  plan.workspace_bytes = (size_t)(bh * splits * (P + 2)) * sizeof(float);
  return plan;
}

hipError_t launch_sma_decode_mfma(const Shape& s, int64_t max_chunks, const DecodePlan& plan,
                                  const void* q, const void* c, const void* e, const void* cache,
                                  const int32_t* n_chunks, const void* y, const void* gate,
                                  int gate_pc, void* out, float* R, float* lse, float* ws,
                                  hipStream_t st) {
  DecArgs a;
  a.q = (const bf16_t*)q;
  a.c = (const bf16_t*)c;
  a.e = (const bf16_t*)e;
  a.cache = (const bf16_t*)cache;
  a.n_chunks = n_chunks;
  a.ws = ws;
  a.max_chunks = max_chunks;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.splits = (int)plan.splits;
  a.cps = (int)plan.chunks_per_split;
  a.e_scale = kLog2e / sqrtf((float)kN);
  const int64_t bh = s.b * s.H;
  if (bh == 0) return hipSuccess;
  if (max_chunks > 0) {
    sma_decode_partial_kernel<<<dim3((unsigned)(bh * plan.splits)), dim3(kThreads), 0, st>>>(a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  sma_decode_combine_kernel<<<dim3((unsigned)bh), dim3(kP), 0, st>>>(
      a, (const bf16_t*)y, (const bf16_t*)gate, gate_pc, (bf16_t*)out, R, lse);
  return hipGetLastError();
}

}  // namespace dart
