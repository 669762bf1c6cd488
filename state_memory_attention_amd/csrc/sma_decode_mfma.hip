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
//   * per chunk a wave runs 16 v_mfma_f32_16x16x32_bf16 with A = [q; c; 0 ...]
//     and the memory as B, so lanes 0..15 receive W = q dH and V = c dH for 16
//     values of p each -- the matrix core does the dot products and the VALU
//     only runs the row-dot with e and the softmax;
//   * the plain decode stages each memory through a wave-private LDS ring in
//     four 4 KB row groups, loaded as whole 256-byte rows with the
//     non-temporal policy (6.9-7.0 TB/s on the decode workload, against
//     6.1-6.2 when the sixteen 16-byte loads per memory went straight into
//     the B-operand registers: each of those touched 16 rows x 64 bytes, so
//     two instructions shared every 128-byte line, and the non-temporal
//     policy then slowed them); the normalised branch, which also reads r_j
//     per chunk, keeps the direct loads;
//   * the 4 waves merge their (max, sum, O) states through LDS and write one
//     partial per range to the workspace; a second kernel merges the ranges
//     of each (b, h) in a fixed order (deterministic) and applies the gate.
//
// With the RMS-normalised score branch [App. B.1 Eq. 25-27] the query row of
// A becomes RMSNorm(q) w_q r_j, which changes per chunk: it is formed in
// float32 from r_j (read from the r cache beside each memory) and split into
// a bfloat16 high part (row 0) and the bfloat16 rounding of the remainder
// (row 2), so W = row 0 + row 2 of the product carries ~16 mantissa bits of
// the scaled query; the two extra rows cost nothing on the 16-row matrix op.
// RMSNorm(e) w_e and the per-token scales are folded into e once.
#include <mutex>

#include "dart.h"
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kThreads = 256;
constexpr int kMemBytes = kP * kN * 2;
constexpr float kTau = 8.f;
// LDS ring depth of the plain decode, per wave (4 KB stages: 64 KB a block, two
// blocks per CU; 6 and 8 stages measured the same)
constexpr int kDecStages = 4;

struct DecArgs {
  const bf16_t* q;
  const bf16_t* c;
  const bf16_t* e;
  const bf16_t* cache;
  const int32_t* n_chunks;
  const float* r_cache;  // normalised branch: [b][H][max_chunks][N]
  const float* wq;       // normalised branch: RMSNorm weights (nullable)
  const float* we;
  float* ws;
  int64_t max_chunks;
  int H, G, hpg, splits, cps;
  float e_scale;
  float eps;
};

__device__ __forceinline__ int64_t valid_chunks(const DecArgs& a, int b) {
  int64_t nb = a.n_chunks ? (int64_t)a.n_chunks[b] : a.max_chunks;
  return nb < 0 ? 0 : (nb > a.max_chunks ? a.max_chunks : nb);
}

template <bool kRms>
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

  // A operand rows: 0 = q, 1 = c, others zero (normalised branch: rows 0 and
  // 2 carry the two parts of the scaled query, set per chunk); lane holds
  // n = 32 kb + 8 kg + 0..7
  const bool qrow = row == 0 || (kRms && row == 2);
  bf16x8_t af[4];
  float qn[4][8];  // normalised branch: RMSNorm(q) w_q in float32
  {
    const bf16_t* src = qrow ? a.q : a.c;
    const int64_t base = ((int64_t)b * a.G + g) * kN + 8 * kg;
    float ss = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qrow || row == 1) v = *(const uint4*)(src + base + 32 * kb);
      af[kb] = __builtin_bit_cast(bf16x8_t, v);
      if (kRms) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qn[kb][2 * k] = bf16lo(w4[k]);
          qn[kb][2 * k + 1] = bf16hi(w4[k]);
          ss = fmaf(qn[kb][2 * k], qn[kb][2 * k], fmaf(qn[kb][2 * k + 1], qn[kb][2 * k + 1], ss));
        }
      }
    }
    if (kRms) {
      // the four lanes of a row (kg = 0..3) hold the whole query [Eq. 25]
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float inv_q = 1.f / sqrtf(ss * (1.f / kN) + a.eps);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) qn[kb][i] *= inv_q * (a.wq ? a.wq[32 * kb + 8 * kg + i] : 1.f);
    }
  }
  float ev[4];
  {
    float ss = 0.f;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      ev[pb] = lane < 16 ? bf16_to_f32(a.e[((int64_t)b * a.G + g) * kP + 16 * pb + lane]) : 0.f;
      ss = fmaf(ev[pb], ev[pb], ss);
    }
    float es = a.e_scale;
    if (kRms) {
      ss += __shfl_xor(ss, 8);
      ss += __shfl_xor(ss, 4);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 1);
      es *= 1.f / sqrtf(ss * (1.f / kP) + a.eps);
    }
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      ev[pb] *= es;
      if (kRms && a.we && lane < 16) ev[pb] *= a.we[16 * pb + lane];
    }
  }
  const float* rhead = kRms ? a.r_cache + (int64_t)bh * a.max_chunks * kN + 8 * kg : nullptr;

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
    if (kRms && qrow) {
      // query row of chunk j: RMSNorm(q) w_q r_j, high part on row 0, the
      // rounding of the remainder on row 2
      const float* rj = rhead + j * kN;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 r0 = *(const float4*)(rj + 32 * kb);
        const float4 r1 = *(const float4*)(rj + 32 * kb + 4);
        const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        uint32_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = qn[kb][2 * k] * rv[2 * k], x1 = qn[kb][2 * k + 1] * rv[2 * k + 1];
          const uint32_t hi = pack_bf16x2(x0, x1);
          pk[k] = row == 0 ? hi : pack_bf16x2(x0 - bf16lo(hi), x1 - bf16hi(hi));
        }
        af[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      }
    }
    float part = 0.f;
    f32x4_t acc[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      acc[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kb], bf[pb][kb], acc[pb], 0, 0, 0);
      // lanes 0..15: W[16 pb + lane] * e' (normalised branch: rows 0 + 2)
      part = fmaf(kRms ? acc[pb][0] + acc[pb][2] : acc[pb][0], ev[pb], part);
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

// Non-normalised decode with the cached memories staged through a wave-private
// LDS ring: a stage is one 16-row group of a memory (4 KB, rows p = 16 pb ..
// 16 pb + 15), loaded by four direct-to-LDS instructions of whole 256-byte
// rows with the non-temporal policy; the MFMA B operands are read from there
// (pieces XOR-swizzled by row, conflict-free).  Every stage index issues
// exactly four loads (zero-length ones past the wave's last chunk), so the
// wait before a stage always lets the next kStg - 1 stages stay in flight.
template <int kStg>
__global__ __launch_bounds__(kThreads) void sma_decode_partial_lds_kernel(DecArgs a) {
  // one LDS object (the ring, then the merge area): with a single object the
  // compiler adds no wait of its own for the ring loads before each read
  constexpr int kRingBytes = 4 * kStg * 4096;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kRingBytes + (4 * kP + 8) * 4];
  uint8_t* const s_ring = s_lds;
  float (*const s_o)[kP] = (float (*)[kP])(s_lds + kRingBytes);
  float* const s_m = (float*)(s_lds + kRingBytes + 4 * kP * 4);
  float* const s_d = s_m + 4;

  const int split = blockIdx.x % a.splits;
  const int bh = blockIdx.x / a.splits;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int64_t nb = valid_chunks(a, b);
  const int64_t c_begin = (int64_t)split * a.cps;
  if (c_begin >= nb) return;  // whole block: this range holds no valid chunk
  const int64_t c_end = (c_begin + a.cps < nb) ? c_begin + a.cps : nb;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int row = lane & 15, kg = lane >> 4;
  (void)h;

  // this wave's chunks c_begin + wave + 4 k, k < n_my; stage s = 4 k + pb
  const int64_t span = c_end - c_begin - wave;
  const int n_my = span > 0 ? (int)((span + 3) / 4) : 0;
  const int total = 4 * n_my;
  const uint8_t* head = (const uint8_t*)(a.cache + (int64_t)bh * a.max_chunks * (kP * kN));
  uint8_t* const ring = s_ring + wave * (kStg * 4096);
  auto issue = [&](int s) {
    const bool live = s < total;
    const uint8_t* base = live ? head + (c_begin + wave + 4 * (int64_t)(s >> 2)) * kMemBytes + (s & 3) * 4096 : head;
    const auto rs = buf_rsrc(wave_uniform(base), live ? 4096u : 0u);
    uint8_t* dst = ring + (s % kStg) * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + (lane >> 4);  // row of the stage this lane fills
      buf_dma16_nt(rs, (uint32_t)(r * 256 + (((lane & 15) ^ r) << 4)), dst + i * 1024);
    }
  };
#pragma unroll
  for (int s = 0; s < kStg; ++s) issue(s);

  // A operand rows: 0 = q, 1 = c, others zero; lane holds n = 32 kb + 8 kg + 0..7
  bf16x8_t af[4];
  {
    const bool qrow = row == 0;
    const bf16_t* src = qrow ? a.q : a.c;
    const int64_t base = ((int64_t)b * a.G + g) * kN + 8 * kg;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qrow || row == 1) v = *(const uint4*)(src + base + 32 * kb);
      af[kb] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  float ev[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
    ev[pb] = (lane < 16 ? bf16_to_f32(a.e[((int64_t)b * a.G + g) * kP + 16 * pb + lane]) : 0.f) * a.e_scale;

  float m = -INFINITY, d = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n_my; ++k) {
    float part = 0.f;
    f32x4_t acc[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const int s = 4 * k + pb;
      // stage s has landed; stages s+1 .. s+kStg-1 may stay in flight
      __builtin_amdgcn_s_waitcnt(0x0f70 | (4 * (kStg - 1) & 15) | ((4 * (kStg - 1) >> 4) << 14));
      asm volatile("" ::: "memory");
      const uint8_t* src = ring + (s % kStg) * 4096 + row * 256;
      bf16x8_t bf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) bf[kb] = *(const bf16x8_t*)(src + (((4 * kb + kg) ^ row) << 4));
      // the reads are done before the buffer is refilled
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("" ::: "memory");
      issue(s + kStg);
      acc[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kb], bf[kb], acc[pb], 0, 0, 0);
      part = fmaf(acc[pb][0], ev[pb], part);
    }
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
    for (int pb = 0; pb < 4; ++pb) o[pb] = fmaf(pj, acc[pb][1], o[pb]);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the stand-in stages have landed

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

// Split partials of dart_sma_decode_noalloc.  Each GPU holds its own copy of
// this array until the process ends.  In host code its name is a host-side
// stand-in, not a device address: host code uses only the address that
// hipGetSymbolAddress returns for the current device (decode_scratch below).
// The partials need no clearing: the combine kernel reads only the ranges
// whose blocks wrote them in the same call.
static __device__ __align__(256) float scratch[DART_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = (float*)p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_sma_decode_mfma(const Shape& s, int64_t max_chunks, const DecodePlan& plan,
                                  const void* q, const void* c, const void* e, const void* cache,
                                  const int32_t* n_chunks, const void* y, const void* gate,
                                  int gate_pc, void* out, float* R, float* lse, float* ws,
                                  const float* r_cache, const float* wq, const float* we, float eps,
                                  hipStream_t st) {
  DecArgs a;
  a.r_cache = r_cache;
  a.wq = wq;
  a.we = we;
  a.eps = eps;
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
    if (r_cache)
      sma_decode_partial_kernel<true><<<dim3((unsigned)(bh * plan.splits)), dim3(kThreads), 0, st>>>(a);
    else
      sma_decode_partial_lds_kernel<kDecStages><<<dim3((unsigned)(bh * plan.splits)), dim3(kThreads), 0, st>>>(a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  sma_decode_combine_kernel<<<dim3((unsigned)bh), dim3(kP), 0, st>>>(
      a, (const bf16_t*)y, (const bf16_t*)gate, gate_pc, (bf16_t*)out, R, lse);
  return hipGetLastError();
}

}  // namespace dart
