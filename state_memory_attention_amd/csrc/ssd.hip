// The Mamba-2 SSM branch by the chunked scan: Y_t = C_t H_t with
// H_t = a_t H_{t-1} + B_t^T X_t, computed alongside the chunk state memories.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §2 Eq. 2 and App. A
// Eq. 15-24.  Per chunk c with first token a_c and last token b_c:
//   dH_[c] = sum_{s in c} A_{s+1:b_c} B_s^T X_s                  (Eq. 20)
//   H_[c]  = A_{a_c:b_c} H_[c-1] + dH_[c],  H_[-1] = H0          (Eq. 17-18)
//   Y_t    = sum_{s in c, s <= t} C_t A_{s+1:t} B_s^T X_s         (Eq. 21)
//          + C_t A_{a_c:t} H_[c-1]                               (Eq. 22)
// Four steps, each a kernel: the chunk states (the SMA's chunk memories,
// shared with dart_chunk_states), the full decay A_{a_c:b_c} of every chunk,
// the scan over chunks (writing the state entering each chunk), and the
// outputs.  Within a chunk the decays enter as
//   A_{s+1:t} = 2^(l_t - l_s),  l_t = sum_{k = a_c}^{t} log2 a_k,
// with tokens whose a_k = 0 left out of l and tracked instead as the last
// zero z_t at or before t: the product is 0 exactly when z_t > s.  Only
// products, sums and exponentials of sums: no division by a decay.
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4_ssd_t __attribute__((ext_vector_type(4)));
constexpr unsigned kWaitVm1 = 0x0f71;  // s_waitcnt vmcnt(1)

// ---------------------------------------------------------------------------
// Full decay of every chunk, A_{a_c:b_c}: one wave per (b, h, c).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void chunk_decay_kernel(Shape s, const float* __restrict__ A,
                                                         float* __restrict__ alpha) {
  const int64_t i = blockIdx.x;  // (b, h, c)
  const int64_t c = i % s.M, bh = i / s.M, b = bh / s.H, h = bh % s.H;
  const int64_t s0 = c * s.S, s1 = (s0 + s.S < s.L) ? s0 + s.S : s.L;
  float v = 1.f;
  for (int64_t t = s0 + threadIdx.x; t < s1; t += 64) v *= A[(b * s.L + t) * s.H + h];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v *= __shfl_xor(v, off);
  if (threadIdx.x == 0) alpha[i] = v;
}

// ---------------------------------------------------------------------------
// Scan over chunks: Hin_c = H_[c-1] (stored in the input dtype, the operand
// of the output kernel), H_[c] = alpha_c H_[c-1] + dH_[c] in float32.
// Every thread owns V consecutive entries of one (b, h) state.
// ---------------------------------------------------------------------------
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(Shape s, int64_t slices,
                                                              const T* __restrict__ dH,
                                                              const float* __restrict__ alpha,
                                                              const float* __restrict__ H0,
                                                              T* __restrict__ Hin,
                                                              float* __restrict__ Hfin) {
  const int64_t bh = blockIdx.x / slices;
  const int64_t e0 = ((blockIdx.x % slices) * kThreads + threadIdx.x) * V;
  const int64_t nPN = s.P * s.N;
  if (e0 >= nPN) return;
  float st[V];
#pragma unroll
  for (int k = 0; k < V; ++k) st[k] = (H0 && e0 + k < nPN) ? H0[bh * nPN + e0 + k] : 0.f;
  const T* src = dH + bh * s.M * nPN + e0;
  T* dst = Hin + bh * s.M * nPN + e0;
  const float* al = alpha + bh * s.M;
#pragma unroll 4
  for (int64_t c = 0; c < s.M; ++c) {
    const float a = al[c];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (V > 1 || e0 + k < nPN) {
        Elem<T>::st(dst + c * nPN, k, st[k]);
        st[k] = fmaf(a, st[k], Elem<T>::ld(src + c * nPN, k));
      }
    }
  }
  if (Hfin)
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (V > 1 || e0 + k < nPN) Hfin[bh * nPN + e0 + k] = st[k];
}

// ---------------------------------------------------------------------------
// Outputs, general kernel: one wave per token (any N, P <= 256).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void ssd_out_general_kernel(Shape s, const T* __restrict__ X,
                                                                   const T* __restrict__ B,
                                                                   const T* __restrict__ C,
                                                                   const float* __restrict__ A,
                                                                   const T* __restrict__ Hin,
                                                                   T* __restrict__ Y,
                                                                   int64_t groups_per_head) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / groups_per_head;
  const int64_t t = (blockIdx.x % groups_per_head) * 4 + wave;
  if (t >= s.L) return;
  const int64_t b = bh / s.H, h = bh % s.H, g = h / (s.H / s.G);
  const int N = (int)s.N, P = (int)s.P;
  const int64_t c = t / s.S, s0 = c * s.S;
  const T* ct = C + ((b * s.L + t) * s.G + g) * N;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  float dec = 1.f;  // A_{s+1:t}
  for (int64_t u = t; u >= s0; --u) {
    const T* bu = B + ((b * s.L + u) * s.G + g) * N;
    float part = 0.f;
    for (int n = lane; n < N; n += 64) part = fmaf(Elem<T>::ld(ct, n), Elem<T>::ld(bu, n), part);
    const float w = wave_sum(part) * dec;  // C_t A_{s+1:t} B_s^T  [Eq. 21]
    const T* xu = X + ((b * s.L + u) * s.H + h) * P;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (lane + 64 * k < P) y[k] = fmaf(w, Elem<T>::ld(xu, lane + 64 * k), y[k]);
    dec *= A[(b * s.L + u) * s.H + h];
  }
  // dec = A_{a_c:t} now: the inter-chunk readout [Eq. 22]
  const T* hc = Hin + (bh * s.M + c) * (int64_t)P * N;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = lane + 64 * k;
    if (p < P) {
      float v = 0.f;
      for (int n = 0; n < N; ++n) v = fmaf(Elem<T>::ld(ct, n), Elem<T>::ld(hc, (int64_t)p * N + n), v);
      Elem<T>::st(Y, ((b * s.L + t) * s.H + h) * P + p, fmaf(dec, v, y[k]));
    }
  }
}

// ---------------------------------------------------------------------------
// Outputs on the matrix core: bfloat16, N = 128, P = 64, S a multiple of 32
// up to 256.  One block per (b, h, chunk); the chunk's tokens form slices of
// 32, one per wave (eight waves; the two waves on a SIMD own slices w and
// 7 - w, equal causal work).  With one token per lane and P along registers
// (the transposed output Y^T), per slice:
//   Y^T  = Hin_c^T C^T  scaled per token by A_{a_c:t}         (Eq. 22)
//   for every 32-token block of earlier or equal tokens s:
//     G^T = B_s C^T  (32 s x 32 t),  masked and decayed by A_{s+1:t},
//     Y^T += X_s^T G^T                                          (Eq. 21)
// The blocks of s are visited by all waves together: block s is staged once
// in an LDS ring (three stages, two in flight) and serves every slice at or
// after it.  G^T leaves the matrix core with s along registers; a swap
// between the half-waves (v_permlane32_swap) puts 8 consecutive s in each
// lane, the layout of the next product's B operand, with no trip through
// LDS.  X^T is read from the chunk's X tile with the transposing LDS read;
// Hin_c^T and B_s like the chunk memories of the SMA forward (256-byte rows,
// pieces XOR-swizzled by the row).
// ---------------------------------------------------------------------------
constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kMaxS = 256;
constexpr int kBStage = 32 * kN * 2;  // 32 rows of B: 8 KB

struct SsdArgs {
  const bf16_t* X;
  const bf16_t* B;
  const bf16_t* C;
  const float* A;
  const bf16_t* Hin;
  bf16_t* Y;
  int64_t L;
  int H, G, hpg, S, M;
};

__device__ __forceinline__ int swz_x(int row) { return (row & 3) << 1; }

// Four transposing reads that return together (the compiler's own form of
// the read would drain the loads in flight before it).
__device__ __forceinline__ void ld_tr4(uint64_t (&o)[4], const uint32_t (&ad)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
}

// Four 16-byte LDS reads at addr + 32 i (i = 0..3) that return together.
// Written out so that the compiler, which cannot tell these reads from the
// B stage being filled by a direct-to-LDS load, does not drain that load
// (the next block's prefetch) before them.
__device__ __forceinline__ void ld_lds4(float4 (&o)[4], uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:32\n\t"
      "ds_read_b128 %2, %4 offset:64\n\t"
      "ds_read_b128 %3, %4 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(addr)
      : "memory");
}

// Intra-chunk terms of block j of s (32 tokens from sa = 32 j, staged at bst)
// for this wave's slice (the lane's token tl, its l_t and z_t): scores
// G^T = B_s C^T (C^T operands cq), weighted by 2^(l_t - l_s) for s <= t with
// no zero decay in (s, t], then Y^T += X_s^T G^T  [App. A Eq. 21].
__device__ __forceinline__ void ssd_intra_block(f32x16_t (&y)[2], const bf16x8_t (&cq)[8], float lt, int zt, int tl,
                                                const uint8_t* bst, const uint8_t* s_x, const float* s_l, int sa,
                                                int col, int half, int grp16, int j16) {
  f32x16_t gt = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8_t bo = *(const bf16x8_t*)(bst + mem_off(col, 2 * kk + half));
    gt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo, cq[kk], gt, 0, 0, 0);
  }
  // gt[r]: s = sa + 8 (r / 4) + 4 half + r % 4, t = tl
  float4 lsq[4];
  ld_lds4(lsq, lds_addr(s_l + sa + 4 * half));
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int sr = sa + 8 * jj + 4 * half;
    const float lsv[4] = {lsq[jj].x, lsq[jj].y, lsq[jj].z, lsq[jj].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sv = sr + e;
      const bool keep = sv <= tl && zt <= sv;
      gt[4 * jj + e] = keep ? gt[4 * jj + e] * fast_exp2(lt - lsv[e]) : 0.f;
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // s to 8 consecutive values per lane: swap registers r and r + 4
    // between the half-waves, then two k-steps of 16 s each
    float xs[4], ys[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(gt[8 * kb + e]),
                                                       __float_as_uint(gt[8 * kb + 4 + e]), false, false);
      xs[e] = __uint_as_float(sw[0]);
      ys[e] = __uint_as_float(sw[1]);
    }
    const bf16x8_t mop = __builtin_bit_cast(
        bf16x8_t, make_uint4(pack_bf16x2(xs[0], xs[1]), pack_bf16x2(xs[2], xs[3]), pack_bf16x2(ys[0], ys[1]),
                             pack_bf16x2(ys[2], ys[3])));
    // X^T operands (p rows, 8 consecutive s) from the X tile: lane (column
    // j16 + 16 grp16, k-octet half) receives tokens ... + 4 hh + 0..3 of read
    // hh, addressing token row ... + 4 hh + j16 / 4
    uint32_t ad[4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = sa + 16 * kb + 8 * half + 4 * hh + (j16 >> 2);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int pb = 32 * f + 16 * grp16 + 4 * (j16 & 3);
        ad[2 * f + hh] = lds_addr(s_x + r * 128 + (((pb >> 3) ^ swz_x(r)) << 4) + ((pb & 7) >> 2) * 8);
      }
    }
    uint64_t rd[4];
    ld_tr4(rd, ad);
    const bf16x8_t x0 = __builtin_bit_cast(bf16x8_t, make_uint4((uint32_t)rd[0], (uint32_t)(rd[0] >> 32),
                                                                (uint32_t)rd[1], (uint32_t)(rd[1] >> 32)));
    const bf16x8_t x1 = __builtin_bit_cast(bf16x8_t, make_uint4((uint32_t)rd[2], (uint32_t)(rd[2] >> 32),
                                                                (uint32_t)rd[3], (uint32_t)(rd[3] >> 32)));
    y[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x0, mop, y[0], 0, 0, 0);
    y[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x1, mop, y[1], 0, 0, 0);
  }
}

// Output kernel: eight waves, one 32-token slice each.  Waves w and w + 4
// share a SIMD and own slices w and 7 - w, so the causal work on every SIMD
// is the same and the two pairs a SIMD has in one block of s run in two
// waves, which overlap.
constexpr int kWavesOut = 8;
constexpr int kThreadsOut = 64 * kWavesOut;

// kNtB: B rows with the non-temporal policy (a group of one head: no other
// block reads them); X and the entering state always (read by this block only)
template <bool kNtB>
__global__ __launch_bounds__(kThreadsOut) __attribute__((amdgpu_waves_per_eu(4, 4)))
void ssd_out_mfma_kernel(SsdArgs a) {
  // One LDS object (so that the compiler adds no waits of its own for the
  // staged loads): X tile (128-byte rows), Hin_c^T, the B ring, l and z.
  constexpr int kOffH = kMaxS * kP * 2;
  constexpr int kOffB = kOffH + kP * kN * 2;
  constexpr int kOffL = kOffB + 3 * kBStage;
  constexpr int kOffZ = kOffL + kMaxS * 4;
  constexpr int kOffT = kOffZ + kMaxS * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kOffT + 32];
  uint8_t* const s_x = s_lds;
  uint8_t* const s_h = s_lds + kOffH;
  float* const s_l = (float*)(s_lds + kOffL);
  int* const s_z = (int*)(s_lds + kOffZ);
  float* const s_tl = (float*)(s_lds + kOffT);
  int* const s_tz = (int*)(s_lds + kOffT + 16);

  const int blk = blockIdx.x;
  const int BH = gridDim.x / a.M;
  const int c = blk / BH, bh = blk % BH;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5, grp16 = (lane >> 4) & 1, j16 = lane & 15;
  const int64_t s0 = (int64_t)c * a.S;
  const int clen = (int)((s0 + a.S < a.L) ? a.S : a.L - s0);
  const int n_sb = (clen + 31) / 32;  // blocks of 32 tokens holding data
  const int64_t row0 = (int64_t)b * a.L;
  // this thread's token decay (threads past the chunk, and the upper half of
  // the block, hold none), loaded before the staged loads so that waiting
  // for it leaves them in flight; without a branch (those threads re-read
  // the chunk's last token), so that the addresses below are not formed in
  // divergent code, where the compiler would keep the buffer resources in
  // vector registers and loop over lanes for every load
  const float a_raw = a.A[(row0 + s0 + (tid < clen ? tid : clen - 1)) * a.H + h];
  const float av = tid < clen ? a_raw : 1.f;

  // ---- staged loads.  X tile: wave w loads row groups w, w+8, ... (8 rows
  // of 128 B each); Hin_c^T: rows 8w .. 8w+7; B block j: rows 4w .. 4w+3 of
  // its stage (one load per wave).  Rows past the chunk end read as zeros.
  const auto rbb = buf_rsrc(wave_uniform(a.B + ((row0 + s0) * a.G + g) * kN), (uint32_t)((clen - 1) * a.G * kN + kN) * 2);
  auto issue_b = [&](int j) {
    uint8_t* st = s_lds + kOffB + (j % 3) * kBStage;
    const int r = 4 * wave + (lane >> 4);  // row within the block
    const int rr = 32 * j + r;             // row within the chunk
    const uint32_t off = (uint32_t)(rr * a.G * kN * 2 + (((lane & 15) ^ (r & 15)) << 4));
    if constexpr (kNtB)
      buf_dma16_nt(rbb, off, st + 4 * wave * 256);
    else
      buf_dma16(rbb, off, st + 4 * wave * 256);
  };
  {
    const auto rx = buf_rsrc(wave_uniform(a.X + ((row0 + s0) * a.H + h) * kP), (uint32_t)((clen - 1) * a.H * kP + kP) * 2);
    // every wave issues the same loads whatever the chunk length (groups
    // past it read zeros into rows nothing reads), so that the compiler's
    // wait for the decay load counts them all and leaves them in flight
#pragma unroll
    for (int i = 0; i < kMaxS / (8 * kWavesOut); ++i) {
      const int rb = 8 * (wave + kWavesOut * i);  // first row of the group
      const int r = rb + (lane >> 3);
      const int piece = (lane & 7) ^ swz_x(r);
      buf_dma16_nt(rx, (uint32_t)(r * a.H * kP + piece * 8) * 2, s_x + rb * 128);
    }
    const auto rh = buf_rsrc(wave_uniform(a.Hin + ((int64_t)bh * a.M + c) * (kP * kN)), kP * kN * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 8 * wave + 4 * i + (lane >> 4);
      buf_dma16_nt(rh, (uint32_t)(row * 256 + (((lane & 15) ^ (row & 15)) << 4)), s_h + (8 * wave + 4 * i) * 256);
    }
    issue_b(0);
    issue_b(1);
  }
  // ---- this wave's slice: C^T operands (lane holds a token, n = 16 kk +
  // 8 half + 0..7), issued with the staged loads: one round trip for all
  const int n_sl = a.S / 32;
  const int sl = wave < 4 ? wave : 11 - wave;
  const bool act = sl < n_sl && 32 * sl < clen;  // uniform per wave
  const int tl = 32 * sl + col;
  bf16x8_t cq[8];
  {
    const int64_t tg = row0 + s0 + (tl < clen ? tl : clen - 1);
    const bf16_t* cp = a.C + (tg * a.G + g) * kN + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) cq[kk] = *(const bf16x8_t*)(cp + 16 * kk);
  }
  // ---- l and z of the chunk's tokens (threads 0 .. kMaxS-1): block-wide
  // inclusive scans (sum, max)
  {
    float lv = av > 0.f ? fast_log2(av) : 0.f;
    int zv = (tid < clen && av == 0.f) ? tid : -1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float lu = __shfl_up(lv, off);
      const int zu = __shfl_up(zv, off);
      if (lane >= off) {
        lv += lu;
        zv = zu > zv ? zu : zv;
      }
    }
    if (lane == 63 && wave < kMaxS / 64) {
      s_tl[wave] = lv;
      s_tz[wave] = zv;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    if (wave < kMaxS / 64) {
      for (int w2 = 0; w2 < wave; ++w2) {
        lv += s_tl[w2];
        zv = s_tz[w2] > zv ? s_tz[w2] : zv;
      }
      s_l[tid] = lv;
      s_z[tid] = zv;
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  // this wave's slice's l_t and z_t
  const float lt = s_l[tl < kMaxS ? tl : kMaxS - 1];
  const int zt = s_z[tl < kMaxS ? tl : kMaxS - 1];

  // ---- inter-chunk readout, then its decay A_{a_c:t}  [Eq. 22]
  f32x16_t y[2] = {f32x16_t{}, f32x16_t{}};
  if (act) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8_t h0 = *(const bf16x8_t*)(s_h + mem_off(col, 2 * kk + half));
      const bf16x8_t h1 = *(const bf16x8_t*)(s_h + mem_off(32 + col, 2 * kk + half));
      y[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, cq[kk], y[0], 0, 0, 0);
      y[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, cq[kk], y[1], 0, 0, 0);
    }
    const float din = zt < 0 ? fast_exp2(lt) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      y[0][r] *= din;
      y[1][r] *= din;
    }
  }

  // ---- intra-chunk terms, all waves on block j of s together  [Eq. 21]
  for (int j = 0; j < n_sb; ++j) {
    if (j > 0) {
      // block j has landed (block j + 1 may still be in flight, one load per
      // wave); every wave is done with block j - 1, whose stage takes block
      // j + 2
      if (j + 1 < n_sb && j + 1 >= 2)
        __builtin_amdgcn_s_waitcnt(kWaitVm1);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
    }
    if (j + 2 < n_sb) issue_b(j + 2);
    if (act && sl >= j)  // uniform per wave
      ssd_intra_block(y, cq, lt, zt, tl, s_lds + kOffB + (j % 3) * kBStage, s_x, s_l, 32 * j, col, half, grp16, j16);
  }

  // ---- Y^T[p][t]: register r of y[f] holds p = 32 f + 8 (r / 4) + 4 half + r % 4.
  // Y leaves through the X tile's area (free once every wave is past its last
  // block of s): the wave writes its slice's 32 token rows (128 bytes, 16-byte
  // pieces XOR-swizzled by the row) and stores them whole, eight rows per
  // instruction; rows past the chunk end fall outside the buffer resource.
  __builtin_amdgcn_s_barrier();
  if (act) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *(uint2*)(s_x + tl * 128 + (((4 * f + jj) ^ (tl & 7)) << 4) + 8 * half) =
            make_uint2(pack_bf16x2(y[f][4 * jj], y[f][4 * jj + 1]), pack_bf16x2(y[f][4 * jj + 2], y[f][4 * jj + 3]));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    const int nv = clen - 32 * sl < 32 ? clen - 32 * sl : 32;
    const auto ry = buf_rsrc(wave_uniform(a.Y + ((row0 + s0 + 32 * sl) * a.H + h) * kP),
                             (uint32_t)((nv - 1) * a.H * kP + kP) * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3), pc = lane & 7;  // row within the slice
      const int rt = 32 * sl + r;                          // row within the chunk
      const uint4 v = *(const uint4*)(s_x + rt * 128 + ((pc ^ (rt & 7)) << 4));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_ssd_t, v), ry,
                                             (uint32_t)(r * a.H * kP + 8 * pc) * 2, 0, 0);
    }
  }
}

}  // namespace

size_t ssd_workspace_bytes(const Shape& s, bool bf16) {
  const size_t alpha = ((size_t)(s.b * s.H * s.M) * 4 + 255) / 256 * 256;
  return alpha + (size_t)(s.b * s.H * s.M * s.P * s.N) * (bf16 ? 2 : 4);
}

hipError_t launch_ssd_fwd(const Shape& s, bool bf16, bool mfma, const void* X, const void* B, const void* C,
                          const float* A, const float* H0, void* Y, void* dH, float* Hfin, void* ws,
                          hipStream_t st) {
  if (s.b * s.H * s.M == 0) return hipSuccess;
  hipError_t e = mfma ? launch_chunk_states_mfma(s, X, B, A, dH, st)
                      : launch_chunk_states_general(s, bf16, X, B, A, dH, st);
  if (e != hipSuccess) return e;
  float* alpha = (float*)ws;
  void* hin = (uint8_t*)ws + ((size_t)(s.b * s.H * s.M) * 4 + 255) / 256 * 256;
  chunk_decay_kernel<<<dim3((unsigned)(s.b * s.H * s.M)), dim3(64), 0, st>>>(s, A, alpha);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nPN = s.P * s.N;
  if (bf16 && nPN % 8 == 0) {
    const int64_t slices = (nPN / 8 + kThreads - 1) / kThreads;
    state_pass_kernel<bf16_t, 8><<<dim3((unsigned)(s.b * s.H * slices)), dim3(kThreads), 0, st>>>(
        s, slices, (const bf16_t*)dH, alpha, H0, (bf16_t*)hin, Hfin);
  } else if (bf16) {
    const int64_t slices = (nPN + kThreads - 1) / kThreads;
    state_pass_kernel<bf16_t, 1><<<dim3((unsigned)(s.b * s.H * slices)), dim3(kThreads), 0, st>>>(
        s, slices, (const bf16_t*)dH, alpha, H0, (bf16_t*)hin, Hfin);
  } else {
    const int64_t slices = (nPN + kThreads - 1) / kThreads;
    state_pass_kernel<float, 1><<<dim3((unsigned)(s.b * s.H * slices)), dim3(kThreads), 0, st>>>(
        s, slices, (const float*)dH, alpha, H0, (float*)hin, Hfin);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mfma && s.S % 32 == 0 && s.S <= kMaxS) {
    SsdArgs a;
    a.X = (const bf16_t*)X;
    a.B = (const bf16_t*)B;
    a.C = (const bf16_t*)C;
    a.A = A;
    a.Hin = (const bf16_t*)hin;
    a.Y = (bf16_t*)Y;
    a.L = s.L;
    a.H = (int)s.H;
    a.G = (int)s.G;
    a.hpg = (int)(s.H / s.G);
    a.S = (int)s.S;
    a.M = (int)s.M;
    if (a.hpg == 1)
      ssd_out_mfma_kernel<true><<<dim3((unsigned)(s.b * s.H * s.M)), dim3(kThreadsOut), 0, st>>>(a);
    else
      ssd_out_mfma_kernel<false><<<dim3((unsigned)(s.b * s.H * s.M)), dim3(kThreadsOut), 0, st>>>(a);
    return hipGetLastError();
  }
  const int64_t gph = (s.L + 3) / 4;
  if (bf16)
    ssd_out_general_kernel<bf16_t><<<dim3((unsigned)(s.b * s.H * gph)), dim3(kThreads), 0, st>>>(
        s, (const bf16_t*)X, (const bf16_t*)B, (const bf16_t*)C, A, (const bf16_t*)hin, (bf16_t*)Y, gph);
  else
    ssd_out_general_kernel<float><<<dim3((unsigned)(s.b * s.H * gph)), dim3(kThreads), 0, st>>>(
        s, (const float*)X, (const float*)B, (const float*)C, A, (const float*)hin, (float*)Y, gph);
  return hipGetLastError();
}

}  // namespace dart
