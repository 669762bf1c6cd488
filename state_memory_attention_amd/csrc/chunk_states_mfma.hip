// Chunk state memories on gfx950 MFMA: bfloat16 storage, N = 128, P = 64,
// float32 accumulation.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §3 Eq. 5 (= App. A
// Eq. 20):  dH_[c] = sum_{s in [c]} A_{s+1:e(c)} B_s^T X_s.
//
// One block per (b, h, chunk); the output dH_[c]^T (64 x 128) is the product
//     D = (diag(w) X_c)^T B_c        (P x S) . (S x N)
// on v_mfma_f32_32x32x16_bf16, wave w owning columns n = 32w..32w+31 and both
// 32-row halves of p.  The contraction runs over tokens, but X and B are
// stored token-major, so each 64-token block is transposed through LDS
// (token axis innermost, rows padded to 144 bytes to spread banks) while the
// decay weights are applied to X in float32 and rounded once to bf16.
//
// Decay weights w_s = prod_{k=s+1}^{e(c)} a_k are a suffix product: token
// blocks are visited from the end of the chunk backward, wave 0 forms the
// in-block suffix product with lane shuffles, and `carry` holds the product
// of all decays after the block.  Underflow to zero is the correct value.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kSB = 64;          // tokens per LDS block
constexpr int kPitch = 144;      // bytes per transposed row (64 bf16 + 16 pad)
constexpr int kThreads = 256;

struct CsArgs {
  const bf16_t* X;
  const bf16_t* B;
  const float* A;
  bf16_t* dH;
  int64_t L;
  int H, G, hpg, S, M;
};

__global__ __launch_bounds__(kThreads) void chunk_states_mfma_kernel(CsArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_xt[kP * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_bt[kN * kPitch];
  __shared__ float s_w[kSB];

  const int c = blockIdx.x % a.M;
  const int bh = blockIdx.x / a.M;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;

  const int64_t s0 = (int64_t)c * a.S;
  const int64_t s1 = (s0 + a.S < a.L) ? s0 + a.S : a.L;
  const int nblk = (int)((s1 - s0 + kSB - 1) / kSB);

  f32x16_t acc0 = {}, acc1 = {};
  float carry = 1.f;  // wave 0: product of a_k over tokens after the current block

  // staging roles: 16 token-quads x 16 n-octets of B (all threads), 16 x 8
  // p-octets of X (threads 0..127)
  const int sq = tid & 15, oct = tid >> 4;

  for (int ib = nblk - 1; ib >= 0; --ib) {
    const int64_t sb = s0 + (int64_t)ib * kSB;
    const int cnt = (int)((s1 - sb) < kSB ? (s1 - sb) : kSB);
    if (wave == 0) {
      float v = lane < cnt ? a.A[((int64_t)b * a.L + sb + lane) * a.H + h] : 1.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_down(v, off);
        if (lane + off < 64) v *= u;
      }
      // v = prod_{j >= lane} a_j within the block; w_lane = carry * v_{lane+1}
      float nxt = __shfl_down(v, 1);
      if (lane == 63) nxt = 1.f;
      s_w[lane] = carry * nxt;
      carry *= __shfl(v, 0);
    }
    __syncthreads();  // s_w ready; previous block's MFMA reads of s_xt/s_bt done

    {  // B: 4 tokens x 8 n  ->  8 rows n of 4 tokens each
      uint4 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * sq + i;
        r[i] = k < cnt ? *(const uint4*)(a.B + (((int64_t)b * a.L + sb + k) * a.G + g) * kN + 8 * oct)
                       : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* u = (const uint32_t*)r;  // u[4 i + e/2] holds n = 8 oct + e of token i
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        const uint32_t t0 = (u[0 * 4 + e / 2] >> sh) & 0xffffu, t1 = (u[1 * 4 + e / 2] >> sh) & 0xffffu;
        const uint32_t t2 = (u[2 * 4 + e / 2] >> sh) & 0xffffu, t3 = (u[3 * 4 + e / 2] >> sh) & 0xffffu;
        *(uint2*)(s_bt + (8 * oct + e) * kPitch + 8 * sq) = make_uint2(t0 | (t1 << 16), t2 | (t3 << 16));
      }
    }
    if (tid < 128) {  // X scaled by w: 4 tokens x 8 p -> 8 rows p
      float xs[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * sq + i;
        uint4 v = make_uint4(0, 0, 0, 0);
        float w = 0.f;
        if (k < cnt) {
          v = *(const uint4*)(a.X + (((int64_t)b * a.L + sb + k) * a.H + h) * kP + 8 * oct);
          w = s_w[k];
        }
        xs[i][0] = bf16lo(v.x) * w; xs[i][1] = bf16hi(v.x) * w;
        xs[i][2] = bf16lo(v.y) * w; xs[i][3] = bf16hi(v.y) * w;
        xs[i][4] = bf16lo(v.z) * w; xs[i][5] = bf16hi(v.z) * w;
        xs[i][6] = bf16lo(v.w) * w; xs[i][7] = bf16hi(v.w) * w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *(uint2*)(s_xt + (8 * oct + e) * kPitch + 8 * sq) =
            make_uint2(pack_bf16x2(xs[0][e], xs[1][e]), pack_bf16x2(xs[2][e], xs[3][e]));
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < kSB / 16; ++ks) {
      const int kofs = (16 * ks + 8 * half) * 2;
      const bf16x8_t a0 = *(const bf16x8_t*)(s_xt + col * kPitch + kofs);
      const bf16x8_t a1 = *(const bf16x8_t*)(s_xt + (32 + col) * kPitch + kofs);
      const bf16x8_t bb = *(const bf16x8_t*)(s_bt + (32 * wave + col) * kPitch + kofs);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bb, acc1, 0, 0, 0);
    }
  }

  // D[p][n]: register r of row block rb is p = 32 rb + 8 (r/4) + 4 half + r%4
  bf16_t* outp = a.dH + ((int64_t)bh * a.M + c) * (kP * kN) + 32 * wave + col;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int p = 8 * (r >> 2) + 4 * half + (r & 3);
    outp[p * kN] = (bf16_t)f32_to_bf16(acc0[r]);
    outp[(32 + p) * kN] = (bf16_t)f32_to_bf16(acc1[r]);
  }
}

}  // namespace

hipError_t launch_chunk_states_mfma(const Shape& s, const void* X, const void* B, const float* A,
                                    void* dH, hipStream_t st) {
  CsArgs a;
  a.X = (const bf16_t*)X;
  a.B = (const bf16_t*)B;
  a.A = A;
  a.dH = (bf16_t*)dH;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  const int64_t blocks = s.b * s.H * s.M;
  if (blocks == 0) return hipSuccess;
  chunk_states_mfma_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dart
