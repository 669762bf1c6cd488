// State-memory attention forward with the RMS-normalised score branch on
// gfx950 MFMA: bfloat16 inputs, N = 128, P = 64, float16 score memory.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §3 Eq. 8-11 with the
// normalised logits of App. B.1 Eq. 25-27:
//     l = RMSNorm(Q_t) . (r_j * (dH_j RMSNorm(E_t))) / sqrt(N).
// The chunk side of the normalisation comes precomputed per chunk as the
// score memory S_j[p][n] = w_e[p] dH_j[p][n] r_j[n] w_q[n] (float16), so
//     l = inv_rms(Q_t) inv_rms(E_t) . sum_p (Q_t S_j^T)[p] E_t[p] / sqrt(N)
// is the plain branch's bilinear form on S_j with two per-token factors.
//
// The kernel is the plain forward (one block = 128 tokens of one head, four
// waves of 32 tokens, chunk memories streamed through LDS and shared by the
// waves, W and V on the matrix core with one token per lane) with three
// changes:
//   * per chunk both dH_j (bf16, for V = C dH_j) and S_j (fp16, for
//     W = Q S_j) are staged: a 32 KB slot, two slots in an LDS ring (the
//     next chunk loads while the current one is used);
//   * W runs on v_mfma_f32_32x32x16_f16: the query enters as Q_t 2^k, with
//     2^k the power of two nearest above 1/rms(Q_t), which float16 holds
//     exactly (a bfloat16 value has 8 significant bits, float16 keeps 11, and
//     |Q_t 2^k| <= 2 sqrt(N)); the rest of the normalisation, inv_rms / 2^k,
//     joins the per-token logit scale.  V stays on the bfloat16 matrix core.
//     The float16 score memory is the only rounding the normalisation adds;
//   * the Q and C tiles go straight to registers (no LDS staging), which
//     frees the LDS for the wider slots; the Y tile has its own 16 KB area
//     (which first stages the E tile as whole rows) and the gate tile takes
//     the ring slot freed by the second-to-last chunk.
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kTile = 128;               // tokens per block
constexpr int kThreads = 256;            // 4 waves x 32 tokens
constexpr int kMemBytes = kP * kN * 2;   // one 16 KB memory (bf16 or fp16)
constexpr int kSlot = 2 * kMemBytes;     // dH_j then S_j
constexpr float kTau = 8.f;

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

struct FwdRmsArgs {
  const bf16_t* Q;
  const bf16_t* C;
  const bf16_t* E;
  const bf16_t* dH;
  const _Float16* dHs;
  const bf16_t* Y;
  const bf16_t* gate;
  bf16_t* out;
  float* R;
  float* lse;
  int64_t L;
  int H, G, hpg, S, M, gate_pc;
  int BH, BHp, n_tiles;
  float e_scale;  // log2(e) / sqrt(N)
  float eps;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_fwd_rms_mfma_kernel(FwdRmsArgs a) {
  // two 32 KB chunk slots and the 16 KB Y / out area: 80 KB, two blocks per CU
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[2 * kSlot + kTile * kP * 2];
  uint8_t* const s_y = s_lds + 2 * kSlot;

  const int blk = blockIdx.x;
  const TileItem item = head_major_tile(blk, a.n_tiles);
  const int bh = item.bh;
  if (bh >= a.BH) return;
  const int tile = item.tile;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int64_t t0 = (int64_t)tile * kTile;
  const int64_t t_last = (t0 + kTile < a.L ? t0 + kTile : a.L) - 1;
  const int n_hist = (int)(t_last / a.S);
  const int64_t t = t0 + wave * 32 + col;  // this lane's token
  const bool tok_ok = t < a.L;
  const int64_t tc = tok_ok ? t : a.L - 1;
  const int my_hist = tok_ok ? (int)(t / a.S) : 0;
  const int64_t row0 = (int64_t)b * a.L;

  // ---- streamed slots: s < n_hist is chunk s (dH_s and S_s into ring slot
  // s % 2), s == n_hist the per-channel gate tile (ring slot s % 2).  A chunk
  // load of wave w writes rows 16w .. 16w+15 of both memories (4 + 4 loads),
  // a token-tile load the wave's own 32 token rows (4 loads of 8 rows of
  // 128 B); the XOR swizzle is applied on the global side.
  const int64_t mem0 = (int64_t)bh * a.M * (kP * kN);
  const uint32_t mem_dma = (16 * wave + (lane >> 4)) * 256;
  const int last_r = (int)(a.L - 1 - t0 < kTile - 1 ? a.L - 1 - t0 : kTile - 1);
  const uint32_t tok_bytes = (uint32_t)(last_r * a.H * kP + kP) * 2;
  auto issue_tok = [&](const bf16_t* base, uint8_t* area) {
    const auto rs = buf_rsrc(base + ((row0 + t0) * a.H + h) * kP, tok_bytes);
    uint8_t* dst = area + wave * 32 * 128;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 32 * wave + 8 * k + (lane >> 3);
      const int rr = r < last_r ? r : last_r;
      buf_dma16(rs, (uint32_t)(rr * a.H * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2, dst + k * 8 * 128);
    }
  };
  auto issue = [&](int s) {
    uint8_t* slot = s_lds + (s & 1) * kSlot;
    if (s < n_hist) {
      const auto rd = buf_rsrc(a.dH + mem0 + (int64_t)s * (kP * kN), kMemBytes);
      const auto rsc = buf_rsrc(a.dHs + mem0 + (int64_t)s * (kP * kN), kMemBytes);
      uint8_t* dst = slot + wave * 16 * 256;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        const uint32_t off = mem_dma + i * 1024 + (((lane & 15) ^ (row & 15)) << 4);
        buf_dma16(rd, off, dst + i * 4 * 256);
        buf_dma16(rsc, off, dst + kMemBytes + i * 4 * 256);
      }
    } else if (s == n_hist && a.gate_pc) {
      issue_tok(a.gate, slot);
    }
  };

  issue(0);
  issue(1);
  // E rows of this wave staged whole in its quarter of the Y area (free
  // until the epilogue; the Y tile follows once E is in registers)
  {
    const auto rse = buf_rsrc(wave_uniform(a.E + ((row0 + t0) * a.G + g) * kP),
                              (uint32_t)(last_r * a.G * kP + kP) * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // rows past the sequence end re-read the last token (finite norms)
      const int r = 32 * wave + 8 * k + (lane >> 3);
      const int rr = r < last_r ? r : last_r;
      buf_dma16(rse, (uint32_t)(rr * a.G * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2,
                s_y + wave * 32 * 128 + k * 1024);
    }
  }

  // ---- token operands straight to registers.  Q and C as MFMA B operands:
  // lane holds token `col`, n = 16 ks + 8 half + 0..7; E in the accumulator
  // layout (register r of row block rb holds p = 32 rb + 8 (r / 4) + 4 half
  // + r % 4).
  f16x8_t qh[8];
  bf16x8_t cf[8];
  float ef[2][16];
  {
    const int64_t qrow = ((row0 + tc) * a.G + g) * kN + 8 * half;
    uint4 qv[8], cv[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qv[ks] = *(const uint4*)(a.Q + qrow + 16 * ks);
      cv[ks] = *(const uint4*)(a.C + qrow + 16 * ks);
    }
    uint2 ev[2][4];
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    {
      const int tr = 32 * wave + col;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          ev[rb][gq] = *(const uint2*)(s_y + tr * 128 + (((4 * rb + gq) ^ (tr & 7)) << 4) + 8 * half);
      // E is in registers before this wave's Y rows overwrite it
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      issue_tok(a.Y, s_y);
    }
    // RMSNorm of Q_t and E_t [App. B.1 Eq. 25]: this lane holds half of each row
    float ssq = 0.f, sse = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint32_t w4[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16lo(w4[k]), hi = bf16hi(w4[k]);
        ssq = fmaf(lo, lo, fmaf(hi, hi, ssq));
      }
      cf[ks] = __builtin_bit_cast(bf16x8_t, cv[ks]);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float e0 = bf16lo(ev[rb][gq].x), e1 = bf16hi(ev[rb][gq].x);
        const float e2 = bf16lo(ev[rb][gq].y), e3 = bf16hi(ev[rb][gq].y);
        sse = fmaf(e0, e0, fmaf(e1, e1, fmaf(e2, e2, fmaf(e3, e3, sse))));
      }
    const float inv_q = 1.f / sqrtf(halves_sum(ssq) * (1.f / kN) + a.eps);
    const float inv_e = 1.f / sqrtf(halves_sum(sse) * (1.f / kP) + a.eps);
    // 2^k >= inv_q > 2^(k-1): Q_t 2^k is exact in float16 (entries below
    // 2^-14 of its RMS, which add nothing visible to the logit, excepted)
    int k2;
    (void)frexpf(inv_q, &k2);
    const float p2 = ldexpf(1.f, k2);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint32_t w4[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
      f16x8_t v;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = (_Float16)(bf16lo(w4[k]) * p2);
        v[2 * k + 1] = (_Float16)(bf16hi(w4[k]) * p2);
      }
      qh[ks] = v;
    }
    const float es = a.e_scale * inv_e * (inv_q / p2);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        ef[rb][4 * gq + 0] = bf16lo(ev[rb][gq].x) * es;
        ef[rb][4 * gq + 1] = bf16hi(ev[rb][gq].x) * es;
        ef[rb][4 * gq + 2] = bf16lo(ev[rb][gq].y) * es;
        ef[rb][4 * gq + 3] = bf16hi(ev[rb][gq].y) * es;
      }
  }

  float o[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[0][r] = o[1][r] = 0.f;
  float m = -INFINITY, d = 0.f;

  // every load above but the Y tile has drained (the wait covered the slot
  // loads too); the barrier makes all waves' parts of slots 0 and 1 visible
  __builtin_amdgcn_s_barrier();

  for (int j = 0; j < n_hist; ++j) {
    // chunk j landed in every wave's part, every wave is done with chunk
    // j - 1: its slot takes slot j + 1 (the only load in flight, with the
    // Y tile until the first of these waits)
    if (j > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      issue(j + 1);
    }
    __builtin_amdgcn_s_setprio(1);
    f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
    const uint8_t* sm = s_lds + (j & 1) * kSlot;
    const uint8_t* ss = sm + kMemBytes;
    // operands one k-step ahead of their MFMAs (order pinned below)
    f16x8_t s0 = *(const f16x8_t*)(ss + mem_off(col, half));
    f16x8_t s1 = *(const f16x8_t*)(ss + mem_off(32 + col, half));
    bf16x8_t n0 = *(const bf16x8_t*)(sm + mem_off(col, half));
    bf16x8_t n1 = *(const bf16x8_t*)(sm + mem_off(32 + col, half));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const f16x8_t as0 = s0, as1 = s1;
      const bf16x8_t a0 = n0, a1 = n1;
      if (ks < 7) {
        s0 = *(const f16x8_t*)(ss + mem_off(col, 2 * ks + 2 + half));
        s1 = *(const f16x8_t*)(ss + mem_off(32 + col, 2 * ks + 2 + half));
      }
      w0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as0, qh[ks], w0, 0, 0, 0);
      w1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as1, qh[ks], w1, 0, 0, 0);
      if (ks < 7) {
        n0 = *(const bf16x8_t*)(sm + mem_off(col, 2 * ks + 2 + half));
        n1 = *(const bf16x8_t*)(sm + mem_off(32 + col, 2 * ks + 2 + half));
      }
      v0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, cf[ks], v0, 0, 0, 0);
      v1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, cf[ks], v1, 0, 0, 0);
      if (ks == 0) __builtin_amdgcn_s_setprio(2);
    }
    // burst order: [2 reads of S, step k+1][2 W MFMAs][2 reads of dH][2 V MFMAs]
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_s_setprio(0);

    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(w0[r], ef[0][r], part);
      part = fmaf(w1[r], ef[1][r], part);
    }
    const float l2 = halves_sum(part);

    const bool valid = j < my_hist;
    const float mn = (valid && l2 > m + kTau) ? l2 : m;
    if (__any(mn != m)) {
      const float alpha = (mn == m) ? 1.f : fast_exp2(m - mn);
      d *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][r] *= alpha;
        o[1][r] *= alpha;
      }
      m = mn;
    }
    const float pj = valid ? fast_exp2(l2 - m) : 0.f;
    d += pj;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o[0][r] = fmaf(pj, v0[r], o[0][r]);
      o[1][r] = fmaf(pj, v1[r], o[1][r]);
    }
  }

  // ---- epilogue: R = O / d, lse = m + log d, out = Y + g * R  [§3 Eq. 10-11].
  // Each wave reads only the Y / gate rows it loaded itself; `out` replaces
  // the wave's Y rows in place (every lane rewrites exactly the bytes it
  // read) and leaves as whole 128-byte rows.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  const float inv = d > 0.f ? 1.f / d : 0.f;
  const int tr = 32 * wave + col;
  const uint8_t* gbuf = s_lds + (n_hist & 1) * kSlot;
  const int64_t orow = (row0 + tc) * a.H + h;
  const float gs = a.gate_pc ? 0.f : bf16_to_f32(a.gate[orow]);
  float* rp = (a.R && tok_ok) ? a.R + orow * kP + 4 * half : nullptr;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t lo = tr * 128 + (((4 * rb + gq) ^ (tr & 7)) << 4) + 8 * half;
      const float r0 = o[rb][4 * gq + 0] * inv, r1 = o[rb][4 * gq + 1] * inv;
      const float r2 = o[rb][4 * gq + 2] * inv, r3 = o[rb][4 * gq + 3] * inv;
      const uint2 yv = *(const uint2*)(s_y + lo);
      float g0 = gs, g1 = gs, g2 = gs, g3 = gs;
      if (a.gate_pc) {
        const uint2 gv = *(const uint2*)(gbuf + lo);
        g0 = bf16lo(gv.x); g1 = bf16hi(gv.x); g2 = bf16lo(gv.y); g3 = bf16hi(gv.y);
      }
      uint2 ov;
      ov.x = pack_bf16x2(fmaf(g0, r0, bf16lo(yv.x)), fmaf(g1, r1, bf16hi(yv.x)));
      ov.y = pack_bf16x2(fmaf(g2, r2, bf16lo(yv.y)), fmaf(g3, r3, bf16hi(yv.y)));
      *(uint2*)(s_y + lo) = ov;
      if (rp) *(float4*)(rp + 32 * rb + 8 * gq) = make_float4(r0, r1, r2, r3);
    }
  if (a.lse && half == 0 && tok_ok)
    a.lse[(int64_t)bh * a.L + t] = d > 0.f ? (m + fast_log2(d)) * kLn2 : -INFINITY;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 32 * wave + 8 * k + (lane >> 3);
    const int f = lane & 7;
    if (t0 + r < a.L) {
      const uint4 v = *(const uint4*)(s_y + r * 128 + ((f ^ (r & 7)) << 4));
      *(uint4*)(a.out + ((row0 + t0 + r) * a.H + h) * kP + f * 8) = v;
    }
  }
}

}  // namespace

hipError_t launch_sma_fwd_rms_mfma(const Shape& s, float eps, const void* Q, const void* C,
                                   const void* E, const void* dH, const void* dHs, const void* Y,
                                   const void* gate, int gate_pc, void* out, float* R, float* lse,
                                   hipStream_t st) {
  FwdRmsArgs a;
  a.Q = (const bf16_t*)Q;
  a.C = (const bf16_t*)C;
  a.E = (const bf16_t*)E;
  a.dH = (const bf16_t*)dH;
  a.dHs = (const _Float16*)dHs;
  a.Y = (const bf16_t*)Y;
  a.gate = (const bf16_t*)gate;
  a.out = (bf16_t*)out;
  a.R = R;
  a.lse = lse;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.gate_pc = gate_pc;
  a.BH = (int)(s.b * s.H);
  a.BHp = (a.BH + 7) / 8 * 8;
  a.n_tiles = (int)((s.L + kTile - 1) / kTile);
  a.e_scale = kLog2e / sqrtf((float)kN);
  a.eps = eps;
  const int64_t blocks = (int64_t)a.BHp * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  sma_fwd_rms_mfma_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dart
