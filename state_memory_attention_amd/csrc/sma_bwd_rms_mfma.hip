// Backward of the RMS-normalised score branch on gfx950 MFMA: bfloat16
// inputs, N = 128, P = 64, the float16 score memory of the forward.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), App. B.1 Eq. 25-27
// differentiated, with the recomputation of §4 "Efficient Training" and
// App. C Eq. 33-35.  With zq = RMSNorm(Q_t) and ze = RMSNorm(E_t) before their
// weights (factors rho_q, rho_e), the score memory dHs_c = diag(w_q r_c) dH_c
// diag(w_e) (stored [p][n]) and dls = dl / sqrt(N):
//     l = zq dHs_c ze / sqrt(N),  V = C_t dH_c,  dl = p (dR . V - D)
//     d zq = sum_c dls dHs_c ze          (the plain dQ on the score memory)
//     d ze = sum_c dls dHs_c^T zq        (the plain dE on the score memory)
//     dC   = sum_c p dH_c dR             (plain)
//     dT_c = sum_t dls zq ze^T = sum_t (dls rho_q rho_e) Q_t^T E_t
//     d dH_c = sum_t p C_t^T dR_t  +  r_c * dS_c - (r_c^3 / P) dH_c * sum_p (dS_c * dH_c),
//              dS_c = diag(w_q) dT_c diag(w_e)
//     dw_q = sum_c r_c * sum_p (w_e dT_c dH_c),  dw_e = sum_c sum_n (w_q r_c dH_c dT_c)
//     dQ_t = rho_q d zq - rho_q^3 Q_t (Q_t . d zq) / N     (E alike, over P)
// so the plain backward's passes serve with operands swapped:
//   A   (this file) the normalised forward's loop (dH and dHs per chunk, W on
//       the float16 matrix core from Q_t 2^k, V on the bfloat16 one) with
//       pass A's epilogue: p, dl, d ze, dgate, dR; the pd rows hold p and
//       dls rho_q rho_e, and rho_q, rho_e go to the workspace;
//   BC  twice, each memory transposed first: the Q side on the score memory
//       (E scaled by rho_e per token), the C side on dH;
//   D   unchanged: its readout term into d_dH, its score term (weights
//       dls rho_q rho_e on E, Q rows as they are) into dT;
//   then the chain through r_c and the weight-gradient terms per chunk
//   memory, the sums over a group's heads, the RMSNorm backward of Q_t and
//   E_t in place, and fixed-order column sums for dw_q, dw_e.
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
constexpr int kSlot = 2 * kMemBytes;     // dH_j then dHs_j

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct BwdRmsAArgs {
  const bf16_t* Q;
  const bf16_t* C;
  const bf16_t* E;
  const bf16_t* dH;
  const _Float16* dHs;
  const bf16_t* gate;
  const bf16_t* dout;
  const float* R;
  const float* lse;
  float* dE;        // [b][L][dE_heads][P]: d ze
  float* pd;        // [b][H][M][2][L]: p, then dl / sqrt(N) rho_q rho_e
  bf16_t* dR;       // [b][L][H][P]
  float* dgate;     // nullable
  float* rho;       // [b][L][G][2]: rho_q, rho_e
  int64_t L;
  int H, G, hpg, S, M, gate_pc, dE_heads;
  int fuse_norm;    // one head per group: dE leaves through the RMSNorm backward
  int BH, BHp, n_tiles;
  float e_scale;    // log2(e) / sqrt(N)
  float inv_sqrt_n;
  float eps;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_bwd_rms_a_kernel(BwdRmsAArgs a) {
  // two 32 KB chunk slots and a 16 KB token area (E rows, then dR rows):
  // 80 KB, two blocks per CU
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

  // chunk s < n_hist: dH_s and dHs_s into ring slot s % 2, wave w rows
  // 16w .. 16w+15 of both (4 + 4 loads), XOR swizzle on the global side
  const int64_t mem0 = (int64_t)bh * a.M * (kP * kN);
  const uint32_t mem_dma = (16 * wave + (lane >> 4)) * 256;
  const int last_r = (int)(a.L - 1 - t0 < kTile - 1 ? a.L - 1 - t0 : kTile - 1);
  auto issue = [&](int s) {
    if (s >= n_hist) return;
    uint8_t* dst = s_lds + (s & 1) * kSlot + wave * 16 * 256;
    const auto rd = buf_rsrc(a.dH + mem0 + (int64_t)s * (kP * kN), kMemBytes);
    const auto rsc = buf_rsrc(a.dHs + mem0 + (int64_t)s * (kP * kN), kMemBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const uint32_t off = mem_dma + i * 1024 + (((lane & 15) ^ (row & 15)) << 4);
      buf_dma16(rd, off, dst + i * 4 * 256);
      buf_dma16(rsc, off, dst + kMemBytes + i * 4 * 256);
    }
  };

  issue(0);
  issue(1);
  // E rows of this wave staged whole in its quarter of the token area
  // (rows past the sequence end re-read the last token: finite norms)
  {
    const auto rse = buf_rsrc(wave_uniform(a.E + ((row0 + t0) * a.G + g) * kP),
                              (uint32_t)(last_r * a.G * kP + kP) * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 32 * wave + 8 * k + (lane >> 3);
      const int rr = r < last_r ? r : last_r;
      buf_dma16(rse, (uint32_t)(rr * a.G * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2,
                s_y + wave * 32 * 128 + k * 1024);
    }
  }

  // Q and C straight to registers (lane: token `col`, n = 16 ks + 8 half + 0..7)
  const int64_t qrow = ((row0 + tc) * a.G + g) * kN + 8 * half;
  uint4 qv[8], cv[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qv[ks] = *(const uint4*)(a.Q + qrow + 16 * ks);
    cv[ks] = *(const uint4*)(a.C + qrow + 16 * ks);
  }
  // dout, gate and R in the row layout (lane l of step k: channels
  // 8 (l % 8) .. +7 of the wave's row 8 k + l / 8; rows past the end read zeros)
  const int64_t obase = ((row0 + t0) * a.H + h) * kP;
  const uint32_t ob16 = (uint32_t)(last_r * a.H * kP + kP) * 2;
  const auto rs_do = buf_rsrc(wave_uniform(a.dout + obase), ob16);
  const auto rs_g = buf_rsrc(wave_uniform(a.gate + (a.gate_pc ? obase : (int64_t)0)), a.gate_pc ? ob16 : 0u);
  const auto rs_r = buf_rsrc(wave_uniform(a.R + obase), 2 * ob16);
  const auto rs_gs = buf_rsrc(wave_uniform(a.gate + (row0 + t0) * a.H + h),
                              a.gate_pc ? 0u : (uint32_t)(last_r * a.H + 1) * 2);
  const int f = lane & 7;
  u32x4_t dv[4], gv[4], rv[4][2];
  uint32_t gsr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 8 * k + (lane >> 3);
    const uint32_t ro = (uint32_t)((32 * wave + rr) * a.H * kP + 8 * f);
    dv[k] = __builtin_amdgcn_raw_buffer_load_b128(rs_do, ro * 2, 0, 0);
    gv[k] = __builtin_amdgcn_raw_buffer_load_b128(rs_g, ro * 2, 0, 0);
    rv[k][0] = __builtin_amdgcn_raw_buffer_load_b128(rs_r, ro * 4, 0, 0);
    rv[k][1] = __builtin_amdgcn_raw_buffer_load_b128(rs_r, ro * 4 + 16, 0, 0);
    gsr[k] = __builtin_amdgcn_raw_buffer_load_b16(rs_gs, (uint32_t)((32 * wave + rr) * a.H) * 2, 0, 0);
  }
  const float lse2 = a.lse[(int64_t)bh * a.L + tc] * kLog2e;
  __builtin_amdgcn_s_waitcnt(kWaitAll);
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(dv[k]), "+v"(gv[k]), "+v"(rv[k][0]), "+v"(rv[k][1]), "+v"(gsr[k]));

  // E from the token area in the accumulator layout (register r of row
  // block rb: p = 32 rb + 8 (r / 4) + 4 half + r % 4)
  const int tr = 32 * wave + col;
  uint2 ev[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      ev[rb][gq] = *(const uint2*)(s_y + tr * 128 + (((4 * rb + gq) ^ (tr & 7)) << 4) + 8 * half);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);

  // dR = g * dout rounded to bfloat16 once (D and every dR . V use the
  // rounded values), D = dR . R and dgate in the row layout; dR to HBM and
  // into the wave's rows of the token area (E is in registers)
  uint8_t* const s_dr = s_y + wave * 32 * 128;
  const auto rs_dr = buf_rsrc(wave_uniform(a.dR + obase), ob16);
  const int64_t gbase = a.gate_pc ? obase : (row0 + t0) * a.H + h;
  const auto rs_dg = buf_rsrc(wave_uniform(a.dgate ? a.dgate + gbase : a.dgate),
                              a.dgate ? (a.gate_pc ? 2 * ob16 : (uint32_t)(last_r * a.H + 1) * 4) : 0u);
  float dsum[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 8 * k + (lane >> 3);
    const uint32_t ro = (uint32_t)((32 * wave + rr) * a.H * kP + 8 * f);
    const uint32_t dw[4] = {dv[k].x, dv[k].y, dv[k].z, dv[k].w};
    const uint32_t gw[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
    const float rf[8] = {__uint_as_float(rv[k][0].x), __uint_as_float(rv[k][0].y),
                         __uint_as_float(rv[k][0].z), __uint_as_float(rv[k][0].w),
                         __uint_as_float(rv[k][1].x), __uint_as_float(rv[k][1].y),
                         __uint_as_float(rv[k][1].z), __uint_as_float(rv[k][1].w)};
    u32x4_t pk, dgl, dgh;
    float part = 0.f, gpart = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float d0 = bf16lo(dw[q]), d1 = bf16hi(dw[q]);
      const float gs = bf16_to_f32(gsr[k]);
      const float g0 = a.gate_pc ? bf16lo(gw[q]) : gs, g1 = a.gate_pc ? bf16hi(gw[q]) : gs;
      const uint32_t w = pack_bf16x2(g0 * d0, g1 * d1);
      pk[q] = w;
      part = fmaf(bf16lo(w), rf[2 * q], fmaf(bf16hi(w), rf[2 * q + 1], part));
      gpart += d0 * rf[2 * q] + d1 * rf[2 * q + 1];
      const float x0 = d0 * rf[2 * q], x1 = d1 * rf[2 * q + 1];  // dgate = dout * R
      if (q < 2) {
        dgl[2 * q] = __float_as_uint(x0);
        dgl[2 * q + 1] = __float_as_uint(x1);
      } else {
        dgh[2 * q - 4] = __float_as_uint(x0);
        dgh[2 * q - 3] = __float_as_uint(x1);
      }
    }
    __builtin_amdgcn_raw_buffer_store_b128(pk, rs_dr, ro * 2, 0, 0);
    *(u32x4_t*)(s_dr + rr * 128 + ((f ^ (rr & 7)) << 4)) = pk;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      part += __shfl_xor(part, m);
      gpart += __shfl_xor(gpart, m);
    }
    dsum[k] = part;  // D of row 8 k + lane / 8, in all 8 lanes of the row
    if (a.gate_pc) {
      __builtin_amdgcn_raw_buffer_store_b128(dgl, rs_dg, ro * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(dgh, rs_dg, ro * 4 + 16, 0, 0);
    } else {
      const uint32_t so = f == 0 ? (uint32_t)((32 * wave + rr) * a.H) * 4 : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gpart), rs_dg, so, 0, 0);
    }
  }
  // D of token `col` (row col = 8 k + col / 8 ... held by lane 8 (col % 8) of step col / 8)
  float D;
  {
    const int src = 8 * (col & 7);
    const float d0 = __shfl(dsum[0], src), d1 = __shfl(dsum[1], src);
    const float d2 = __shfl(dsum[2], src), d3 = __shfl(dsum[3], src);
    const int k = col >> 3;
    D = k == 0 ? d0 : (k == 1 ? d1 : (k == 2 ? d2 : d3));
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  uint2 drv[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      drv[rb][gq] = *(const uint2*)(s_dr + col * 128 + (((4 * rb + gq) ^ (col & 7)) << 4) + 8 * half);

  // RMSNorm factors [App. B.1 Eq. 25]; the query enters W as Q_t 2^k, exact
  // in float16, and E carries the rest of the scale, as in the forward
  float ssq = 0.f, sse = 0.f;
  bf16x8_t cf[8];
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
  int k2;
  (void)frexpf(inv_q, &k2);
  const float p2 = ldexpf(1.f, k2);
  f16x8_t qh[8];
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
  float ef[2][16];
  {
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
  // one head of the group stores the token's factors
  if (h % a.hpg == 0 && half == 0 && tok_ok)
    *(float2*)(a.rho + 2 * ((row0 + t) * a.G + g)) = make_float2(inv_q, inv_e);
  const float dl_rho = a.inv_sqrt_n * inv_q * inv_e;

  float de[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) de[0][r] = de[1][r] = 0.f;

  // (p, dl) rows of this wave's 32 tokens: stores by every lane, those of the
  // second half-wave and of tokens past the end outside the resource
  const int64_t pd_base = (int64_t)bh * a.M * 2 * a.L + t0 + 32 * wave;
  const int64_t nv = a.L - (t0 + 32 * wave);
  const uint32_t pd_bytes = (uint32_t)(nv < 32 ? (nv > 0 ? nv : 0) : 32) * 4;
  const uint32_t pd_voff = half ? 0x80000000u : (uint32_t)col * 4;

  // every load above has drained (slots 0 and 1 included); the barrier makes
  // all waves' parts of both slots visible
  __builtin_amdgcn_s_barrier();

  for (int j = 0; j < n_hist; ++j) {
    // chunk j landed in every wave's part and every wave is done with chunk
    // j - 1, whose slot takes chunk j + 1.  In flight here: chunk j's loads
    // (issued during chunk j - 1), then chunk j - 1's two (p, dl) stores;
    // vector-memory operations complete in order, so vmcnt(2) covers the loads.
    if (j > 0) {
      __builtin_amdgcn_s_waitcnt(0x0f72);  // vmcnt(2)
      __builtin_amdgcn_s_barrier();
      issue(j + 1);
    }
    __builtin_amdgcn_s_setprio(1);
    f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
    const uint8_t* sm = s_lds + (j & 1) * kSlot;
    const uint8_t* ss = sm + kMemBytes;
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
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_s_setprio(0);

    // logit (base 2, the forward's arithmetic) and dR . V
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      asm volatile("" : "+v"(drv[rb][0].x), "+v"(drv[rb][0].y), "+v"(drv[rb][1].x), "+v"(drv[rb][1].y),
                   "+v"(drv[rb][2].x), "+v"(drv[rb][2].y), "+v"(drv[rb][3].x), "+v"(drv[rb][3].y));
    float pl = 0.f, pv = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pl = fmaf(w0[r], ef[0][r], pl);
      pl = fmaf(w1[r], ef[1][r], pl);
    }
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      pv = fmaf(v0[4 * gq + 0], bf16lo(drv[0][gq].x), pv);
      pv = fmaf(v0[4 * gq + 1], bf16hi(drv[0][gq].x), pv);
      pv = fmaf(v0[4 * gq + 2], bf16lo(drv[0][gq].y), pv);
      pv = fmaf(v0[4 * gq + 3], bf16hi(drv[0][gq].y), pv);
      pv = fmaf(v1[4 * gq + 0], bf16lo(drv[1][gq].x), pv);
      pv = fmaf(v1[4 * gq + 1], bf16hi(drv[1][gq].x), pv);
      pv = fmaf(v1[4 * gq + 2], bf16lo(drv[1][gq].y), pv);
      pv = fmaf(v1[4 * gq + 3], bf16hi(drv[1][gq].y), pv);
    }
    const float l2 = halves_sum(pl);
    const float dp = halves_sum(pv);
    const bool valid = j < my_hist;
    const float pj = valid ? fast_exp2(l2 - lse2) : 0.f;
    const float dl = pj * (dp - D);
    const float dls = dl * a.inv_sqrt_n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      de[0][r] = fmaf(dls, w0[r], de[0][r]);
      de[1][r] = fmaf(dls, w1[r], de[1][r]);
    }
    {
      const int64_t rowj = pd_base + (int64_t)j * 2 * a.L;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pj), buf_rsrc(a.pd + rowj, pd_bytes), pd_voff, 0,
                                            kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dl * dl_rho), buf_rsrc(a.pd + rowj + a.L, pd_bytes),
                                            pd_voff, 0, kNonTemporal);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // d ze = (rho_q / 2^k) sum_c dls W_c (W_c from Q_t 2^k)
  {
    const float sc = inv_q / p2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      de[0][r] *= sc;
      de[1][r] *= sc;
    }
  }
  if (a.fuse_norm) {
    // RMSNorm backward of E_t [App. B.1 Eq. 25]: dE = rho dz - rho^3 E (E . dz) / P
    const bf16_t* er = a.E + ((row0 + tc) * a.G + g) * kP + 4 * half;
    uint2 ev2[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) ev2[rb][gq] = *(const uint2*)(er + 32 * rb + 8 * gq);
    float part = 0.f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        part = fmaf(bf16lo(ev2[rb][gq].x), de[rb][4 * gq], part);
        part = fmaf(bf16hi(ev2[rb][gq].x), de[rb][4 * gq + 1], part);
        part = fmaf(bf16lo(ev2[rb][gq].y), de[rb][4 * gq + 2], part);
        part = fmaf(bf16hi(ev2[rb][gq].y), de[rb][4 * gq + 3], part);
      }
    const float c3 = inv_e * inv_e * inv_e * halves_sum(part) * (1.f / kP);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        de[rb][4 * gq] = fmaf(inv_e, de[rb][4 * gq], -c3 * bf16lo(ev2[rb][gq].x));
        de[rb][4 * gq + 1] = fmaf(inv_e, de[rb][4 * gq + 1], -c3 * bf16hi(ev2[rb][gq].x));
        de[rb][4 * gq + 2] = fmaf(inv_e, de[rb][4 * gq + 2], -c3 * bf16lo(ev2[rb][gq].y));
        de[rb][4 * gq + 3] = fmaf(inv_e, de[rb][4 * gq + 3], -c3 * bf16hi(ev2[rb][gq].y));
      }
  }
  if (tok_ok) {
    float* dp = a.dE + (((row0 + t) * a.dE_heads) + (a.dE_heads == a.H ? h : g)) * kP + 4 * half;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *(float4*)(dp + 32 * rb + 8 * gq) =
            make_float4(de[rb][4 * gq + 0], de[rb][4 * gq + 1], de[rb][4 * gq + 2], de[rb][4 * gq + 3]);
  }
}

// Through S_c = diag(r_c) dH_c, one block per chunk memory: with
// dS = w_q[n] w_e[p] dT[p][n] and u_n = sum_p w_e[p] dT[p][n] dH[p][n],
//   d_dH[p][n] += r_n dS[p][n] - (r_n^3 / P) dH[p][n] w_q[n] u_n,
//   wpq[mem][n] = r_n u_n,   wpe[mem][p] = sum_n w_q[n] r_n dH[p][n] dT[p][n].
// Four waves; wave w owns rows p = 16 w .. 16 w + 15 and lane l the columns
// n = 2 l, 2 l + 1 (4- and 8-byte loads, a wave covers whole rows), keeping
// its dH and dT values in registers between the two passes.  The sums over p
// (r_n, u_n) add the four waves' parts in wave order through LDS; the sum
// over n (wpe) is one wave sum per row.
__global__ __launch_bounds__(256) void rms_chain_kernel(float eps, const bf16_t* __restrict__ dH,
                                                        const float* __restrict__ dT, const float* __restrict__ wq,
                                                        const float* __restrict__ we, float* __restrict__ ddh,
                                                        float* __restrict__ wpq, float* __restrict__ wpe) {
  constexpr int kRows = kP / 4;
  __shared__ float s_ss[4][kN], s_u[4][kN];
  const int64_t mem = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n0 = 2 * lane, p0 = kRows * wave;
  const int64_t base = mem * (int64_t)(kP * kN) + (int64_t)p0 * kN + n0;
  uint32_t xv[kRows];
  float2 tv[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    xv[i] = *(const uint32_t*)(dH + base + i * kN);
    tv[i] = *(const float2*)(dT + base + i * kN);
  }
  float ss0 = 0.f, ss1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const float x0 = bf16lo(xv[i]), x1 = bf16hi(xv[i]);
    const float wp = we ? we[p0 + i] : 1.f;
    ss0 = fmaf(x0, x0, ss0);
    ss1 = fmaf(x1, x1, ss1);
    u0 = fmaf(wp * tv[i].x, x0, u0);
    u1 = fmaf(wp * tv[i].y, x1, u1);
  }
  s_ss[wave][n0] = ss0;
  s_ss[wave][n0 + 1] = ss1;
  s_u[wave][n0] = u0;
  s_u[wave][n0 + 1] = u1;
  __syncthreads();
  ss0 = ss1 = u0 = u1 = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    ss0 += s_ss[w][n0];
    ss1 += s_ss[w][n0 + 1];
    u0 += s_u[w][n0];
    u1 += s_u[w][n0 + 1];
  }
  const float r0 = 1.f / sqrtf(ss0 / (float)kP + eps), r1 = 1.f / sqrtf(ss1 / (float)kP + eps);  // [Eq. 26]
  const float wq0 = wq ? wq[n0] : 1.f, wq1 = wq ? wq[n0 + 1] : 1.f;
  const float k30 = r0 * r0 * r0 / (float)kP * wq0 * u0, k31 = r1 * r1 * r1 / (float)kP * wq1 * u1;
  if (wpq && wave == 0) *(float2*)(wpq + mem * kN + n0) = make_float2(r0 * u0, r1 * u1);
  const float rw0 = r0 * wq0, rw1 = r1 * wq1;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const float x0 = bf16lo(xv[i]), x1 = bf16hi(xv[i]);
    const float wp = we ? we[p0 + i] : 1.f;
    float2* o = (float2*)(ddh + base + i * kN);
    float2 d = *o;
    d.x = fmaf(rw0 * wp, tv[i].x, fmaf(-k30, x0, d.x));
    d.y = fmaf(rw1 * wp, tv[i].y, fmaf(-k31, x1, d.y));
    *o = d;
    if (wpe) {
      const float sv = wave_sum(fmaf(rw0 * x0, tv[i].x, rw1 * x1 * tv[i].y));
      if (lane == 0) wpe[mem * kP + p0 + i] = sv;
    }
  }
}

// RMSNorm backward in place, one wave per row (token, group) of K <= 256:
// dz <- rho dz - rho^3 x (x . dz) / K.
__global__ __launch_bounds__(256) void rms_norm_rows_kernel(int64_t rows, int K, const bf16_t* __restrict__ x,
                                                            const float* __restrict__ rho, int side,
                                                            float* __restrict__ dz) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float r = rho[2 * row + side];
  float xv[4], gv[4], part = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * k;
    xv[k] = gv[k] = 0.f;
    if (i < K) {
      xv[k] = bf16_to_f32(x[row * K + i]);
      gv[k] = dz[row * K + i];
      part = fmaf(xv[k], gv[k], part);
    }
  }
  const float c3 = r * r * r * wave_sum(part) / (float)K;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * k;
    if (i < K) dz[row * K + i] = fmaf(r, gv[k], -c3 * xv[k]);
  }
}

// Workspace: the plain MFMA backward's parts (pd, dR, per-head partials),
// then rho [b][L][G][2], dT [b][H][M][P][N], the weight-gradient terms
// [b][H][M][N] and [b][H][M][P], and the column-sum partials, each from a
// 256-byte boundary.
size_t r256(size_t n) { return (n + 255) / 256 * 256; }
struct RmsMfmaWs {
  size_t memTs, rho, dT, wpq, wpe, part, total;
};
// The plain backward's workspace (with dH transposed at its end), then the
// score memory transposed, the RMSNorm factors, dT, the weight-gradient rows
// and the column-sum partials.
RmsMfmaWs rms_mfma_layout(const Shape& s) {
  RmsMfmaWs w;
  size_t o = r256(sma_bwd_mfma_workspace_bytes(s));
  w.memTs = o; o += r256((size_t)(s.b * s.H * s.M * s.P * s.N) * 2);
  w.rho = o;  o += r256((size_t)(2 * s.b * s.L * s.G) * 4);
  w.dT = o;   o += r256((size_t)(s.b * s.H * s.M * s.P * s.N) * 4);
  w.wpq = o;  o += r256((size_t)(s.b * s.H * s.M * s.N) * 4);
  w.wpe = o;  o += r256((size_t)(s.b * s.H * s.M * s.P) * 4);
  w.part = o; o += r256((size_t)(col_sum_split(s.b * s.H * s.M) * (s.N + s.P)) * 4);
  w.total = o;
  return w;
}

}  // namespace

size_t sma_bwd_rms_mfma_workspace_bytes(const Shape& s) { return rms_mfma_layout(s).total; }

hipError_t launch_sma_bwd_rms_mfma(const Shape& s, float eps, const void* Q, const void* C, const void* E,
                                   const void* dH, const void* dHs, const float* wq, const float* we,
                                   const void* gate, int gate_pc, const float* R, const float* lse,
                                   const void* dout, float* dQ, float* dC, float* dE, float* ddH, float* dgate,
                                   float* dwq, float* dwe, void* ws, hipStream_t st) {
  // the plain backward's parts of the workspace: (p, dl) rows, dR, per-head partials
  uint8_t* w = (uint8_t*)ws;
  const size_t pd_b = r256((size_t)(2 * s.b * s.H * s.M * s.L) * 4);
  const size_t dr_b = r256((size_t)(s.b * s.L * s.H * s.P) * 2);
  float* pd = (float*)w;
  void* dR = w + pd_b;
  const bool grouped = s.H != s.G;
  float* hq = grouped ? (float*)(w + pd_b + dr_b) : dQ;
  float* hc = grouped ? hq + s.b * s.L * s.H * s.N : dC;
  float* he = grouped ? hc + s.b * s.L * s.H * s.N : dE;
  const int heads = grouped ? (int)s.H : (int)s.G;
  const RmsMfmaWs lay = rms_mfma_layout(s);
  float* rho = (float*)(w + lay.rho);
  float* dT = (float*)(w + lay.dT);
  float* wpq = dwq ? (float*)(w + lay.wpq) : nullptr;
  float* wpe = dwe ? (float*)(w + lay.wpe) : nullptr;
  float* part = (float*)(w + lay.part);

  BwdRmsAArgs a;
  a.Q = (const bf16_t*)Q;
  a.C = (const bf16_t*)C;
  a.E = (const bf16_t*)E;
  a.dH = (const bf16_t*)dH;
  a.dHs = (const _Float16*)dHs;
  a.gate = (const bf16_t*)gate;
  a.dout = (const bf16_t*)dout;
  a.R = R;
  a.lse = lse;
  a.dE = he;
  a.pd = pd;
  a.dR = (bf16_t*)dR;
  a.dgate = dgate;
  a.rho = rho;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.gate_pc = gate_pc;
  a.dE_heads = heads;
  a.fuse_norm = grouped ? 0 : 1;
  a.BH = (int)(s.b * s.H);
  a.BHp = (a.BH + 7) / 8 * 8;
  a.n_tiles = (int)((s.L + kTile - 1) / kTile);
  a.e_scale = kLog2e / sqrtf((float)kN);
  a.inv_sqrt_n = 1.f / sqrtf((float)kN);
  a.eps = eps;
  const int64_t blocks = (int64_t)a.BHp * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  sma_bwd_rms_a_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void* memT = w + sma_bwd_memt_offset(s);
  void* memTs = w + lay.memTs;
  const int64_t n_mem = s.b * s.H * s.M;
  if ((e = launch_mem_transpose(dHs, memTs, n_mem, st)) != hipSuccess) return e;
  if ((e = launch_mem_transpose(dH, memT, n_mem, st)) != hipSuccess) return e;
  if ((e = launch_sma_bwd_bc_mfma(s, kBcScoreQ, E, dR, memTs, pd, rho, grouped ? nullptr : Q, hq, nullptr, heads,
                                  st)) != hipSuccess)
    return e;
  if ((e = launch_sma_bwd_bc_mfma(s, kBcC, E, dR, memT, pd, nullptr, nullptr, nullptr, hc, heads, st)) != hipSuccess)
    return e;
  if ((e = launch_sma_bwd_d_mfma(s, dR, E, C, Q, pd, ddH, dT, st)) != hipSuccess) return e;
  rms_chain_kernel<<<dim3((unsigned)n_mem), dim3(256), 0, st>>>(eps, (const bf16_t*)dH, dT, wq, we, ddH, wpq, wpe);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rows = s.b * s.L, hpg = s.H / s.G;
  if (grouped) {
    if ((e = launch_group_sum(hq, dQ, rows, s.G, hpg, s.N, st)) != hipSuccess) return e;
    if ((e = launch_group_sum(hc, dC, rows, s.G, hpg, s.N, st)) != hipSuccess) return e;
    if ((e = launch_group_sum(he, dE, rows, s.G, hpg, s.P, st)) != hipSuccess) return e;
  }
  if (grouped) {  // otherwise the two epilogues applied the RMSNorm backward
    const int64_t tg = rows * s.G;
    const unsigned nb = (unsigned)((tg + 3) / 4);
    rms_norm_rows_kernel<<<dim3(nb), dim3(256), 0, st>>>(tg, kN, (const bf16_t*)Q, rho, 0, dQ);
    rms_norm_rows_kernel<<<dim3(nb), dim3(256), 0, st>>>(tg, kP, (const bf16_t*)E, rho, 1, dE);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dwq && (e = launch_col_sum(wpq, part, dwq, n_mem, kN, st)) != hipSuccess) return e;
  if (dwe && (e = launch_col_sum(wpe, part, dwe, n_mem, kP, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace dart
