// State-memory attention backward on gfx950 MFMA: bfloat16 inputs, N = 128,
// P = 64, float32 arithmetic and gradients.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032).  Training keeps only R
// and lse from the forward and recomputes every logit; the chunk weights come
// back as p = exp(l - lse) [§4 "Efficient Training"; App. C "Recomputation",
// Eq. 33-35].  The chain rule through §3 Eq. 8-11 gives, with dR = g * dout,
// D_t = dR_t . R_t, W = Q_t dH_c, V = C_t dH_c and dl = p (dR_t . V - D_t):
//     dE_t = sum_c dl W / sqrt(N)
//     dQ_t = sum_c dl dH_c E_t / sqrt(N),      dC_t = sum_c p dH_c dR_t
//     d_dH_c = sum_{t: chunk(t) > c} p C_t^T dR_t + dl Q_t^T E_t / sqrt(N).
//
// Three passes, each sized to the register file (two waves per SIMD, three
// for pass BC with one product):
//   A  token tiles x chunks: recompute W and V on the matrix core exactly as
//      the forward does, then p, dl (stored per (chunk, token)), dE, dgate
//      and dR (stored in bfloat16 for pass D);
//   BC token tiles x chunks: dQ^T += dH_c (E * dl/sqrt(N))^T and
//      dC^T += dH_c (dR * p)^T, the chunk memory as the A operand, read from
//      a copy transposed to N x P by a small kernel;
//   D  chunks x later token tiles: the two token contractions of d_dH, the
//      per-token weights scaling one operand (the chunk-state kernel's form).
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kTile = 128;       // tokens per block in the token-major passes
constexpr int kThreads = 256;
constexpr int kMemBytes = kP * kN * 2;
constexpr int kRing = 4;         // LDS buffers for chunk memories (3 in flight)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Eight 8-byte LDS reads and one 4-byte read, with their wait in the same
// asm block: written as plain loads, the compiler cannot tell their area from
// the one a direct-to-LDS load in flight is filling, and places a
// vector-memory wait before them that also drains the stores issued since.
__device__ __forceinline__ void ld_lds_8x8_4(u32x2_t (&o)[8], float& d, const uint32_t (&ad)[8], uint32_t a_d) {
  asm volatile(
      "ds_read_b64 %0, %9\n\t"
      "ds_read_b64 %1, %10\n\t"
      "ds_read_b64 %2, %11\n\t"
      "ds_read_b64 %3, %12\n\t"
      "ds_read_b64 %4, %13\n\t"
      "ds_read_b64 %5, %14\n\t"
      "ds_read_b64 %6, %15\n\t"
      "ds_read_b64 %7, %16\n\t"
      "ds_read_b32 %8, %17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7]), "=&v"(d)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(a_d)
      : "memory");
}

// ---------------------------------------------------------------------------
// Pass A
// ---------------------------------------------------------------------------

struct BwdAArgs {
  const bf16_t* Q;
  const bf16_t* C;
  const bf16_t* E;
  const bf16_t* dH;
  const bf16_t* gate;
  const bf16_t* dout;
  const float* R;
  const float* lse;
  float* dE;        // [b][L][dE_heads][P]
  float* pd;        // [b][H][M][2][L]: row of p then row of dl / sqrt(N) per chunk
  bf16_t* dR;       // [b][L][H][P]
  float* dgate;     // nullable
  int64_t L;
  int H, G, hpg, S, M, gate_pc, dE_heads;
  int BH, BHp, n_tiles;
  float e_scale;    // log2(e) / sqrt(N)
  float inv_sqrt_n;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_bwd_a_kernel(BwdAArgs a) {
  // The forward's LDS plan: a 64 KB ring of chunk memories (first used to
  // stage the Q and C tiles) and a 16 KB area that takes chunk 0.
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kRing * kMemBytes + kMemBytes];
  uint8_t* const s_mem = s_lds;
  uint8_t* const s_e = s_lds + kRing * kMemBytes;

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

  // chunk slots: chunk 0 in the 16 KB area, chunk s >= 1 in ring buffer
  // (s - 1) % 4; every wave loads rows 16w .. 16w+15 of each (4 loads).
  const uint8_t* mem_head = (const uint8_t*)(a.dH + (int64_t)bh * a.M * (kP * kN));
  const uint32_t mem_dma = (16 * wave + (lane >> 4)) * 256;
  auto slot_buf = [&](int s) -> uint8_t* { return s == 0 ? s_e : s_mem + ((s - 1) % kRing) * kMemBytes; };
  // A slot past the last chunk is a zero-length stand-in (it reads nothing
  // and fills a buffer no later chunk uses), so that every slot costs every
  // wave 4 loads and the loop's waits are fixed counts.
  auto issue_mem = [&](int s) {
    const bool real = s < n_hist;
    const auto rs = buf_rsrc(mem_head + (int64_t)(real ? s : 0) * kMemBytes, real ? kMemBytes : 0u);
    uint8_t* dst = slot_buf(s) + wave * 16 * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      buf_dma16(rs, mem_dma + i * 1024 + (((lane & 15) ^ (row & 15)) << 4), dst + i * 4 * 256);
    }
  };

  // ---- token operands (see the forward kernel): Q and C as MFMA B
  // operands; E and dR kept as bfloat16 pairs in the accumulator layout
  // (register r of row block rb holds p = 32 rb + 8 (r / 4) + 4 half + r % 4).
  // dR = g * dout is rounded to bfloat16 once, and D = dR . R and every
  // dR . V use the rounded values: the gradients are then exactly those of a
  // dout perturbed by at most one bfloat16 rounding, with no cancellation
  // error in dp - D.
  //
  // Every token row is read and written whole: Q and C staged through the
  // ring (wave w: rows 32w .. 32w+31 in bytes [8 KB w, 8 KB w + 8 KB) of the
  // Q and C halves), E staged in the wave's quarter of the chunk-0 area, and
  // dout, gate and R loaded in a row layout (lane l of step k: channels
  // 8 (l % 8) .. +7 of the wave's row 8 k + l / 8), where dR, D and dgate are
  // formed; dR and D reach the accumulator layout through the wave's Q area
  // once Q is in registers.  Chunk 0 then loads into the chunk-0 area, each
  // wave's part over exactly the bytes its E rows occupied.
  bf16x8_t qf[8], cf[8];
  uint2 drv[2][4];
  float ef[2][16];
  float D, lse2;
  {
    const int last_r = (int)(a.L - 1 - t0 < kTile - 1 ? a.L - 1 - t0 : kTile - 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 32 * wave + 4 * k + (lane >> 4);
      const int64_t tok = (t0 + r < a.L) ? t0 + r : a.L - 1;
      const int64_t off = ((row0 + tok) * a.G + g) * kN + (((lane & 15) ^ (r & 15)) << 3);
      dma16(a.Q + off, s_mem + (32 * wave + 4 * k) * 256);
      dma16(a.C + off, s_mem + 32768 + (32 * wave + 4 * k) * 256);
    }
    {
      // E rows 32 wave + 8 k + lane / 8 (rows past the end read zeros), pieces
      // XOR-swizzled by the row within its 128 bytes
      const auto rse = buf_rsrc(wave_uniform(a.E + ((row0 + t0) * a.G + g) * kP),
                                (uint32_t)(last_r * a.G * kP + kP) * 2);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 32 * wave + 8 * k + (lane >> 3);
        buf_dma16(rse, (uint32_t)(r * a.G * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2,
                  s_e + wave * 4096 + k * 1024);
      }
    }
    // per-token rows [b][L][H][P] of this tile (rows past the end: zeros in,
    // dropped out)
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
    lse2 = a.lse[(int64_t)bh * a.L + tc] * kLog2e;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // pinned here, where they have landed: left alone the compiler may use a
    // value early and wait for every load in flight to do so
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      asm volatile("" : "+v"(dv[k]), "+v"(gv[k]), "+v"(rv[k][0]), "+v"(rv[k][1]), "+v"(gsr[k]));
    }
    {
      const int r = 32 * wave + col;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint32_t o = r * 256 + (((2 * ks + half) ^ (r & 15)) << 4);
        qf[ks] = *(const bf16x8_t*)(s_mem + o);
        cf[ks] = *(const bf16x8_t*)(s_mem + 32768 + o);
      }
      // E in float32, scaled by log2(e) / sqrt(N) as in the forward, so that
      // the logit below is formed exactly as the forward formed it
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint2 v = *(const uint2*)(s_e + r * 128 + (((4 * rb + gq) ^ (r & 7)) << 4) + 8 * half);
          ef[rb][4 * gq + 0] = bf16lo(v.x) * a.e_scale;
          ef[rb][4 * gq + 1] = bf16hi(v.x) * a.e_scale;
          ef[rb][4 * gq + 2] = bf16lo(v.y) * a.e_scale;
          ef[rb][4 * gq + 3] = bf16hi(v.y) * a.e_scale;
        }
    }
    // Q, C and E are in registers: the wave's Q area takes dR and D, and its
    // E area chunk 0 (a stand-in if there is no history)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    issue_mem(0);
    uint8_t* const s_dr = s_mem + wave * 8192;
    const auto rs_dr = buf_rsrc(wave_uniform(a.dR + obase), ob16);
    // dgate: [b][L][H][P] per channel, [b][L][H] for a scalar gate
    const int64_t gbase = a.gate_pc ? obase : (row0 + t0) * a.H + h;
    const auto rs_dg = buf_rsrc(wave_uniform(a.dgate ? a.dgate + gbase : a.dgate),
                                a.dgate ? (a.gate_pc ? 2 * ob16 : (uint32_t)(last_r * a.H + 1) * 4) : 0u);
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
        // dgate = dout * R per channel  [§3 Eq. 11]
        const float x0 = d0 * rf[2 * q], x1 = d1 * rf[2 * q + 1];
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
      // D and the scalar gate's gradient: sums over the 8 lanes of the row
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
        part += __shfl_xor(part, m);
        gpart += __shfl_xor(gpart, m);
      }
      if (f == 0) *(float*)(s_dr + 4096 + rr * 4) = part;
      if (a.gate_pc) {
        __builtin_amdgcn_raw_buffer_store_b128(dgl, rs_dg, ro * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(dgh, rs_dg, ro * 4 + 16, 0, 0);
      } else {
        // one lane per row writes the row's sum; the others fall outside
        const uint32_t so = f == 0 ? (uint32_t)((32 * wave + rr) * a.H) * 4 : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gpart), rs_dg, so, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(0u, rs_dg, 0x80000000u, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    {
      uint32_t ad[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ad[i] = lds_addr(s_dr + col * 128 + ((i ^ (col & 7)) << 4) + 8 * half);
      u32x2_t o[8];
      ld_lds_8x8_4(o, D, ad, lds_addr(s_dr + 4096 + col * 4));
#pragma unroll
      for (int i = 0; i < 8; ++i) drv[i >> 2][i & 3] = make_uint2(o[i].x, o[i].y);
    }
  }

  float de[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) de[0][r] = de[1][r] = 0.f;

  // Chunk 0 has landed in every wave's part (the 12 stores issued after it
  // may still be in flight) and no wave reads its Q area any more: slots 1
  // and 2 go to ring buffers 0 and 1.
  __builtin_amdgcn_s_waitcnt(0x007c);  // vmcnt(12) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  if (n_hist > 0) {
    issue_mem(1);
    issue_mem(2);
  }

  // (p, dl) rows of this wave's 32 tokens: a uniform base per chunk plus the
  // lane.  Both rows are written by buffer stores of every lane (those of
  // the second half-wave, and tokens past the end, fall outside the
  // resource and are dropped), so that each chunk costs exactly 2 stores.
  const int64_t pd_base = (int64_t)bh * a.M * 2 * a.L + t0 + 32 * wave;
  const int64_t nv = a.L - (t0 + 32 * wave);
  const uint32_t pd_bytes = (uint32_t)(nv < 32 ? (nv > 0 ? nv : 0) : 32) * 4;
  const uint32_t pd_voff = half ? 0x80000000u : (uint32_t)col * 4;
  for (int j = 0; j < n_hist; ++j) {
    // Chunk j landed everywhere, chunk j-1 free (see the forward kernel).
    // In flight after slot j's loads: slots j+1 and j+2 (4 loads each, real
    // or stand-in) and the (p, dl) stores of the chunks since slot j was
    // issued (2 each: chunks j-3 .. j-1, or 0 .. j-1 for the slots issued
    // before the loop).
    if (j == 1)
      __builtin_amdgcn_s_waitcnt(0x007a);  // vmcnt(10) lgkmcnt(0)
    else if (j == 2)
      __builtin_amdgcn_s_waitcnt(0x007c);  // vmcnt(12) lgkmcnt(0)
    else if (j > 2)
      __builtin_amdgcn_s_waitcnt(0x007e);  // vmcnt(14) lgkmcnt(0)
    if (j > 0) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(1);
    f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
    const uint8_t* sm = slot_buf(j);
    // dH_j^T operands one k-step ahead of their MFMAs (the forward's schedule)
    bf16x8_t n0 = *(const bf16x8_t*)(sm + mem_off(col, half));
    bf16x8_t n1 = *(const bf16x8_t*)(sm + mem_off(32 + col, half));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t a0 = n0, a1 = n1;
      if (ks < 7) {
        n0 = *(const bf16x8_t*)(sm + mem_off(col, 2 * ks + 2 + half));
        n1 = *(const bf16x8_t*)(sm + mem_off(32 + col, 2 * ks + 2 + half));
      }
      w0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], w0, 0, 0, 0);
      w1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], w1, 0, 0, 0);
      v0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, cf[ks], v0, 0, 0, 0);
      v1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, cf[ks], v1, 0, 0, 0);
      if (ks == 1) issue_mem(j + kRing - 1);
      if (ks == 0) __builtin_amdgcn_s_setprio(2);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);              // MFMA
    }
    __builtin_amdgcn_s_setprio(0);

    // logit (base 2, the forward's arithmetic) and dR . V, each over this
    // half-wave's 32 p then both.  The bfloat16 pairs of dR are unpacked
    // here, every iteration: the empty asm keeps the compiler from hoisting
    // 32 unpacked floats out of the loop.
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
      // streamed out, read back by later passes only: non-temporal
      const int64_t rowj = pd_base + (int64_t)j * 2 * a.L;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pj), buf_rsrc(a.pd + rowj, pd_bytes), pd_voff, 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dls), buf_rsrc(a.pd + rowj + a.L, pd_bytes), pd_voff, 0,
                                            kNonTemporal);
    }
  }
  // the stand-in slots past the last chunk land before the block ends
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

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

}  // namespace

hipError_t launch_sma_bwd_a_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                                 const void* dH, const void* gate, int gate_pc, const void* dout,
                                 const float* R, const float* lse, float* dE, int dE_heads,
                                 float* pd, void* dR, float* dgate, hipStream_t st) {
  BwdAArgs a;
  a.Q = (const bf16_t*)Q;
  a.C = (const bf16_t*)C;
  a.E = (const bf16_t*)E;
  a.dH = (const bf16_t*)dH;
  a.gate = (const bf16_t*)gate;
  a.dout = (const bf16_t*)dout;
  a.R = R;
  a.lse = lse;
  a.dE = dE;
  a.pd = pd;
  a.dR = (bf16_t*)dR;
  a.dgate = dgate;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.gate_pc = gate_pc;
  a.dE_heads = dE_heads;
  a.BH = (int)(s.b * s.H);
  a.BHp = (a.BH + 7) / 8 * 8;
  a.n_tiles = (int)((s.L + kTile - 1) / kTile);
  a.e_scale = kLog2e / sqrtf((float)kN);
  a.inv_sqrt_n = 1.f / sqrtf((float)kN);
  const int64_t blocks = (int64_t)a.BHp * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  sma_bwd_a_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pass BC: dQ^T += dH_c (E * dl / sqrt(N))^T,  dC^T += dH_c (dR * p)^T
// ---------------------------------------------------------------------------
namespace {

constexpr int kPdBytes = 4 * 2 * 32 * 4;          // (p, dl) of 4 waves x 32 tokens
constexpr int kSlotBC = kMemBytes + kPdBytes;     // one chunk memory + its weights

struct BwdBCArgs {
  const bf16_t* E;
  const bf16_t* dR;    // [b][L][H][P], from pass A
  const void* memT;    // chunk memories transposed, [b][H][M][N][P]: dH (bf16), or the
                       // float16 score memory (Q side only)
  const float* pd;     // [b][H][M][2][L], from pass A (p, dl / sqrt(N))
  const float* rho;    // [b][L][G][2] (Q side on the score memory): RMSNorm factors of Q_t, E_t
  const bf16_t* Qn;    // score-memory mode with one head per group: Q, and dQ is written
                       // through the RMSNorm backward (else NULL: the gradient of RMSNorm(Q_t))
  float* dQ;           // [b][L][out_heads][N]
  float* dC;
  int64_t L;
  int H, G, hpg, S, M, out_heads;
  int BH, BHp, n_tiles;
  float inv_sqrt_n;
};

// Byte offset of 16-byte piece `piece` (0..7, p = 8 piece .. +7) of row n of a
// staged transposed memory: 128-byte rows, pieces XOR-swizzled by (n >> 1) & 7,
// so that the operand reads below (16 lanes at a time on 16 consecutive rows,
// or 8 at a time) touch every bank once.
__device__ __forceinline__ uint32_t memt_off(int n, int piece) {
  return (uint32_t)(n * 128 + ((piece ^ ((n >> 1) & 7)) << 4));
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// 8 bf16 scaled by s in float32 and rounded to float16.
__device__ __forceinline__ f16x8_t scale8h(bf16x8_t x, float s) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  f16x8_t r;
  r[0] = (_Float16)(bf16lo(u.x) * s);
  r[1] = (_Float16)(bf16hi(u.x) * s);
  r[2] = (_Float16)(bf16lo(u.y) * s);
  r[3] = (_Float16)(bf16hi(u.y) * s);
  r[4] = (_Float16)(bf16lo(u.z) * s);
  r[5] = (_Float16)(bf16hi(u.z) * s);
  r[6] = (_Float16)(bf16lo(u.w) * s);
  r[7] = (_Float16)(bf16hi(u.w) * s);
  return r;
}

// 8 bf16 scaled by s in float32 and rounded back.
__device__ __forceinline__ bf16x8_t scale8(bf16x8_t x, float s) {
  const uint4 u = __builtin_bit_cast(uint4, x);
  uint4 r;
  r.x = pack_bf16x2(bf16lo(u.x) * s, bf16hi(u.x) * s);
  r.y = pack_bf16x2(bf16lo(u.y) * s, bf16hi(u.y) * s);
  r.z = pack_bf16x2(bf16lo(u.z) * s, bf16hi(u.z) * s);
  r.w = pack_bf16x2(bf16lo(u.w) * s, bf16hi(u.w) * s);
  return __builtin_bit_cast(bf16x8_t, r);
}

// kMode: kBcBoth (dQ and dC from dH), kBcScoreQ (dQ only, from the float16
// score memory of the normalised branch, whose Q-side gradient
// sum_c dHs_c (E_t rho_e,t dl_tc / sqrt(N)) takes the E operand scaled by the
// token's RMSNorm factor: the pd row then holds dl / sqrt(N) rho_q rho_e and is
// divided by rho_q here), kBcC (dC only, from dH).
//
// The memories arrive transposed (rows n, p contiguous), so the MFMA A
// operand (rows n, k = p) is one plain 16-byte LDS read per lane, issued one
// k-step ahead of the MFMAs that use it.  Both gradients (two accumulator sets)
// keep two waves per SIMD and a 4-deep ring; one gradient needs fewer than 168
// registers, and a 3-deep ring (51 KB) fits three blocks per CU.
template <int kMode>
constexpr int bc_ring() { return kMode == kBcBoth ? 4 : 3; }

template <int kMode>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kMode == kBcBoth ? 2 : 3, kMode == kBcBoth ? 2 : 3)))
void sma_bwd_bc_kernel(BwdBCArgs a) {
  constexpr bool kDoQ = kMode != kBcC, kDoC = kMode != kBcScoreQ;
  constexpr int kR = bc_ring<kMode>();
  // One LDS object: with a single object the compiler adds no wait of its own
  // for the direct-to-LDS loads in flight before the ring's plain reads.
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kR * kSlotBC];

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
  const int64_t t = t0 + wave * 32 + col;
  const bool tok_ok = t < a.L;
  const int64_t tc = tok_ok ? t : a.L - 1;
  const int64_t row0 = (int64_t)b * a.L;

  // Slot s = chunk s in ring buffer s % kR: the transposed memory (rows
  // n = 32w .. 32w+31 loaded by wave w, 4 loads of 8 rows; one load writes
  // 1 KB contiguously, so the swizzle is applied on the global side: the lane
  // that fills physical piece f of row n fetches logical piece
  // f ^ ((n >> 1) & 7)) and the (p, dl) pair of the wave's 32 tokens (one
  // 4-byte-per-lane load: lanes 0-31 p, lanes 32-63 dl).  Five loads per wave
  // per slot.
  const uint8_t* mem_head = (const uint8_t*)a.memT + (int64_t)bh * a.M * kMemBytes;
  const uint32_t pd_lane = (uint32_t)((half ? a.L : 0) + t0 + 32 * wave + col) * 4;
  auto issue = [&](int s) {
    uint8_t* dst = s_ring + (s % kR) * kSlotBC;
    const auto rs = buf_rsrc(mem_head + (int64_t)s * kMemBytes, kMemBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wave + 8 * i + (lane >> 3);
      buf_dma16(rs, (uint32_t)(row * 128 + (((lane & 7) ^ ((row >> 1) & 7)) << 4)), dst + wave * 4096 + i * 1024);
    }
    const auto rp = buf_rsrc(a.pd + ((int64_t)bh * a.M + s) * 2 * a.L, (uint32_t)(2 * a.L * 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rp, (__attribute__((address_space(3))) void*)(dst + kMemBytes + wave * 256), 4, pd_lane, 0, 0, 0);
  };

  // B operands: lane holds token `col`, p = 16 ks + 8 half + 0..7.  The E
  // and dR rows of the wave's 32 tokens are staged whole (128-byte rows,
  // 16-byte pieces XOR-swizzled by the row) in the wave's part of ring
  // buffer 2 (E, or dR when only dC is computed) and of buffer 3 (dR when
  // both are) while slots 0 and 1 load.  A wave's part of a slot covers
  // exactly the bytes of its staged rows, so a buffer takes its slot once
  // the wave's own reads of it are done: with both gradients slot 2 is issued
  // right after them and slot 3 in the loop; with one (3-deep ring) slot 2 is
  // issued in the loop, after its first barrier.
  bf16x8_t eop[4], rop[4];
  // score-memory mode: 1 / rho_q of this lane's token (the pd row's dl
  // carries rho_q rho_e; the Q-side operand needs rho_e only)
  float rq = 1.f, irq = 1.f;
  if (kMode == kBcScoreQ) {
    rq = a.rho[2 * ((row0 + tc) * a.G + g)];
    irq = 1.f / rq;
  }
  {
    if (0 < n_hist) issue(0);
    if (1 < n_hist) issue(1);
    const int last_r = (int)(a.L - 1 - t0 < kTile - 1 ? a.L - 1 - t0 : kTile - 1);
    uint8_t* const s_se = s_ring + 2 * kSlotBC + wave * 4096;
    uint8_t* const s_sr = s_ring + (kDoQ ? 3 : 2) * kSlotBC + wave * 4096;
    const auto rse = buf_rsrc(wave_uniform(a.E + ((row0 + t0) * a.G + g) * kP), (uint32_t)(last_r * a.G * kP + kP) * 2);
    const auto rsr = buf_rsrc(wave_uniform(a.dR + ((row0 + t0) * a.H + h) * kP), (uint32_t)(last_r * a.H * kP + kP) * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 32 * wave + 8 * k + (lane >> 3);
      const uint32_t sw = (uint32_t)(((lane & 7) ^ (r & 7)) << 3);
      if (kDoQ) buf_dma16(rse, (uint32_t)(r * a.G * kP + sw) * 2, s_se + k * 1024);
      if (kDoC) buf_dma16(rsr, (uint32_t)(r * a.H * kP + sw) * 2, s_sr + k * 1024);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t o = col * 128 + (((2 * ks + half) ^ (col & 7)) << 4);
      if (kDoQ) eop[ks] = *(const bf16x8_t*)(s_se + o);
      if (kDoC) rop[ks] = *(const bf16x8_t*)(s_sr + o);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (kR == 4 && 2 < n_hist) issue(2);
  }

  // A operand (rows n, k = p): lane reads row n = 32 rb + col, logical piece
  // 2 ks + half; the swizzle term depends on col only, so one per-lane offset
  // per k-step and the row block as an immediate.
  uint32_t aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = memt_off(col, 2 * ks + half);

  f32x16_t dq[4], dc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) dq[rb] = dc[rb] = f32x16_t{};

  for (int j = 0; j < n_hist; ++j) {
    // slot j landed (its 5 loads) in every wave's part; slot j-1 free.  Slots
    // j+1 .. j+kR-2 that exist may stay in flight.
    asm volatile("" ::: "memory");
    if (kR == 4 && n_hist - 1 - j >= 2)
      __builtin_amdgcn_s_waitcnt(0x0f7a);      // vmcnt(10)
    else if (n_hist - 1 - j >= 1)
      __builtin_amdgcn_s_waitcnt(0x0f75);      // vmcnt(5)
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (j + kR - 1 < n_hist) issue(j + kR - 1);

    const uint8_t* slot = s_ring + (j % kR) * kSlotBC;
    const float* wpd = (const float*)(slot + kMemBytes + wave * 256);
    const float ps = wpd[col], dls = wpd[32 + col];
    // The burst runs at raised priority, and a wave whose burst is under way
    // outranks one about to start its own (as in the forward), so the waves
    // sharing a SIMD take the matrix core in turns.
    __builtin_amdgcn_s_setprio(1);
    bf16x8_t nx[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) nx[rb] = *(const bf16x8_t*)(slot + aoff[0] + rb * 4096);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t av[4], be, br;
      f16x8_t beh;
      if (kMode == kBcScoreQ) beh = scale8h(eop[ks], dls * irq);
      if (kMode == kBcBoth) be = scale8(eop[ks], dls);
      if (kDoC) br = scale8(rop[ks], ps);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) av[rb] = nx[rb];
      if (ks < 3) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) nx[rb] = *(const bf16x8_t*)(slot + aoff[ks + 1] + rb * 4096);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (kMode == kBcScoreQ) {
          dq[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, av[rb]), beh, dq[rb], 0, 0, 0);
        } else {
          if (kDoQ) dq[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[rb], be, dq[rb], 0, 0, 0);
          if (kDoC) dc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[rb], br, dc[rb], 0, 0, 0);
        }
      }
      if (ks == 0) __builtin_amdgcn_s_setprio(2);
    }
    // burst order: [4 LDS reads for step k+1][the MFMAs of step k], k = 0..3
    // (left alone, the scheduler sinks each read to just before its use)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, (kDoQ && kDoC) ? 8 : 4, 0);       // MFMA
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // dQ^T, dC^T: lane column = token, register r of row block rb is
  // n = 32 rb + 8 (r / 4) + 4 half + r % 4
  if (kMode == kBcScoreQ && a.Qn) {
    // RMSNorm backward of Q_t [App. B.1 Eq. 25]: dQ = rho dz - rho^3 Q (Q . dz) / N,
    // the dot product over this half-wave's 64 n and then both halves
    const bf16_t* qr = a.Qn + ((row0 + tc) * a.G + g) * kN + 4 * half;
    uint2 qv[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) qv[rb][q] = *(const uint2*)(qr + 32 * rb + 8 * q);
    float part = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        part = fmaf(bf16lo(qv[rb][q].x), dq[rb][4 * q], part);
        part = fmaf(bf16hi(qv[rb][q].x), dq[rb][4 * q + 1], part);
        part = fmaf(bf16lo(qv[rb][q].y), dq[rb][4 * q + 2], part);
        part = fmaf(bf16hi(qv[rb][q].y), dq[rb][4 * q + 3], part);
      }
    const float c3 = rq * rq * rq * halves_sum(part) * (1.f / kN);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dq[rb][4 * q] = fmaf(rq, dq[rb][4 * q], -c3 * bf16lo(qv[rb][q].x));
        dq[rb][4 * q + 1] = fmaf(rq, dq[rb][4 * q + 1], -c3 * bf16hi(qv[rb][q].x));
        dq[rb][4 * q + 2] = fmaf(rq, dq[rb][4 * q + 2], -c3 * bf16lo(qv[rb][q].y));
        dq[rb][4 * q + 3] = fmaf(rq, dq[rb][4 * q + 3], -c3 * bf16hi(qv[rb][q].y));
      }
  }
  if (tok_ok) {
    const int64_t orow = ((row0 + t) * a.out_heads + (a.out_heads == a.H ? h : g)) * kN + 4 * half;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * rb + 8 * q;
        if (kDoQ)
          *(float4*)(a.dQ + orow + n) = make_float4(dq[rb][4 * q], dq[rb][4 * q + 1], dq[rb][4 * q + 2], dq[rb][4 * q + 3]);
        if (kDoC)
          *(float4*)(a.dC + orow + n) = make_float4(dc[rb][4 * q], dc[rb][4 * q + 1], dc[rb][4 * q + 2], dc[rb][4 * q + 3]);
      }
  }
}

}  // namespace

hipError_t launch_sma_bwd_bc_mfma(const Shape& s, int mode, const void* E, const void* dR, const void* memT,
                                  const float* pd, const float* rho, const void* Q_norm, float* dQ, float* dC,
                                  int out_heads, hipStream_t st) {
  BwdBCArgs a;
  a.E = (const bf16_t*)E;
  a.dR = (const bf16_t*)dR;
  a.memT = memT;
  a.pd = pd;
  a.rho = rho;
  a.Qn = (const bf16_t*)Q_norm;
  a.dQ = dQ;
  a.dC = dC;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.out_heads = out_heads;
  a.BH = (int)(s.b * s.H);
  a.BHp = (a.BH + 7) / 8 * 8;
  a.n_tiles = (int)((s.L + kTile - 1) / kTile);
  a.inv_sqrt_n = 1.f / sqrtf((float)kN);
  const int64_t blocks = (int64_t)a.BHp * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  if (mode == kBcScoreQ)
    sma_bwd_bc_kernel<kBcScoreQ><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  else if (mode == kBcC)
    sma_bwd_bc_kernel<kBcC><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  else
    sma_bwd_bc_kernel<kBcBoth><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Pass D: d_dH_c^T[p][n] = sum_{t >= (c+1)S} p_tc dR_t[p] C_t[n] + dl_tc/sqrt(N) E_t[p] Q_t[n]
// ---------------------------------------------------------------------------
namespace {

constexpr int kSB = 64;                      // tokens per sub-block
constexpr int kChunksD = 4;                  // chunks per block (one per wave's weight row)
constexpr int kStagesD = 3;
constexpr int kATile = kSB * kP * 2;         // dR or E: 64 rows of 128 B
constexpr int kBTile = kSB * kN * 2;         // C or Q: 64 rows of 256 B
constexpr int kWBytes = kChunksD * kSB * 4;  // weights of the block's chunks
constexpr int kStageD = kATile + kBTile + kWBytes;

struct BwdDArgs {
  const bf16_t* dR;   // [b][L][H][P]
  const bf16_t* E;    // [b][L][G][P]
  const bf16_t* C;    // [b][L][G][N]
  const bf16_t* Q;
  const float* pd;    // [b][H][M][2][L]: p, dl / sqrt(N)
  float* ddH;         // [b][H][M][P][N]: the readout term (term 0)
  float* ddH1;        // where the score term (term 1) goes: ddH, or a buffer of its own
  int64_t L;
  int H, G, hpg, S, M, n_groups, BH, BHp;
  float inv_sqrt_n;
};

__device__ __forceinline__ int swz_x(int row) { return (row & 3) << 1; }
__device__ __forceinline__ int swz_b(int row) { return (row & 3) << 2; }

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

// Ten transposing reads plus one 4-byte read (this lane's weight), returned
// together like ld_tr6: the compiler would otherwise drain the loads in
// flight before reading the weights of the staged slot.  k-step KS of a
// sub-block reads 16 KS token rows further on: its addresses are those of
// k-step 0 plus immediate offsets (rows of 128 B for ad[0..1], 256 B for
// ad[2..9], 4 B per weight).
template <int KS>
__device__ __forceinline__ void ld_tr10_w1(uint64_t (&o)[10], uint32_t& w, const uint32_t (&ad)[10], uint32_t wad) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %11 offset:%22\n\t"
      "ds_read_b64_tr_b16 %1, %12 offset:%22\n\t"
      "ds_read_b64_tr_b16 %2, %13 offset:%23\n\t"
      "ds_read_b64_tr_b16 %3, %14 offset:%23\n\t"
      "ds_read_b64_tr_b16 %4, %15 offset:%23\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:%23\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:%23\n\t"
      "ds_read_b64_tr_b16 %7, %18 offset:%23\n\t"
      "ds_read_b64_tr_b16 %8, %19 offset:%23\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:%23\n\t"
      "ds_read_b32 %10, %21 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(w)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(ad[8]), "v"(ad[9]), "v"(wad), "i"(KS * 16 * 128), "i"(KS * 16 * 256), "i"(KS * 16 * 4)
      : "memory");
}

// Weight of lane I of this lane's row of 16 (a DPP row broadcast, folded by
// the compiler into the multiply that uses it).
template <int I>
__device__ __forceinline__ float row_bcast(uint32_t wbits) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)wbits, 0x150 + I, 0xf, 0xf, false));
}

// 8 bf16 (a k-step's 8 tokens of one row) times the weights of chunk E (row
// lanes 8 E + 0..7 hold that chunk's weights of the lane's 8 tokens), rounded
// back to bf16.
template <int E>
__device__ __forceinline__ bf16x8_t scale_by_row_weights(const float (&x)[8], uint32_t wbits) {
  uint4 r;
  r.x = pack_bf16x2(x[0] * row_bcast<8 * E + 0>(wbits), x[1] * row_bcast<8 * E + 1>(wbits));
  r.y = pack_bf16x2(x[2] * row_bcast<8 * E + 2>(wbits), x[3] * row_bcast<8 * E + 3>(wbits));
  r.z = pack_bf16x2(x[4] * row_bcast<8 * E + 4>(wbits), x[5] * row_bcast<8 * E + 5>(wbits));
  r.w = pack_bf16x2(x[6] * row_bcast<8 * E + 6>(wbits), x[7] * row_bcast<8 * E + 7>(wbits));
  return __builtin_bit_cast(bf16x8_t, r);
}

// One k-step (16 tokens) of a staged sub-block of pass D: this lane's reads
// at `ad` (k-step 0) plus the k-step's offsets (token rows 16 KS + r keep
// the swizzle of rows r, which depends on r & 3), its weight slot at `wad`.
template <int KS>
__device__ __forceinline__ void d_kstep(const uint32_t (&ad)[10], uint32_t wad, int64_t sb, int64_t first1,
                                      int64_t wfirst, int half, int lane, f32x16_t (&acc)[2][4]) {
  uint64_t rd[10];
  uint32_t wbits;
  ld_tr10_w1<KS>(rd, wbits, ad, wad);
  // tokens before the weight's chunk sees them carry no weight
  if (sb < first1) {
    const int64_t tok = sb + 16 * KS + 8 * half + (lane & 7);
    wbits = tok >= wfirst ? wbits : 0u;
  }
  float x[8];
  x[0] = bf16lo((uint32_t)rd[0]); x[1] = bf16hi((uint32_t)rd[0]);
  x[2] = bf16lo((uint32_t)(rd[0] >> 32)); x[3] = bf16hi((uint32_t)(rd[0] >> 32));
  x[4] = bf16lo((uint32_t)rd[1]); x[5] = bf16hi((uint32_t)rd[1]);
  x[6] = bf16lo((uint32_t)(rd[1] >> 32)); x[7] = bf16hi((uint32_t)(rd[1] >> 32));
  // both chunks every k-step (branches here would copy accumulators): a
  // chunk that sees none of the sub-block has all weights zeroed above,
  // and a chunk past the last one is never stored
  const bf16x8_t as0 = scale_by_row_weights<0>(x, wbits);
  const bf16x8_t as1 = scale_by_row_weights<1>(x, wbits);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const bf16x8_t bn = __builtin_bit_cast(
        bf16x8_t, make_uint4((uint32_t)rd[2 + 2 * nb], (uint32_t)(rd[2 + 2 * nb] >> 32),
                             (uint32_t)rd[3 + 2 * nb], (uint32_t)(rd[3 + 2 * nb] >> 32)));
    acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as0, bn, acc[0][nb], 0, 0, 0);
    acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as1, bn, acc[1][nb], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_bwd_d_kernel(BwdDArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kStagesD * kStageD];

  // One block per (head, chunk group, term): heads fastest, then the two
  // terms, chunk groups from the first (longest token stream) on.  The two
  // terms of a chunk group stream disjoint inputs (dR, C and p; E, Q and dl)
  // and add into a zeroed d_dH: two addends per entry, so the sum does not
  // depend on their order.
  const int blk = blockIdx.x;
  const int bh = blk % a.BHp;
  if (bh >= a.BH) return;
  const int term = (blk / a.BHp) & 1;
  const int cg = blk / (2 * a.BHp);
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, grp16 = (lane >> 4) & 1, j16 = lane & 15;
  const int c0 = cg * kChunksD;
  const int64_t row0 = (int64_t)b * a.L;
  const int64_t ts = (int64_t)(c0 + 1) * a.S;          // first token any chunk of the block sees
  const int64_t n_tok = ts < a.L ? a.L - ts : 0;
  const int n_steps = (int)((n_tok + kSB - 1) / kSB);   // sub-blocks of 64 tokens

  // Step q streams sub-block n_steps - 1 - q: the tokens are streamed from
  // the end of the sequence, so the chunk groups of one head (same XCD)
  // start on the same tiles and share them in L2.  Wave w loads rows
  // 16w..16w+15 of both tiles (2 + 4 loads) and the weights of chunk c0 + w
  // (1 load).
  auto issue = [&](int q) {
    const bool live = q < n_steps;
    const int sbk = live ? n_steps - 1 - q : 0;
    const int64_t sb = ts + (int64_t)sbk * kSB;
    const int cnt = live ? (int)((a.L - sb) < kSB ? (a.L - sb) : kSB) : 1;
    uint8_t* st = s_lds + (q % kStagesD) * kStageD;
    const bf16_t* abase = term == 0 ? a.dR + ((row0 + sb) * a.H + h) * kP : a.E + ((row0 + sb) * a.G + g) * kP;
    const int astride = term == 0 ? a.H * kP : a.G * kP;
    const auto ra = buf_rsrc(abase, live ? (uint32_t)((cnt - 1) * astride + kP) * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i + (lane >> 3);
      const int piece = (lane & 7) ^ swz_x(r);
      buf_dma16(ra, (uint32_t)(r * astride + piece * 8) * 2, st + (16 * wave + 8 * i) * 128);
    }
    const bf16_t* bbase = (term == 0 ? a.C : a.Q) + ((row0 + sb) * a.G + g) * kN;
    const auto rbr = buf_rsrc(bbase, live ? (uint32_t)((cnt - 1) * a.G * kN + kN) * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      const int piece = (lane & 15) ^ swz_b(r);
      buf_dma16(rbr, (uint32_t)(r * a.G * kN + piece * 8) * 2, st + kATile + (16 * wave + 4 * i) * 256);
    }
    // weights of chunk c0 + wave for tokens sb .. sb+63 (p row or dl row)
    const int c = c0 + wave;
    const bool wl = live && c < a.M;
    const float* wrow = a.pd + ((int64_t)bh * a.M + (c < a.M ? c : 0)) * 2 * a.L + (term ? a.L : 0);
    const auto rw = buf_rsrc(wrow, wl ? (uint32_t)(a.L * 4) : 0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, (__attribute__((address_space(3))) void*)(st + kATile + kBTile + wave * kSB * 4), 4,
        (uint32_t)((sb - 0) + lane) * 4, 0, 0, 0);
  };

#pragma unroll
  for (int q = 0; q < kStagesD; ++q) issue(q);

  // Wave w computes p rows 32 ph .. 32 ph + 31 (ph = w & 1) of the two
  // chunks c0 + 2 cp, c0 + 2 cp + 1 (cp = w >> 1) over all 128 n: the scaled
  // operand (dR or E, 8 values per lane and k-step) serves four MFMAs per
  // chunk.
  const int ph = wave & 1, cp = wave >> 1;
  f32x16_t acc[2][4];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[e][nb] = f32x16_t{};
  // first token chunk c0 + 2 cp + e sees; this lane's weight slot: chunk
  // 2 cp + e with e = (lane >> 3) & 1, token 8 half + (lane & 7) of a k-step
  const int64_t first0 = (int64_t)(c0 + 2 * cp + 1) * a.S, first1 = first0 + a.S;
  const int we = (lane >> 3) & 1;
  const int64_t wfirst = we ? first1 : first0;
  const uint32_t w_lane = (uint32_t)((2 * cp + we) * kSB + 8 * half + (lane & 7)) * 4;
  // this lane's read offsets in k-step 0 of a staged sub-block: dR or E
  // (row p 32 ph + ..., 128-byte token rows) and C or Q (n block nb,
  // 256-byte token rows), each as two reads of 4 tokens
  uint32_t lane_off[10];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * half + 4 * hh + (j16 >> 2);
    const int cb = 16 * grp16 + 4 * (j16 & 3);
    const int pb = 32 * ph + cb;
    lane_off[hh] = r * 128 + (((pb >> 3) ^ swz_x(r)) << 4) + ((pb & 7) >> 2) * 8;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nc = 32 * nb + cb;
      lane_off[2 + 2 * nb + hh] = r * 256 + (((nc >> 3) ^ swz_b(r)) << 4) + ((nc & 7) >> 2) * 8;
    }
  }

  for (int q = 0; q < n_steps; ++q) {
    // Step q has landed once at most the loads issued after it remain:
    // before the first, the prologue's steps 1 and 2 (real or zero-length);
    // later only q + 1, which the prologue issued (q + 1 <= 2) or iteration
    // q - 1 did if it exists -- q + 2 is issued below, after the wait.
    asm volatile("" ::: "memory");
    if (q == 0)
      __builtin_amdgcn_s_waitcnt(0x0f7e);      // vmcnt(14): steps 1 and 2 in flight
    else if (q + 1 <= 2 || q + 1 < n_steps)
      __builtin_amdgcn_s_waitcnt(0x0f77);      // vmcnt(7): step q + 1 in flight
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (q >= 1 && q + 2 < n_steps) issue(q + 2);

    const int64_t sb = ts + (int64_t)(n_steps - 1 - q) * kSB;
    // skip a sub-block that neither chunk of the wave sees (uniform); a
    // chunk whose first visible token lies inside or after it has the
    // earlier tokens' weights zeroed
    if (c0 + 2 * cp >= a.M || sb + kSB <= first0) continue;
    const uint8_t* st = s_lds + (q % kStagesD) * kStageD;
    const uint32_t sa = lds_addr(st), sbb = sa + kATile;
    const uint32_t swt = sa + kATile + kBTile;  // weights: chunk k at + 256 k
    uint32_t ad[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) ad[i] = (i < 2 ? sa : sbb) + lane_off[i];
    __builtin_amdgcn_s_setprio(1);
    d_kstep<0>(ad, swt + w_lane, sb, first1, wfirst, half, lane, acc);
    d_kstep<1>(ad, swt + w_lane, sb, first1, wfirst, half, lane, acc);
    d_kstep<2>(ad, swt + w_lane, sb, first1, wfirst, half, lane, acc);
    d_kstep<3>(ad, swt + w_lane, sb, first1, wfirst, half, lane, acc);
    __builtin_amdgcn_s_setprio(0);
  }

  // a block with no token to stream still issued its (zero-length) prologue
  // loads into LDS: let them land before the block ends
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (n_steps == 0) return;

  // d_dH_c^T[p][n] += this term: register r holds p = 32 ph + 8 (r/4) +
  // 4 half + r%4, n = 32 nb + lane % 32
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = c0 + 2 * cp + e;
    if (c >= a.M) continue;
    float* outp = (term ? a.ddH1 : a.ddH) + ((int64_t)bh * a.M + c) * (kP * kN) + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = 32 * ph + 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) unsafeAtomicAdd(outp + p * kN + 32 * nb, acc[e][nb][r]);
    }
  }
}

// d_dH = 0 before the two terms add into it.
__global__ __launch_bounds__(256) void zero_f32_kernel(float4* p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_sma_bwd_d_mfma(const Shape& s, const void* dR, const void* E, const void* C,
                                 const void* Q, const float* pd, float* ddH, float* ddH_score,
                                 hipStream_t st) {
  BwdDArgs a;
  a.dR = (const bf16_t*)dR;
  a.E = (const bf16_t*)E;
  a.C = (const bf16_t*)C;
  a.Q = (const bf16_t*)Q;
  a.pd = pd;
  a.ddH = ddH;
  a.ddH1 = ddH_score ? ddH_score : ddH;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.n_groups = (int)((s.M + kChunksD - 1) / kChunksD);
  a.BH = (int)(s.b * s.H);
  a.BHp = (a.BH + 7) / 8 * 8;
  a.inv_sqrt_n = 1.f / sqrtf((float)kN);
  const int64_t blocks = (int64_t)a.BHp * a.n_groups * 2;
  if (blocks == 0) return hipSuccess;
  // every d_dH entry is a sum of the two terms' blocks (kP * kN floats per
  // chunk memory: a whole number of float4)
  const int64_t n4 = s.b * s.H * s.M * (kP * kN) / 4;
  const unsigned zb = (unsigned)(n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096);
  zero_f32_kernel<<<dim3(zb), dim3(256), 0, st>>>((float4*)ddH, n4);
  if (a.ddH1 != ddH) zero_f32_kernel<<<dim3(zb), dim3(256), 0, st>>>((float4*)a.ddH1, n4);
  sma_bwd_d_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

// Workspace of the MFMA backward: (p, dl) rows [b][H][M][2][L] float32, dR
// [b][L][H][P] bfloat16 and, for grouped heads, per-head dQ, dC [b][L][H][N]
// and dE [b][L][H][P] float32 (summed over the group at the end).
// ---------------------------------------------------------------------------
// Chunk memories transposed for pass BC: out[m][n][p] = in[m][p][n], 64 x 128
// two-byte entries per memory.  A thread moves an 8 x 8 tile (eight 16-byte
// rows in, eight out), two memories per block of 256 threads.
// ---------------------------------------------------------------------------
namespace {

__global__ __launch_bounds__(256) void mem_transpose_kernel(const uint4* in, uint4* out, int64_t count) {
  const int64_t m = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  if (m >= count) return;
  const int t = threadIdx.x & 127, nb = t & 15, pb = t >> 4;   // n = 8 nb .. +7, p = 8 pb .. +7
  const uint4* src = in + m * (kMemBytes / 16) + (pb * 8) * 16 + nb;
  uint4 r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = src[i * 16];   // row p = 8 pb + i
  // entry c (n = 8 nb + c) of row i: 16-bit half c % 2 of word c / 2
  auto el = [&](int i, int c) -> uint32_t {
    const uint32_t w = (c >> 1) == 0 ? r[i].x : (c >> 1) == 1 ? r[i].y : (c >> 1) == 2 ? r[i].z : r[i].w;
    return (c & 1) ? (w >> 16) : (w & 0xffffu);
  };
  uint4* dst = out + m * (kMemBytes / 16) + (nb * 8) * 8 + pb;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 o;
    o.x = el(0, c) | (el(1, c) << 16);
    o.y = el(2, c) | (el(3, c) << 16);
    o.z = el(4, c) | (el(5, c) << 16);
    o.w = el(6, c) | (el(7, c) << 16);
    dst[c * 8] = o;                                   // row n = 8 nb + c
  }
}

}  // namespace

hipError_t launch_mem_transpose(const void* in, void* out, int64_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  mem_transpose_kernel<<<dim3((unsigned)((count + 1) / 2)), dim3(256), 0, st>>>((const uint4*)in, (uint4*)out,
                                                                                 count);
  return hipGetLastError();
}

// Every part starts on a 256-byte boundary: dR takes 16-byte stores and
// 16-byte direct-to-LDS loads, the per-head partials 16-byte stores, and the
// transposed memories 16-byte stores and direct-to-LDS loads.
namespace {
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t pd_bytes_of(const Shape& s) { return round256((size_t)(2 * s.b * s.H * s.M * s.L) * 4); }
size_t dr_bytes_of(const Shape& s) { return round256((size_t)(s.b * s.L * s.H * s.P) * 2); }
size_t part_bytes_of(const Shape& s) {
  return s.H != s.G ? round256((size_t)(s.b * s.L * s.H * (2 * s.N + s.P)) * 4) : 0;
}
}  // namespace

// Layout: (p, dl) rows | dR | per-head partials (grouped heads) | dH transposed.
size_t sma_bwd_memt_offset(const Shape& s) { return pd_bytes_of(s) + dr_bytes_of(s) + part_bytes_of(s); }

size_t sma_bwd_mfma_workspace_bytes(const Shape& s) {
  return sma_bwd_memt_offset(s) + round256((size_t)(s.b * s.H * s.M) * kMemBytes);
}

hipError_t launch_sma_bwd_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                               const void* dH, const void* gate, int gate_pc, const float* R,
                               const float* lse, const void* dout, float* dQ, float* dC, float* dE,
                               float* ddH, float* dgate, void* ws, hipStream_t st) {
  uint8_t* w = (uint8_t*)ws;
  float* pd = (float*)w;
  void* dR = w + pd_bytes_of(s);
  const bool grouped = s.H != s.G;
  const size_t off = pd_bytes_of(s) + dr_bytes_of(s);
  float* hq = grouped ? (float*)(w + off) : dQ;
  float* hc = grouped ? hq + s.b * s.L * s.H * s.N : dC;
  float* he = grouped ? hc + s.b * s.L * s.H * s.N : dE;
  const int heads = grouped ? (int)s.H : (int)s.G;
  void* memT = w + sma_bwd_memt_offset(s);
  hipError_t e = launch_sma_bwd_a_mfma(s, Q, C, E, dH, gate, gate_pc, dout, R, lse, he, heads, pd, dR,
                                       dgate, st);
  if (e != hipSuccess) return e;
  if ((e = launch_mem_transpose(dH, memT, s.b * s.H * s.M, st)) != hipSuccess) return e;
  e = launch_sma_bwd_bc_mfma(s, kBcBoth, E, dR, memT, pd, nullptr, nullptr, hq, hc, heads, st);
  if (e != hipSuccess) return e;
  e = launch_sma_bwd_d_mfma(s, dR, E, C, Q, pd, ddH, nullptr, st);
  if (e != hipSuccess || !grouped) return e;
  const int64_t rows = s.b * s.L, hpg = s.H / s.G;
  if ((e = launch_group_sum(hq, dQ, rows, s.G, hpg, s.N, st)) != hipSuccess) return e;
  if ((e = launch_group_sum(hc, dC, rows, s.G, hpg, s.N, st)) != hipSuccess) return e;
  return launch_group_sum(he, dE, rows, s.G, hpg, s.P, st);
}

// ---------------------------------------------------------------------------
// Chunk-state backward: for the chunk's d_dH (G, staged as bf16 G^T[p][n])
//   T^T = G^T B_c^T  (P x S tokens):  dX_s = w_s T_s,  dw_s = X_s . T_s
//   dB^T = G X_c^T   (N x S tokens):  dB_s = w_s (dB^T)_s
// [§3 Eq. 5 differentiated]; dw goes to the decay recurrence kernel.
// ---------------------------------------------------------------------------
namespace {

constexpr int kGroupCS = 256;   // tokens per decay-weight group (one per thread)

// Byte offset of bf16 entry (row p, column n) of a chunk memory staged for the
// transposing reads: 256-byte rows of 16-byte pieces, piece ^ ((p & 3) << 2).
__device__ __forceinline__ uint32_t tr_off(int p, int n) {
  return (uint32_t)(p * 256 + ((((n >> 3) ^ ((p & 3) << 2))) << 4) + (n & 7) * 2);
}

// Eight transposing reads (4 bf16 = 8 bytes each) that return together; the
// tiles read are complete by construction (explicit wait + barrier), and the
// asm waits for its own results (the compiler's form of this read would drain
// every direct-to-LDS load in flight first).
__device__ __forceinline__ void ld_tr8(uint64_t (&o)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
      : "memory");
}

struct CsBwdArgs {
  const bf16_t* X;
  const bf16_t* B;
  const float* A;
  const float* ddH;    // [b][H][M][P][N] float32
  float* dX;           // [b][L][H][P]
  float* dB;           // [b][L][db_heads][N]
  float* wsw;          // [b][H][L]: w_s
  float* wsdw;         // [b][H][L]: dw_s
  int64_t L;
  int H, G, hpg, S, M, db_heads;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void chunk_states_bwd_mfma_kernel(CsBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_g[kMemBytes];   // G^T, tr-read swizzle
  __shared__ float s_w[kGroupCS + 4];
  // per wave: 8 KB of B rows (later the dX / dB rows on their way out) and
  // 4 KB of X rows
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[4 * 12288];

  const int nh = a.H;
  const int bb = blockIdx.x / (a.M * nh);
  const int rem = blockIdx.x - bb * (a.M * nh);
  const int c = rem / nh;
  const int bh = bb * nh + rem % nh;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int grp16 = (lane >> 4) & 1, j16 = lane & 15;
  const int64_t s0 = (int64_t)c * a.S;
  const int64_t s1 = (s0 + a.S < a.L) ? s0 + a.S : a.L;
  const int64_t row0 = (int64_t)b * a.L;

  // stage G^T (float32 in HBM) as bfloat16 for the matrix core
  {
    const float* gp = a.ddH + ((int64_t)bh * a.M + c) * (kP * kN);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (tid + 256 * i) * 8;  // 8 consecutive n of one row p
      const int p = e / kN, n = e % kN;
      const float4 v0 = *(const float4*)(gp + e), v1 = *(const float4*)(gp + e + 4);
      uint4 pk;
      pk.x = pack_bf16x2(v0.x, v0.y);
      pk.y = pack_bf16x2(v0.z, v0.w);
      pk.z = pack_bf16x2(v1.x, v1.y);
      pk.w = pack_bf16x2(v1.z, v1.w);
      *(uint4*)(s_g + tr_off(p, n)) = pk;
    }
  }
  // A operand of T^T: G^T rows p (k = n), read in 16-byte pieces
  auto gt_frag = [&](int prow, int ks) -> bf16x8_t {
    return *(const bf16x8_t*)(s_g + tr_off(prow, 16 * ks + 8 * half));
  };
  // A operand of dB^T: G rows n (k = p) by transposing reads (ld_tr8)
  uint32_t abase[4];
  const uint32_t sgb = lds_addr(s_g);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    abase[rb] = sgb + tr_off(8 * half + (j16 >> 2), 32 * rb + 16 * grp16 + 4 * (j16 & 3));

  float carry = 1.f;
  const int64_t n_tok = s1 - s0;
  for (int64_t gend = n_tok; gend > 0; gend -= kGroupCS) {   // groups from the chunk end
    const int64_t g0 = gend - kGroupCS > 0 ? gend - kGroupCS : 0;
    // weights of the group: in-wave suffix scan, then later waves and groups
    {
      const int64_t tg = s0 + g0 + tid;
      float v = (g0 + tid < gend) ? a.A[(row0 + tg) * a.H + h] : 1.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float u = __shfl_down(v, off);
        if (lane + off < 64) v *= u;
      }
      float nxt = __shfl_down(v, 1);
      if (lane == 63) nxt = 1.f;
      __syncthreads();  // previous group's weights are read; G staged
      if (lane == 0) s_w[kGroupCS + wave] = v;
      __syncthreads();
      float later = carry;
      for (int w2 = wave + 1; w2 < 4; ++w2) later *= s_w[kGroupCS + w2];
      const float wv = (g0 + tid < gend) ? later * nxt : 0.f;
      carry *= s_w[kGroupCS] * s_w[kGroupCS + 1] * s_w[kGroupCS + 2] * s_w[kGroupCS + 3];
      __syncthreads();
      s_w[tid] = wv;
      __syncthreads();
    }
    for (int64_t pb = g0; pb < gend; pb += kTile) {           // 128-token passes
      // This wave's 32 tokens from pb + 32 wave (nv of them hold data): the B
      // and X rows are staged whole in the wave's area (B: 256-byte rows, X:
      // 128-byte rows, 16-byte pieces XOR-swizzled by the row) and the MFMA
      // operands and the epilogue's X are read from there; dX and dB (float32)
      // leave through the B part as whole rows.  Rows past the group end read
      // zeros and their stores fall outside the buffer resources.
      uint8_t* const s_b = s_stage + wave * 12288;
      uint8_t* const s_x = s_b + 8192;
      const int64_t tw = pb + 32 * wave;  // chunk-local first token of the wave
      const int nv = (int)(gend - tw < 32 ? (gend - tw > 0 ? gend - tw : 0) : 32);
      const int64_t tok0 = row0 + s0 + tw;
      const int hh = a.db_heads == a.H ? h : g;
      const auto rsb = buf_rsrc(wave_uniform(a.B + (tok0 * a.G + g) * kN),
                                nv > 0 ? (uint32_t)((nv - 1) * a.G * kN + kN) * 2 : 0u);
      const auto rsx = buf_rsrc(wave_uniform(a.X + (tok0 * a.H + h) * kP),
                                nv > 0 ? (uint32_t)((nv - 1) * a.H * kP + kP) * 2 : 0u);
      const auto rdx = buf_rsrc(wave_uniform(a.dX + (tok0 * a.H + h) * kP),
                                nv > 0 ? (uint32_t)((nv - 1) * a.H * kP + kP) * 4 : 0u);
      const auto rdb = buf_rsrc(wave_uniform(a.dB + (tok0 * a.db_heads + hh) * kN),
                                nv > 0 ? (uint32_t)((nv - 1) * a.db_heads * kN + kN) * 4 : 0u);
      // the previous pass's reads of the area are done before the loads refill it
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4);
        buf_dma16(rsb, (uint32_t)(r * a.G * kN + (((lane & 15) ^ (r & 15)) << 3)) * 2, s_b + k * 1024);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3);
        buf_dma16(rsx, (uint32_t)(r * a.H * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2, s_x + k * 1024);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      // T^T = G^T B_c^T first (B operand: B_c^T, k = n, 8 per lane per step),
      // and its epilogue, then dB^T = G X_c^T: one accumulator set at a time.
      // Lane column = token; accumulator register r of row block rb holds row
      // 32 rb + 8 (r / 4) + 4 half + r % 4 (p for T, n for dB).
      const float w = s_w[(int)(tw - g0) + col];
      const int orow = lane >> 4, opc = lane & 15;
      {
        f32x16_t t0 = {}, t1 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t bv = *(const bf16x8_t*)(s_b + col * 256 + (((2 * ks + half) ^ (col & 15)) << 4));
          t0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gt_frag(col, ks), bv, t0, 0, 0, 0);
          t1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gt_frag(32 + col, ks), bv, t1, 0, 0, 0);
        }
        // dX = w T into the B part (its B rows are all read), dw = X . T
        float part = 0.f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16_t& tt = rb ? t1 : t0;
            const uint2 xv = *(const uint2*)(s_x + col * 128 + (((4 * rb + q) ^ (col & 7)) << 4) + 8 * half);
            part = fmaf(bf16lo(xv.x), tt[4 * q + 0], part);
            part = fmaf(bf16hi(xv.x), tt[4 * q + 1], part);
            part = fmaf(bf16lo(xv.y), tt[4 * q + 2], part);
            part = fmaf(bf16hi(xv.y), tt[4 * q + 3], part);
            *(float4*)(s_b + col * 256 + (((8 * rb + 2 * q + half) ^ (col & 15)) << 4)) =
                make_float4(w * tt[4 * q + 0], w * tt[4 * q + 1], w * tt[4 * q + 2], w * tt[4 * q + 3]);
          }
        const float dw = halves_sum(part);
        if (col < nv && half == 0) {
          a.wsw[(int64_t)bh * a.L + s0 + tw + col] = w;
          a.wsdw[(int64_t)bh * a.L + s0 + tw + col] = dw;
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 4 * k + orow;
          const u32x4_t v = *(const u32x4_t*)(s_b + r * 256 + ((opc ^ (r & 15)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(v, rdx, (uint32_t)(r * a.H * kP + 4 * opc) * 4, 0, 0);
        }
      }
      f32x16_t db[4] = {{}, {}, {}, {}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t xv = *(const bf16x8_t*)(s_x + col * 128 + (((2 * ks + half) ^ (col & 7)) << 4));
        uint32_t ad[8];
        uint64_t rd[8];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          ad[2 * rb] = abase[rb] + (uint32_t)(16 * ks) * 256;
          ad[2 * rb + 1] = ad[2 * rb] + 4 * 256;
        }
        ld_tr8(rd, ad);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const bf16x8_t af = __builtin_bit_cast(
              bf16x8_t, make_uint4((uint32_t)rd[2 * rb], (uint32_t)(rd[2 * rb] >> 32),
                                   (uint32_t)rd[2 * rb + 1], (uint32_t)(rd[2 * rb + 1] >> 32)));
          db[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, xv, db[rb], 0, 0, 0);
        }
      }
      // dB = w dB^T, 64 n at a time through the B part
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        // the rows above are read before this half overwrites them
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
        for (int rbb = 0; rbb < 2; ++rbb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16_t& dd = db[2 * hb + rbb];
            *(float4*)(s_b + col * 256 + (((8 * rbb + 2 * q + half) ^ (col & 15)) << 4)) =
                make_float4(w * dd[4 * q + 0], w * dd[4 * q + 1], w * dd[4 * q + 2], w * dd[4 * q + 3]);
          }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 4 * k + orow;
          const u32x4_t v = *(const u32x4_t*)(s_b + r * 256 + ((opc ^ (r & 15)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(v, rdb, (uint32_t)(r * a.db_heads * kN + 64 * hb + 4 * opc) * 4,
                                                 0, 0);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_states_bwd_mfma(const Shape& s, const void* X, const void* B, const float* A,
                                        const float* ddH, float* dX, float* dB, int db_heads,
                                        float* wsw, float* wsdw, hipStream_t st) {
  CsBwdArgs a;
  a.X = (const bf16_t*)X;
  a.B = (const bf16_t*)B;
  a.A = A;
  a.ddH = ddH;
  a.dX = dX;
  a.dB = dB;
  a.wsw = wsw;
  a.wsdw = wsdw;
  a.L = s.L;
  a.H = (int)s.H;
  a.G = (int)s.G;
  a.hpg = (int)(s.H / s.G);
  a.S = (int)s.S;
  a.M = (int)s.M;
  a.db_heads = db_heads;
  const int64_t blocks = s.b * s.H * s.M;
  if (blocks == 0) return hipSuccess;
  chunk_states_bwd_mfma_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dart
