// Chunk state memories on gfx950 MFMA: bfloat16 storage, N = 128, P = 64,
// float32 accumulation.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §3 Eq. 5 (= App. A
// Eq. 20):  dH_[c] = sum_{s in [c]} A_{s+1:e(c)} B_s^T X_s.
//
// One block per (b, h, chunk); the output dH_[c]^T (64 x 128) is the product
//     D = X_c^T (diag(w) B_c)        (P x S) . (S x N)
// on v_mfma_f32_32x32x16_bf16, wave w owning columns n = 32w..32w+31 and both
// 32-row halves of p.  The kernel only streams its inputs once, so it is
// bound by HBM: every load is a direct global->LDS load of whole token rows
// (64-token sub-blocks of X and B exactly as they are stored, 24 KB), three
// sub-blocks in flight per block and two blocks per CU, non-temporal where no
// other block reads the rows again (X always, B when a group has one head:
// 7-9% faster than plain loads).  The contraction runs
// over tokens, and the MFMA operands want 8 consecutive tokens per lane, so
// they are fetched from the token-major tiles with the transposing LDS read
// (ds_read_b64_tr_b16: within a 16-lane group, lane i receives element i % 4
// of the 4-element rows addressed by lanes 4e + i / 4, e = 0..3).  The tiles
// are XOR-swizzled by row so that those reads are bank-conflict free; the
// swizzle is applied on the global side of the loads.
//
// Decay weights w_s = prod_{k=s+1}^{e(c)} a_k are a suffix product over the
// chunk.  Sub-blocks are consumed from the end of the chunk backward; for each
// 256-token group the block forms all weights at once (one token per thread:
// wave suffix scan with lane shuffles, then the products of the later waves
// and of the later groups, `carry`).  The weights scale the B operand in
// float32, rounded once to bf16.  Underflow to zero is the correct value.
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kSB = 64;                    // tokens per sub-block
constexpr int kStages = 3;                 // LDS ring of sub-blocks
constexpr int kXTile = kSB * kP * 2;       // 8 KB, rows of 128 B
constexpr int kBTile = kSB * kN * 2;       // 16 KB, rows of 256 B
constexpr int kStage = kXTile + kBTile;
constexpr int kGroup = 256;                // tokens per decay-weight group
constexpr int kThreads = 256;
static_assert(kGroup == kThreads, "one token per thread in the weight scan");
static_assert(kStages == 3, "the wait counts below assume two sub-blocks in flight");

struct CsArgs {
  const bf16_t* X;
  const bf16_t* B;
  const float* A;
  bf16_t* dH;
  // RMS-normalised score branch (all nullable): inverse RMS of each key row
  // r [b][H][M][N] and the float16 score memory, RMSNorm weights folded in
  float* r;
  _Float16* dHs;
  const float* wq;
  const float* we;
  float eps;
  int64_t L;
  int H, G, hpg, S, M;
};


// Six transposing reads (4 bf16 = 8 bytes each) that return together.  The
// compiler treats its own form of this read as possibly overlapping the
// global->LDS loads in flight and drains them all before it; here the tiles
// read are complete by construction (explicit wait + barrier), so the reads
// are issued as one asm block that waits for its own results before it ends.
__device__ __forceinline__ void ld_tr6(uint64_t (&o)[6], const uint32_t (&ad)[6]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %6\n\t"
      "ds_read_b64_tr_b16 %1, %7\n\t"
      "ds_read_b64_tr_b16 %2, %8\n\t"
      "ds_read_b64_tr_b16 %3, %9\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5])
      : "memory");
}

// Swizzled 16-byte piece of a tile row (X rows: 8 pieces, B rows: 16).
__device__ __forceinline__ int swz_x(int row) { return (row & 3) << 1; }
__device__ __forceinline__ int swz_b(int row) { return (row & 3) << 2; }

// s_waitcnt immediates beyond the shared ones: vmcnt(6), vmcnt(12)
constexpr unsigned kWaitVm6 = 0x0f76;
constexpr unsigned kWaitVm12 = 0x0f7c;

// Block barrier for data exchanged through LDS only.  __syncthreads() would
// also wait for every outstanding global->LDS load (its fence covers global
// memory); the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Barrier after waiting until at most `n` (0, 6 or 12) of this wave's loads
// are outstanding.
__device__ __forceinline__ void barrier_loads(int n) {
  asm volatile("" ::: "memory");
  if (n >= 12)
    __builtin_amdgcn_s_waitcnt(kWaitVm12);
  else if (n >= 6)
    __builtin_amdgcn_s_waitcnt(kWaitVm6);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool kRms, bool kNtB>
__global__ __launch_bounds__(kThreads) void chunk_states_mfma_kernel(CsArgs a) {
  // Sub-block ring, and (a separate object, so that reading it does not make
  // the compiler wait for the loads into the ring) the current group's
  // weights and the per-wave decay products.
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kStages * kStage];
  __shared__ __attribute__((aligned(16))) float s_wt[kGroup + 4];
  float* const s_w = s_wt;
  float* const s_tot = s_wt + kGroup;

  // Blocks are numbered head-fastest within a batch row: the blocks in flight
  // together read all heads' slices of the same token rows, whole rows of X
  // and B at a time, instead of thin slices of a few heads spread over the
  // sequence.
  const int nh = a.H;
  const int bb = blockIdx.x / (a.M * nh);
  const int rem = blockIdx.x - bb * (a.M * nh);
  const int c = rem / nh;
  const int bh = bb * nh + rem % nh;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int half = lane >> 5, grp16 = (lane >> 4) & 1, j16 = lane & 15;

  const int64_t s0 = (int64_t)c * a.S;
  const int64_t s1 = (s0 + a.S < a.L) ? s0 + a.S : a.L;
  const int nblk = (int)((s1 - s0 + kSB - 1) / kSB);
  const int64_t row0 = (int64_t)b * a.L;

  // Sub-block q in consumption order is ib = nblk-1-q; it goes to stage q % 3.
  // Each wave loads rows 16w .. 16w+15 of both tiles: 2 loads of 8 X rows and
  // 4 loads of 4 B rows (6 per wave per sub-block).  Rows past the chunk end
  // lie past the end of the resource and read as zeros.  For q >= nblk the
  // loads have length 0 (they touch no memory) and fill a stage no sub-block
  // uses: the prologue then issues the same number of loads on one path, and
  // the compiler's wait for the decays can leave all of them in flight.
  auto issue = [&](int q) {
    const bool live = q < nblk;
    const int ib = live ? nblk - 1 - q : 0;
    const int64_t sb = s0 + (int64_t)ib * kSB;
    const int cnt = (int)((s1 - sb) < kSB ? (s1 - sb) : kSB);
    uint8_t* st = s_lds + (q % kStages) * kStage;
    const auto rx = buf_rsrc(wave_uniform(a.X + ((row0 + sb) * a.H + h) * kP),
                             live ? (uint32_t)((cnt - 1) * a.H * kP + kP) * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wave + 8 * i + (lane >> 3);
      const int piece = (lane & 7) ^ swz_x(r);
      buf_dma16_nt(rx, (uint32_t)(r * a.H * kP + piece * 8) * 2, st + (16 * wave + 8 * i) * 128);
    }
    const auto rb = buf_rsrc(wave_uniform(a.B + ((row0 + sb) * a.G + g) * kN),
                             live ? (uint32_t)((cnt - 1) * a.G * kN + kN) * 2 : 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4);
      const int piece = (lane & 15) ^ swz_b(r);
      const uint32_t off = (uint32_t)(r * a.G * kN + piece * 8) * 2;
      if constexpr (kNtB)
        buf_dma16_nt(rb, off, st + kXTile + (16 * wave + 4 * i) * 256);
      else  // the group's other heads read these B rows again
        buf_dma16(rb, off, st + kXTile + (16 * wave + 4 * i) * 256);
    }
  };

  // decay of this thread's token in the group that holds sub-block ib;
  // without a branch (threads past the chunk end re-read its last token),
  // so that no address is formed in divergent code, where the compiler
  // would take it for a per-lane value
  auto load_decay = [&](int ib) {
    const int64_t t = s0 + (int64_t)(ib / 4) * kGroup + tid;
    const float v = a.A[(row0 + (t < s1 ? t : s1 - 1)) * a.H + h];
    return t < s1 ? v : 1.f;
  };

  float carry = 1.f;  // product of a_k over the tokens of later groups
  // Weights of the group holding sub-block ib, from this thread's decay `v`:
  // in-wave inclusive suffix product, then the later waves of the group and
  // the later groups.  Tokens past the chunk end get weight 0.
  auto form_weights = [&](int ib, float v) {
    const int64_t tg = s0 + (int64_t)(ib / 4) * kGroup + tid;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float u = __shfl_down(v, off);
      if (lane + off < 64) v *= u;
    }
    if (lane == 0) s_tot[wave] = v;
    float nxt = __shfl_down(v, 1);
    if (lane == 63) nxt = 1.f;
    barrier_lds();
    float later = carry;
    for (int w2 = wave + 1; w2 < 4; ++w2) later *= s_tot[w2];
    s_w[tid] = tg < s1 ? later * nxt : 0.f;
    carry *= s_tot[0] * s_tot[1] * s_tot[2] * s_tot[3];
    barrier_lds();
  };

  // The last group's decays are loaded before the sub-blocks, so that the
  // wait for them leaves the sub-block loads in flight.
  const float a_last = load_decay(nblk - 1);
#pragma unroll
  for (int q = 0; q < kStages; ++q) issue(q);
  form_weights(nblk - 1, a_last);

  f32x16_t acc0 = {}, acc1 = {};
  for (int q = 0; q < nblk; ++q) {
    const int ib = nblk - 1 - q;
    // Sub-block q has landed once at most the loads issued after it remain:
    // before the first, the prologue's sub-blocks 1 and 2 (real or
    // zero-length); later only q + 1, which the prologue issued (q + 1 <= 2)
    // or iteration q - 1 did if it exists -- q + 2 is issued below, after
    // the wait.  The barrier makes every wave's part visible and frees stage
    // (q - 1) % 3.
    barrier_loads(q == 0 ? 12 : (q + 1 <= 2 || q + 1 < nblk) ? 6 : 0);
    if (q >= 1 && q + 2 < nblk) issue(q + 2);
    // Chunks longer than one group: the next group's weights (its decays
    // are loaded here, so this wait does drain the loads in flight).
    if (q > 0 && (ib & 3) == 3) form_weights(ib, load_decay(ib));

    const uint8_t* xt = s_lds + (q % kStages) * kStage;
    const uint8_t* bt = xt + kXTile;
    const float* wq = s_w + (ib & 3) * kSB;
#pragma unroll
    for (int ks = 0; ks < kSB / 16; ++ks) {
      // lane (column j16 + 16 grp16 of its operand, k-octet `half`) receives
      // tokens 16 ks + 8 half + 4 hh + 0..3 from read hh; it addresses token
      // row 16 ks + 8 half + 4 hh + j16/4 at column 16 grp16 + 4 (j16 % 4)
      uint32_t ad[6];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 16 * ks + 8 * half + 4 * hh + (j16 >> 2);
        const int cb = 16 * grp16 + 4 * (j16 & 3);  // column within a 32-wide operand
        const int nb = 32 * wave + cb;              // n
        ad[hh] = lds_addr(bt + r * 256 + (((nb >> 3) ^ swz_b(r)) << 4) + ((nb & 7) >> 2) * 8);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int pb = 32 * f + cb;  // p
          ad[2 + 2 * f + hh] = lds_addr(xt + r * 128 + (((pb >> 3) ^ swz_x(r)) << 4) + ((pb & 7) >> 2) * 8);
        }
      }
      uint64_t rd[6];
      ld_tr6(rd, ad);
      uint2 br[2], xr[2][2];
      br[0] = __builtin_bit_cast(uint2, rd[0]);
      br[1] = __builtin_bit_cast(uint2, rd[1]);
      xr[0][0] = __builtin_bit_cast(uint2, rd[2]);
      xr[0][1] = __builtin_bit_cast(uint2, rd[3]);
      xr[1][0] = __builtin_bit_cast(uint2, rd[4]);
      xr[1][1] = __builtin_bit_cast(uint2, rd[5]);
      // weights of this lane's 8 tokens scale the B operand
      const float4 w0 = *(const float4*)(wq + 16 * ks + 8 * half);
      const float4 w1 = *(const float4*)(wq + 16 * ks + 8 * half + 4);
      uint4 bs;
      bs.x = pack_bf16x2(bf16lo(br[0].x) * w0.x, bf16hi(br[0].x) * w0.y);
      bs.y = pack_bf16x2(bf16lo(br[0].y) * w0.z, bf16hi(br[0].y) * w0.w);
      bs.z = pack_bf16x2(bf16lo(br[1].x) * w1.x, bf16hi(br[1].x) * w1.y);
      bs.w = pack_bf16x2(bf16lo(br[1].y) * w1.z, bf16hi(br[1].y) * w1.w);
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bs);
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, make_uint4(xr[0][0].x, xr[0][0].y, xr[0][1].x, xr[0][1].y));
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, make_uint4(xr[1][0].x, xr[1][0].y, xr[1][1].x, xr[1][1].y));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bop, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bop, acc1, 0, 0, 0);
    }
  }

  // D[p][n]: register r of row block rb is p = 32 rb + 8 (r/4) + 4 half + r%4
  const int64_t mem = ((int64_t)bh * a.M + c) * (kP * kN);
  const int n = 32 * wave + (lane & 31);
  bf16_t* outp = a.dH + mem + n;
  uint32_t h0[16], h1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int p = 8 * (r >> 2) + 4 * half + (r & 3);
    h0[r] = f32_to_bf16(acc0[r]);
    h1[r] = f32_to_bf16(acc1[r]);
    outp[p * kN] = (bf16_t)h0[r];
    outp[(32 + p) * kN] = (bf16_t)h1[r];
  }
  if (kRms) {
    // r_c[n] = (mean_p dH[p][n]^2 + eps)^(-1/2) of the memory as stored
    // [App. B.1 Eq. 26]: this lane holds 32 of the 64 p of key row n, lane
    // l ^ 32 the others; then the score memory w_e[p] dH[p][n] r[n] w_q[n]
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x0 = bf16_to_f32(h0[r]), x1 = bf16_to_f32(h1[r]);
      ss = fmaf(x0, x0, fmaf(x1, x1, ss));
    }
    const float rn = 1.f / sqrtf(halves_sum(ss) * (1.f / kP) + a.eps);
    if (a.r && half == 0) a.r[((int64_t)bh * a.M + c) * kN + n] = rn;
    if (a.dHs) {
      const float rq = a.wq ? rn * a.wq[n] : rn;
      _Float16* sp = a.dHs + mem + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = 8 * (r >> 2) + 4 * half + (r & 3);
        const float w0 = a.we ? a.we[p] : 1.f, w1 = a.we ? a.we[32 + p] : 1.f;
        sp[p * kN] = (_Float16)(bf16_to_f32(h0[r]) * rq * w0);
        sp[(32 + p) * kN] = (_Float16)(bf16_to_f32(h1[r]) * rq * w1);
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_states_mfma(const Shape& s, const void* X, const void* B, const float* A,
                                    void* dH, hipStream_t st, float eps, const float* wq,
                                    const float* we, float* r, void* dHs) {
  CsArgs a;
  a.r = r;
  a.dHs = (_Float16*)dHs;
  a.wq = wq;
  a.we = we;
  a.eps = eps;
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
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (r || dHs) {
    if (a.hpg == 1)
      chunk_states_mfma_kernel<true, true><<<grid, block, 0, st>>>(a);
    else
      chunk_states_mfma_kernel<true, false><<<grid, block, 0, st>>>(a);
  } else {
    if (a.hpg == 1)
      chunk_states_mfma_kernel<false, true><<<grid, block, 0, st>>>(a);
    else
      chunk_states_mfma_kernel<false, false><<<grid, block, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dart
