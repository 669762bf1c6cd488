// State-memory attention forward on gfx950 MFMA: bfloat16 storage, N = 128,
// P = 64, float32 accumulation and softmax.
//
// Paper: "DART: Decoded Attention over Recurrent States for Efficient
// Long-Context Sequence Modeling" (arXiv 2608.02032), §3 Eq. 8-11 and §4
// Algorithm 1 (a query tile stays on chip while the history chunks stream).
//
// Work decomposition.  A block owns 128 consecutive tokens of one head
// (4 waves x 32 tokens) and streams the chunk memories dH_j, j = 0..n-1,
// where n is the chunk of the tile's last token.  Each dH_j^T (64 x 128 bf16,
// 16 KB) is staged once per block in LDS (double-buffered, XOR-swizzled
// 16-byte pieces, so the MFMA operand reads are bank-conflict free) and
// shared by the four waves.
//
// Per wave and history chunk, two products on v_mfma_f32_32x32x16_bf16:
//     W^T = dH_j^T Q_tile^T   (64 x 32)       V^T = dH_j^T C_tile^T   (64 x 32)
// The MFMA output puts one token per lane (column) and P along registers, so
//     l_t = sum_p W[t,p] E[t,p] / sqrt(N)      (= Q_t dH_j E_t / sqrt(N), Eq. 9)
// is 32 in-lane FMAs plus one swap between the two half-waves, and the online
// softmax (App. C Eq. 29-31) is purely per lane.  The paper forms the key
// K = dH_j E_t first and then Q_t K (Algorithm 1 steps 8-9); taking Q_t dH_j
// first is the same bilinear form by associativity, shares the dH_j operand
// with the value product and costs P instead of N FMAs per (token, chunk).
//
// Softmax in base 2 with a lazy running maximum: the reference point m is
// raised only when a logit exceeds it by more than kTau (base-2 units), so
// terms are at most 2^kTau and the rescale of O and d (which would otherwise
// run for every chunk) is almost never taken.  R = O/d and lse = m + log d are
// unchanged by the choice of m up to rounding.
//
// Block order: blocks are numbered tile-major (last tile first, i.e. longest
// history first) and head-minor over a head count padded to a multiple of 8.
// Consecutive block numbers go round-robin to the 8 XCDs, so every tile of one
// (b, h) lands on the same XCD and reuses that head's chunk memories in its L2.
#include "dart_internal.h"
#include "dev_common.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kTile = 128;       // tokens per block
constexpr int kThreads = 256;    // 4 waves x 32 tokens
constexpr int kMemBytes = kP * kN * 2;
constexpr float kTau = 8.f;

struct FwdArgs {
  const bf16_t* Q;
  const bf16_t* C;
  const bf16_t* E;
  const bf16_t* dH;
  const bf16_t* Y;
  const bf16_t* gate;
  bf16_t* out;
  float* R;
  float* lse;
  int64_t L;
  int H, G, hpg, S, M, gate_pc;
  int BH, BHp, n_tiles;
  float e_scale;  // log2(e) / sqrt(N)
};

// Byte offset of 16-byte piece `piece` (0..15) of row `row` (0..63) of a
// staged dH_j^T: rows are 256 bytes, pieces XOR-swizzled by the row.
__device__ __forceinline__ uint32_t mem_off(int row, int piece) {
  return (uint32_t)(row * 256 + ((piece ^ (row & 15)) << 4));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_fwd_mfma_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_mem[2][kMemBytes];

  const int blk = blockIdx.x;
  const int bh = blk % a.BHp;
  if (bh >= a.BH) return;
  const int tile = a.n_tiles - 1 - blk / a.BHp;
  const int b = bh / a.H, h = bh % a.H, g = h / a.hpg;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int64_t t0 = (int64_t)tile * kTile;
  const int64_t t = t0 + wave * 32 + col;
  const bool tok_ok = t < a.L;
  const int64_t tc = tok_ok ? t : a.L - 1;
  const int64_t t_last = (t0 + kTile < a.L ? t0 + kTile : a.L) - 1;
  const int n_hist = (int)(t_last / a.S);             // chunks read by the tile
  const int my_hist = tok_ok ? (int)(t / a.S) : 0;    // this token sees chunks < my_hist

  // ---- token operands: Q, C as MFMA B operands (8 n per lane per k-step)
  const int64_t grow = ((int64_t)b * a.L + tc) * a.G + g;
  bf16x8_t qf[8], cf[8];
  {
    const bf16x8_t* qp = (const bf16x8_t*)(a.Q + grow * kN + 8 * half);
    const bf16x8_t* cp = (const bf16x8_t*)(a.C + grow * kN + 8 * half);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = qp[2 * ks];
      cf[ks] = cp[2 * ks];
    }
  }
  // E in the accumulator layout: register r of row-block rb holds
  // p = 32 rb + 8 (r / 4) + 4 half + r % 4.
  float ef[2][16];
  {
    const bf16_t* ep = a.E + grow * kP + 4 * half;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint2 v = *(const uint2*)(ep + 32 * rb + 8 * gq);
        ef[rb][4 * gq + 0] = bf16lo(v.x) * a.e_scale;
        ef[rb][4 * gq + 1] = bf16hi(v.x) * a.e_scale;
        ef[rb][4 * gq + 2] = bf16lo(v.y) * a.e_scale;
        ef[rb][4 * gq + 3] = bf16hi(v.y) * a.e_scale;
      }
  }

  float o[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[0][r] = o[1][r] = 0.f;
  float m = -INFINITY, d = 0.f;

  if (n_hist > 0) {
    const uint8_t* mem_head = (const uint8_t*)(a.dH + (int64_t)bh * a.M * (kP * kN));
    const int srow = tid >> 4, spiece = tid & 15;  // staging: rows srow + 16 i, piece spiece
    const uint8_t* src0 = mem_head + spiece * 16 + srow * 256;
    uint4 st0, st1, st2, st3;  // this thread's four 16-byte pieces of the next memory
#define DART_GLOAD(j)                                                     \
  do {                                                                    \
    const uint8_t* src_ = src0 + (int64_t)(j) * kMemBytes;                \
    st0 = *(const uint4*)(src_);                                          \
    st1 = *(const uint4*)(src_ + 16 * 256);                               \
    st2 = *(const uint4*)(src_ + 32 * 256);                               \
    st3 = *(const uint4*)(src_ + 48 * 256);                               \
  } while (0)
#define DART_LSTORE(buf)                                                  \
  do {                                                                    \
    *(uint4*)(s_mem[buf] + mem_off(srow, spiece)) = st0;                  \
    *(uint4*)(s_mem[buf] + mem_off(srow + 16, spiece)) = st1;             \
    *(uint4*)(s_mem[buf] + mem_off(srow + 32, spiece)) = st2;             \
    *(uint4*)(s_mem[buf] + mem_off(srow + 48, spiece)) = st3;             \
  } while (0)
    DART_GLOAD(0);
    DART_LSTORE(0);
    // Drain every prologue load here: otherwise the waits for the token
    // operands are placed inside the loop, where they would also wait for
    // the prefetch of the next chunk memory on every iteration.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int j = 0; j < n_hist; ++j) {
      const int buf = j & 1;
      const bool more = j + 1 < n_hist;
      if (more) DART_GLOAD(j + 1);

      f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
      const uint8_t* sm = s_mem[buf];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t a0 = *(const bf16x8_t*)(sm + mem_off(col, 2 * ks + half));
        const bf16x8_t a1 = *(const bf16x8_t*)(sm + mem_off(32 + col, 2 * ks + half));
        w0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], w0, 0, 0, 0);
        w1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], w1, 0, 0, 0);
        v0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, cf[ks], v0, 0, 0, 0);
        v1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, cf[ks], v1, 0, 0, 0);
      }

      // chunk logit (base 2): this half-wave's 32 p values, then the other half's
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part = fmaf(w0[r], ef[0][r], part);
        part = fmaf(w1[r], ef[1][r], part);
      }
      const float l2 = part + __shfl_xor(part, 32);

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

      if (more) DART_LSTORE(buf ^ 1);
      __syncthreads();
    }
#undef DART_GLOAD
#undef DART_LSTORE
  }

  // ---- epilogue: R = O / d, lse = m + log d, out = Y + g * R  [§3 Eq. 10-11]
  if (!tok_ok) return;
  const float inv = d > 0.f ? 1.f / d : 0.f;
  const int64_t orow = ((int64_t)b * a.L + t) * a.H + h;
  const bf16_t* yp = a.Y + orow * kP + 4 * half;
  const bf16_t* gp = a.gate + (a.gate_pc ? orow * kP + 4 * half : orow);
  bf16_t* op = a.out + orow * kP + 4 * half;
  float* rp = a.R ? a.R + orow * kP + 4 * half : nullptr;
  const float gs = a.gate_pc ? 0.f : bf16_to_f32(*gp);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int off = 32 * rb + 8 * gq;
      const float r0 = o[rb][4 * gq + 0] * inv, r1 = o[rb][4 * gq + 1] * inv;
      const float r2 = o[rb][4 * gq + 2] * inv, r3 = o[rb][4 * gq + 3] * inv;
      const uint2 yv = *(const uint2*)(yp + off);
      float g0 = gs, g1 = gs, g2 = gs, g3 = gs;
      if (a.gate_pc) {
        const uint2 gv = *(const uint2*)(gp + off);
        g0 = bf16lo(gv.x); g1 = bf16hi(gv.x); g2 = bf16lo(gv.y); g3 = bf16hi(gv.y);
      }
      uint2 ov;
      ov.x = pack_bf16x2(fmaf(g0, r0, bf16lo(yv.x)), fmaf(g1, r1, bf16hi(yv.x)));
      ov.y = pack_bf16x2(fmaf(g2, r2, bf16lo(yv.y)), fmaf(g3, r3, bf16hi(yv.y)));
      *(uint2*)(op + off) = ov;
      if (rp) *(float4*)(rp + off) = make_float4(r0, r1, r2, r3);
    }
  if (a.lse && half == 0)
    a.lse[(int64_t)bh * a.L + t] = d > 0.f ? (m + fast_log2(d)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_sma_fwd_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                               const void* dH, const void* Y, const void* gate, int gate_pc,
                               void* out, float* R, float* lse, hipStream_t st) {
  FwdArgs a;
  a.Q = (const bf16_t*)Q;
  a.C = (const bf16_t*)C;
  a.E = (const bf16_t*)E;
  a.dH = (const bf16_t*)dH;
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
  const int64_t blocks = (int64_t)a.BHp * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  sma_fwd_mfma_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dart
