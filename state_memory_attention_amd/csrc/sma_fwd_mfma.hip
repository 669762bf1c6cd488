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
// 16 KB) is staged once per block in LDS and shared by the four waves: a ring
// of 4 buffers filled by direct global->LDS loads three chunks ahead (the
// memories mostly come from the last-level cache, whose latency one chunk of
// MFMA work does not cover), with XOR-swizzled 16-byte pieces so the MFMA
// operand reads are bank-conflict free.
//
// Per wave and history chunk, two products on v_mfma_f32_32x32x16_bf16:
//     W^T = dH_j^T Q_tile^T   (64 x 32)       V^T = dH_j^T C_tile^T   (64 x 32)
// The MFMA output puts one token per lane (column) and P along registers, so
//     l_t = sum_p W[t,p] E[t,p] / sqrt(N)      (= Q_t dH_j E_t / sqrt(N), Eq. 9)
// is 32 in-lane FMAs plus one swap between the two half-waves, and the online
// softmax (App. C Eq. 29-31) is purely per lane.  The paper forms the key
// K = dH_j E_t first and then Q_t K (§4 Algorithm 1, key readout); taking Q_t dH_j
// first is the same bilinear form by associativity, shares the dH_j operand
// with the value product and costs P instead of N FMAs per (token, chunk).
//
// Softmax in base 2 with a lazy running maximum: the reference point m is
// raised only when a logit exceeds it by more than kTau (base-2 units), so
// terms are at most 2^kTau and the rescale of O and d (which would otherwise
// run for every chunk) is almost never taken.  R = O/d and lse = m + log d are
// unchanged by the choice of m up to rounding.
//
// Block order (head_major_tile): every tile of one (b, h) lands on the same
// XCD, each XCD works through its heads one after another, longest history
// first, so the tiles in flight reuse one or two heads' chunk memories from
// that XCD's L2.
#include "dart_internal.h"
#include "dev_common.h"
#include "lds_dma.h"

namespace dart {
namespace {

constexpr int kN = 128;
constexpr int kP = 64;
constexpr int kTile = 128;       // tokens per block
constexpr int kThreads = 256;    // 4 waves x 32 tokens
constexpr int kMemBytes = kP * kN * 2;
constexpr int kRing = 4;         // LDS buffers for chunk memories (3 in flight)
constexpr float kTau = 8.f;
static_assert(kRing == 4, "the loop's wait counts assume 3 chunks in flight");

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

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sma_fwd_mfma_kernel(FwdArgs a) {
  // 64 KB ring of chunk memories and a 16 KB area for the Y tile (later the
  // out tile): 80 KB, two blocks per CU.  One LDS object on purpose: the
  // loop's waits for the in-flight chunk loads are explicit (below), and with
  // a single object the compiler adds no wait of its own for them before
  // each read of the ring.
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kRing * kMemBytes + kTile * kP * 2];
  uint8_t* const s_mem = s_lds;
  uint8_t* const s_y = s_lds + kRing * kMemBytes;

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
  const int n_hist = (int)(t_last / a.S);  // chunks read by the tile
  // this lane's token t0 + 32 wave + col sees chunks < my_hist
  const int my_hist = (t0 + wave * 32 + col < a.L) ? (int)((t0 + wave * 32 + col) / a.S) : 0;

  // ---- streamed inputs.  Slots in order: chunk memories 0..n_hist-1, then
  // the per-channel gate tile; slot s goes to ring buffer s % kRing.  Every
  // slot costs every wave exactly 4 direct-to-LDS loads, so the waits below
  // only count slots; the first three slots are always issued (zero-length
  // loads stand in for missing ones), the Y tile goes to its own area once
  // the prologue is done with it.  A chunk load of wave w writes rows 16w .. 16w+15 of dH_j^T (4
  // loads of 4 rows); a token-tile load of wave w writes the wave's own token
  // rows 32w .. 32w+31 (4 loads of 8 rows of 128 B).  One such load writes
  // 1 KB contiguously, so the XOR swizzle is applied on the global side: the
  // lane that fills physical piece f of row r fetches logical piece
  // f ^ (r & 15) (256-byte rows) or f ^ (r & 7) (128-byte rows).
  const int64_t row0 = (int64_t)b * a.L;  // token index of this batch row
  const uint8_t* mem_head = (const uint8_t*)(a.dH + (int64_t)bh * a.M * (kP * kN));
  // lane part of a chunk load: row 16 wave + 4 i + lane/16 (+ 4 rows per i)
  const uint32_t mem_dma = (16 * wave + (lane >> 4)) * 256;
  const int n_slots = n_hist + (a.gate_pc ? 1 : 0);
  auto slot_buf = [&](int s) -> uint8_t* { return s_mem + (s % kRing) * kMemBytes; };
  auto issue_mem = [&](int s) {
    const auto rs = buf_rsrc(mem_head + (int64_t)s * kMemBytes, kMemBytes);
    uint8_t* dst = slot_buf(s) + wave * 16 * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      buf_dma16(rs, mem_dma + i * 1024 + (((lane & 15) ^ (row & 15)) << 4), dst + i * 4 * 256);
    }
  };
  // token rows of this tile past the sequence end re-read the last token
  const int last_r = (int)(a.L - 1 - t0 < kTile - 1 ? a.L - 1 - t0 : kTile - 1);
  const uint32_t tok_bytes = (uint32_t)(last_r * a.H * kP + kP) * 2;
  auto issue_tok = [&](const bf16_t* base, uint8_t* area) {
    const auto rs = buf_rsrc(base + ((row0 + t0) * a.H + h) * kP, tok_bytes);
    uint8_t* dst = area + wave * 16 * 256;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 32 * wave + 8 * k + (lane >> 3);
      const int rr = r < last_r ? r : last_r;
      buf_dma16(rs, (uint32_t)(rr * a.H * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2, dst + k * 8 * 128);
    }
  };
  // Slot s (a chunk, the gate tile or, past the last slot, a zero-length
  // stand-in) without branches: the compiler places its waits for the token
  // operands below from the loads issued on every path, and with a branch
  // here it would count the fewest and drain the slots as well.
  const uint8_t* tok_gate = (const uint8_t*)(a.gate + ((row0 + t0) * a.H + h) * kP);
  auto issue = [&](int s) {
    const bool is_mem = s < n_hist, is_tok = !is_mem && s < n_slots;
    const uint8_t* base = is_mem ? mem_head + (int64_t)s * kMemBytes : (is_tok ? tok_gate : mem_head);
    const auto rs = buf_rsrc(base, is_mem ? kMemBytes : (is_tok ? tok_bytes : 0u));
    uint8_t* dst = slot_buf(s) + wave * 16 * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const uint32_t vm = mem_dma + i * 1024 + (((lane & 15) ^ (row & 15)) << 4);
      const int r = 32 * wave + 8 * i + (lane >> 3);
      const int rr = r < last_r ? r : last_r;
      const uint32_t vt = (uint32_t)(rr * a.H * kP + (((lane & 7) ^ (r & 7)) << 3)) * 2;
      buf_dma16(rs, is_tok ? vt : vm, dst + i * 1024);
    }
  };

  // ---- the first three slots, then the token operands to registers: Q and
  // C as MFMA B operands (lane holds token `col`, n = 16 ks + 8 half + 0..7),
  // E in the accumulator layout (register r of row-block rb holds
  // p = 32 rb + 8 (r / 4) + 4 half + r % 4).  Q and C are staged as whole
  // rows through a wave-private 8 KB area (ring buffer 3 and the Y area are
  // not needed before the loop), Q with the slots and E, C in a second round:
  // loads straight to registers in the MFMA operand layout would touch 32
  // token rows of 32 bytes each per instruction, and cost more than the
  // extra round.
  issue(0);
  issue(1);
  issue(2);
  uint8_t* const s_st = s_mem + 3 * kMemBytes + wave * 8192;
  const uint32_t qc_bytes = (uint32_t)(last_r * a.G * kN + kN) * 2;
  const int64_t qc_base = ((row0 + t0) * a.G + g) * kN;
  // token rows 32 wave + 4 k + lane/16 (past the sequence end: the last
  // token), local row lr = 4 k + lane/16 at s_st + 256 lr, pieces swizzled
  // as in a staged chunk memory (mem_off)
  auto stage = [&](const bf16_t* base) {
    const auto rs = buf_rsrc(wave_uniform(base + qc_base), qc_bytes);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int lr = 4 * k + (lane >> 4);
      const int r = 32 * wave + lr;
      const int rr = r < last_r ? r : last_r;
      buf_dma16(rs, (uint32_t)(rr * a.G * kN + (((lane & 15) ^ (lr & 15)) << 3)) * 2, s_st + k * 1024);
    }
  };
  stage(a.Q);
  bf16x8_t qf[8], cf[8];
  float ef[2][16];
  {
    const int64_t tl = t0 + wave * 32 + col;
    const int64_t tok = row0 + (tl < a.L ? tl : a.L - 1);
    uint2 ev[2][4];
    const bf16_t* ep = a.E + (tok * a.G + g) * kP + 4 * half;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) ev[rb][gq] = *(const uint2*)(ep + 32 * rb + 8 * gq);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8_t*)(s_st + mem_off(col, 2 * ks + half));
    // the Q rows have been read before the C rows overwrite them
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    stage(a.C);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 v = ev[rb][gq];
        ef[rb][4 * gq + 0] = bf16lo(v.x) * a.e_scale;
        ef[rb][4 * gq + 1] = bf16hi(v.x) * a.e_scale;
        ef[rb][4 * gq + 2] = bf16lo(v.y) * a.e_scale;
        ef[rb][4 * gq + 3] = bf16hi(v.y) * a.e_scale;
      }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) cf[ks] = *(const bf16x8_t*)(s_st + mem_off(col, 2 * ks + half));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  float o[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[0][r] = o[1][r] = 0.f;
  float m = -INFINITY, d = 0.f;

  // Slots 0..2 have landed in every wave's part and no wave reads its
  // staging area any more: the Y tile goes to its area now, ahead of slot 3
  // (so the loop's waits for slots 3 and later cover it as well).
  __builtin_amdgcn_s_barrier();
  issue_tok(a.Y, s_y);

  for (int j = 0; j < n_hist; ++j) {
    // Chunk j must have landed in every wave's part, and every wave must be
    // done with chunk j-1 before its buffer is refilled (by slot j+kRing-1: a
    // chunk prefetch is issued inside the MFMA burst below so that its issue
    // cost hides behind queued matrix work).  The vector-memory operations
    // in flight are these slot loads and the Y tile (older than every slot
    // past 2), so wait until at most slots j+1 .. j+kRing-2 remain
    // (__syncthreads() would wait for all of them).  Slots 0..2 landed
    // before the barrier above; later slots are issued only if they exist.
    if (j > 0) {
      // loads that may stay in flight: those of slots j+1 and j+2 issued in
      // the loop (slots past 2 that exist)
      const int after = (j + 1 >= 3 && j + 1 < n_slots) + (j + 2 >= 3 && j + 2 < n_slots);
      if (after == 2)
        __builtin_amdgcn_s_waitcnt(kWaitVm8Lgkm0);
      else if (after == 1)
        __builtin_amdgcn_s_waitcnt(kWaitVm4Lgkm0);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVm0 & kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
    }

    if (j + kRing - 1 == n_hist && j + kRing - 1 < n_slots) issue_tok(a.gate, slot_buf(j + kRing - 1));

    // The MFMA burst runs at raised wave priority, so that a wave entering
    // it is not held back by the other block's softmax work on this SIMD.
    __builtin_amdgcn_s_setprio(1);
    f32x16_t w0 = {}, w1 = {}, v0 = {}, v1 = {};
    const uint8_t* sm = slot_buf(j);
    // dH_j^T operands are read one k-step ahead of the MFMAs that use them;
    // the scheduling barriers after the loop pin that order (left alone, the
    // scheduler sinks each read to just before its use and the LDS latency
    // shows up between MFMA groups).
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
      if (ks == 1 && j + kRing - 1 < n_hist) issue_mem(j + kRing - 1);
      // A wave whose burst is under way outranks one about to start its own,
      // so the two waves sharing a SIMD take the matrix core in turns and
      // each one's softmax tail overlaps the other's burst (at equal priority
      // they interleave, finish together and then idle the matrix core
      // through both tails).
      if (ks == 0) __builtin_amdgcn_s_setprio(2);
    }
    // burst order: [2 LDS reads for step k+1][4 MFMAs of step k], k = 0..7
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);              // MFMA
    }
    __builtin_amdgcn_s_setprio(0);

    // chunk logit (base 2): this half-wave's 32 p values, then the other half's
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(w0[r], ef[0][r], part);
      part = fmaf(w1[r], ef[1][r], part);
    }
    // + the other half-wave's part (lanes l and l ^ 32 swap halves)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                     false, false);
    const float l2 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);

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

  // ---- epilogue: R = O / d, lse = m + log d, out = Y + g * R  [§3 Eq. 10-11]
  // Each wave reads only the Y / gate rows it loaded itself, so waiting for
  // its own loads is enough.  `out` replaces the wave's Y rows in place
  // (every lane rewrites exactly the bytes it read) and leaves as whole
  // 128-byte rows.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  const int64_t t = t0 + wave * 32 + col;
  const bool tok_ok = t < a.L;
  const int64_t tc = tok_ok ? t : a.L - 1;
  const float inv = d > 0.f ? 1.f / d : 0.f;
  const int tr = 32 * wave + col;  // this lane's token row in the tile
  const uint8_t* ybuf = s_y;
  const uint8_t* gbuf = slot_buf(n_hist);
  const int64_t orow = (row0 + tc) * a.H + h;
  const float gs = a.gate_pc ? 0.f : bf16_to_f32(a.gate[orow]);
  float* rp = (a.R && tok_ok) ? a.R + orow * kP + 4 * half : nullptr;
  // every Y and gate read is issued before the first use (a per-step branch
  // on the gate form made each read wait for itself); with a scalar gate the
  // gate slot holds a zero-length stand-in whose bytes are read and ignored
  uint2 yv[2][4], gv[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t lo = tr * 128 + (((4 * rb + gq) ^ (tr & 7)) << 4) + 8 * half;
      yv[rb][gq] = *(const uint2*)(ybuf + lo);
      gv[rb][gq] = *(const uint2*)(gbuf + lo);
    }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t lo = tr * 128 + (((4 * rb + gq) ^ (tr & 7)) << 4) + 8 * half;
      const float r0 = o[rb][4 * gq + 0] * inv, r1 = o[rb][4 * gq + 1] * inv;
      const float r2 = o[rb][4 * gq + 2] * inv, r3 = o[rb][4 * gq + 3] * inv;
      const uint2 y = yv[rb][gq], g = gv[rb][gq];
      const float g0 = a.gate_pc ? bf16lo(g.x) : gs, g1 = a.gate_pc ? bf16hi(g.x) : gs;
      const float g2 = a.gate_pc ? bf16lo(g.y) : gs, g3 = a.gate_pc ? bf16hi(g.y) : gs;
      uint2 ov;
      ov.x = pack_bf16x2(fmaf(g0, r0, bf16lo(y.x)), fmaf(g1, r1, bf16hi(y.x)));
      ov.y = pack_bf16x2(fmaf(g2, r2, bf16lo(y.y)), fmaf(g3, r3, bf16hi(y.y)));
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
