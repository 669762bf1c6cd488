// C ABI of the DART hot path: argument validation (host only, before any HIP
// call) and dispatch to the MFMA or general kernels.  See include/dart.h for
// the contract of every entry point.
#include "dart.h"

#include <stdarg.h>
#include <stdint.h>
#include <math.h>
#include <stdio.h>

#include <initializer_list>

#include "dart_internal.h"

namespace {

thread_local char t_err[512] = "";
thread_local int t_path = DART_PATH_AUTO;

constexpr int64_t kMaxDim = 256;          // N, P limit of the general kernels
constexpr int64_t kMaxIndex = INT64_C(1) << 31;  // grid and per-call index limits

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_err, sizeof(t_err), fmt, ap);
  va_end(ap);
  return code;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Product of the given non-negative factors, or -1 on overflow.
int64_t prod(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs)
    if (!mul_ok(r, x, &r)) return -1;
  return r;
}

struct Buf {
  const void* p;
  int64_t bytes;
  const char* name;
};

int check_ptrs(std::initializer_list<Buf> req) {
  for (const Buf& b : req) {
    if (b.p == nullptr) return fail(DART_ERR_NULL, "%s is NULL", b.name);
    if (((uintptr_t)b.p & 15u) != 0) return fail(DART_ERR_ALIGN, "%s is not 16-byte aligned", b.name);
  }
  return DART_OK;
}

int check_opt_align(const void* p, const char* name) {
  if (p != nullptr && ((uintptr_t)p & 15u) != 0)
    return fail(DART_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return DART_OK;
}

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
  return a0 < b1 && b0 < a1;
}

// `outs` must not overlap each other or any of `ins`, except `allowed_alias`
// (out == Y_ssm, identical pointer).
int check_alias(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins,
                const void* alias_out, const void* alias_in) {
  for (const Buf& o : outs) {
    for (const Buf& i : ins) {
      if (o.p == alias_out && i.p == alias_in && o.p == i.p) continue;
      if (overlap(o, i)) return fail(DART_ERR_SHAPE, "output %s overlaps input %s", o.name, i.name);
    }
    for (const Buf& o2 : outs)
      if (&o2 < &o && overlap(o, o2)) return fail(DART_ERR_SHAPE, "outputs %s and %s overlap", o.name, o2.name);
  }
  return DART_OK;
}

// Common dimension checks.  need_seq: seqlen and chunk are used.
int check_dims(const dart_dims_t* d, int dtype, bool need_seq) {
  if (d == nullptr) return fail(DART_ERR_NULL, "dims is NULL");
  if (dtype != DART_F32 && dtype != DART_BF16)
    return fail(DART_ERR_UNSUPPORTED, "dtype %d is not DART_F32 or DART_BF16", dtype);
  if (d->batch < 0) return fail(DART_ERR_SHAPE, "batch = %lld < 0", (long long)d->batch);
  if (need_seq && d->seqlen < 0) return fail(DART_ERR_SHAPE, "seqlen = %lld < 0", (long long)d->seqlen);
  if (d->nheads <= 0) return fail(DART_ERR_SHAPE, "nheads = %lld must be > 0", (long long)d->nheads);
  if (d->ngroups <= 0) return fail(DART_ERR_SHAPE, "ngroups = %lld must be > 0", (long long)d->ngroups);
  if (d->nheads % d->ngroups != 0)
    return fail(DART_ERR_SHAPE, "ngroups = %lld does not divide nheads = %lld", (long long)d->ngroups,
                (long long)d->nheads);
  if (d->d_state <= 0) return fail(DART_ERR_SHAPE, "d_state = %lld must be > 0", (long long)d->d_state);
  if (d->d_head <= 0) return fail(DART_ERR_SHAPE, "d_head = %lld must be > 0", (long long)d->d_head);
  if (need_seq && d->chunk <= 0) return fail(DART_ERR_SHAPE, "chunk = %lld must be > 0", (long long)d->chunk);
  if (d->d_state > kMaxDim || d->d_head > kMaxDim)
    return fail(DART_ERR_UNSUPPORTED, "d_state = %lld, d_head = %lld: both must be <= %lld",
                (long long)d->d_state, (long long)d->d_head, (long long)kMaxDim);
  if (need_seq && d->seqlen >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "seqlen = %lld must be < 2^31", (long long)d->seqlen);
  const int64_t rows = prod({d->batch, need_seq ? d->seqlen : 1, d->nheads, kMaxDim, kMaxDim});
  if (rows < 0 || rows > INT64_MAX / 16) return fail(DART_ERR_SHAPE, "problem size overflows 64-bit indexing");
  return DART_OK;
}

dart::Shape make_shape(const dart_dims_t* d) {
  dart::Shape s;
  s.b = d->batch;
  s.L = d->seqlen;
  s.H = d->nheads;
  s.G = d->ngroups;
  s.N = d->d_state;
  s.P = d->d_head;
  // A chunk longer than the sequence behaves as one chunk of length L.
  s.S = (d->chunk > d->seqlen && d->seqlen > 0) ? d->seqlen : d->chunk;
  s.M = s.S > 0 ? (s.L + s.S - 1) / s.S : 0;
  return s;
}

size_t bwd_workspace(const dart::Shape& s) {
  const size_t g = dart::sma_bwd_workspace_bytes(s), m = dart::sma_bwd_mfma_workspace_bytes(s);
  return g > m ? g : m;
}

// The MFMA kernels address a token tile (up to 256 rows of nheads * P or
// ngroups * N elements) and a head's per-chunk weight rows (8 seqlen bytes)
// with 32-bit buffer offsets; these bounds keep every such offset below 2^31.
// Larger shapes run the general kernels, which index in 64 bits.
constexpr int64_t kMfmaMaxHeads = 4096;
constexpr int64_t kMfmaMaxSeq = (int64_t)1 << 28;

bool use_mfma(int dtype, const dart_dims_t* d) {
  return t_path == DART_PATH_AUTO && dtype == DART_BF16 && d->d_state == 128 && d->d_head == 64 &&
         d->nheads <= kMfmaMaxHeads && d->ngroups <= kMfmaMaxHeads && d->seqlen < kMfmaMaxSeq;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DART_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DART_OK;
}

}  // namespace

extern "C" {

int dart_abi_version(void) { return DART_ABI_VERSION; }

const char* dart_last_error(void) { return t_err; }

int dart_set_path(int path) {
  const int prev = t_path;
  t_path = (path == DART_PATH_GENERAL) ? DART_PATH_GENERAL : DART_PATH_AUTO;
  return prev;
}

const char* dart_status_string(int status) {
  switch (status) {
    case DART_OK: return "DART_OK";
    case DART_ERR_NULL: return "DART_ERR_NULL";
    case DART_ERR_SHAPE: return "DART_ERR_SHAPE";
    case DART_ERR_UNSUPPORTED: return "DART_ERR_UNSUPPORTED";
    case DART_ERR_WORKSPACE: return "DART_ERR_WORKSPACE";
    case DART_ERR_HIP: return "DART_ERR_HIP";
    case DART_ERR_ALIGN: return "DART_ERR_ALIGN";
    default: return "DART_ERR_UNKNOWN";
  }
}

int dart_chunk_states(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                      const float* A, void* dH, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bx{X, prod({s.b, s.L, s.H, s.P}) * es, "X"};
  const Buf bb{B, prod({s.b, s.L, s.G, s.N}) * es, "B"};
  const Buf ba{A, prod({s.b, s.L, s.H}) * 4, "A"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  if ((st = check_ptrs({bx, bb, ba, bd}))) return st;
  if ((st = check_alias({bd}, {bx, bb, ba}, nullptr, nullptr))) return st;
  const int64_t tiles = (s.N * s.P + 255) / 256;
  if (prod({s.b, s.H, s.M, tiles}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H * M is too large for one launch");
  hipStream_t strm = (hipStream_t)stream;
  if (use_mfma(dtype, dims))
    return hip_status(dart::launch_chunk_states_mfma(s, X, B, A, dH, strm), "dart_chunk_states");
  return hip_status(dart::launch_chunk_states_general(s, dtype == DART_BF16, X, B, A, dH, strm),
                    "dart_chunk_states");
}

}  // extern "C"

namespace {

// dart_sma_fwd and dart_sma_fwd_rms (rms: dHs is the score memory).
int sma_fwd_impl(const dart_dims_t* dims, int dtype, bool rms, float eps, const void* Q, const void* C,
                 const void* E, const void* dH, const void* dHs, const void* Y_ssm, const void* gate,
                 int gate_per_channel, void* out, float* R, float* lse, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  if (rms && !(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const int gpc = gate_per_channel ? 1 : 0;
  const Buf bq{Q, prod({s.b, s.L, s.G, s.N}) * es, "Q"};
  const Buf bc{C, prod({s.b, s.L, s.G, s.N}) * es, "C"};
  const Buf be{E, prod({s.b, s.L, s.G, s.P}) * es, "E"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bs{dHs, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH_score"};
  const Buf by{Y_ssm, prod({s.b, s.L, s.H, s.P}) * es, "Y_ssm"};
  const Buf bg{gate, prod({s.b, s.L, s.H, gpc ? s.P : 1}) * es, "gate"};
  const Buf bo{out, prod({s.b, s.L, s.H, s.P}) * es, "out"};
  const Buf br{R, prod({s.b, s.L, s.H, s.P}) * 4, "R"};
  const Buf bl{lse, prod({s.b, s.H, s.L}) * 4, "lse"};
  if ((st = check_ptrs({bq, bc, be, bd, by, bg, bo}))) return st;
  if (rms && (st = check_ptrs({bs}))) return st;
  if ((st = check_opt_align(R, "R")) || (st = check_opt_align(lse, "lse"))) return st;
  if ((st = check_alias({bo, br, bl}, {bq, bc, be, bd, by, bg, rms ? bs : Buf{nullptr, 0, ""}}, out, Y_ssm)))
    return st;
  if (prod({s.b, s.H, (s.L + 3) / 4}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H * L is too large for one launch");
  hipStream_t strm = (hipStream_t)stream;
  const bool bf16 = dtype == DART_BF16;
  if (rms && use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_fwd_rms_mfma(s, eps, Q, C, E, dH, dHs, Y_ssm, gate, gpc, out, R, lse,
                                                    strm),
                      "dart_sma_fwd_rms");
  if (rms)
    return hip_status(dart::launch_sma_fwd_rms_general(s, bf16, eps, Q, C, E, dH, dHs, Y_ssm, gate, gpc, out,
                                                       R, lse, strm),
                      "dart_sma_fwd_rms");
  if (use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_fwd_mfma(s, Q, C, E, dH, Y_ssm, gate, gpc, out, R, lse, strm),
                      "dart_sma_fwd");
  return hip_status(dart::launch_sma_fwd_general(s, bf16, Q, C, E, dH, Y_ssm, gate, gpc, out, R, lse, strm),
                    "dart_sma_fwd");
}

// Weights of an RMSNorm: NULL or n float32 values at 4-byte alignment.
int check_weight(const float* w, const char* name) {
  if (w != nullptr && ((uintptr_t)w & 3u) != 0) return fail(DART_ERR_ALIGN, "%s is not 4-byte aligned", name);
  return DART_OK;
}

}  // namespace

extern "C" {

int dart_sma_fwd(const dart_dims_t* dims, int dtype, const void* Q, const void* C, const void* E,
                 const void* dH, const void* Y_ssm, const void* gate, int gate_per_channel,
                 void* out, float* R, float* lse, void* stream) {
  return sma_fwd_impl(dims, dtype, false, 0.f, Q, C, E, dH, nullptr, Y_ssm, gate, gate_per_channel, out, R,
                      lse, stream);
}

int dart_sma_fwd_rms(const dart_dims_t* dims, int dtype, const void* Q, const void* C,
                     const void* E, const void* dH, const void* dH_score, const void* Y_ssm,
                     const void* gate, int gate_per_channel, float eps, void* out, float* R,
                     float* lse, void* stream) {
  return sma_fwd_impl(dims, dtype, true, eps, Q, C, E, dH, dH_score, Y_ssm, gate, gate_per_channel, out, R,
                      lse, stream);
}

int dart_chunk_rms(const dart_dims_t* dims, int dtype, const void* dH, float eps, const float* w_q,
                   const float* w_e, float* r, void* dH_score, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  if (!(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bwq{w_q, s.N * 4, "w_q"};
  const Buf bwe{w_e, s.P * 4, "w_e"};
  const Buf br{r, prod({s.b, s.H, s.M, s.N}) * 4, "r"};
  const Buf bs{dH_score, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH_score"};
  if ((st = check_ptrs({bd}))) return st;
  if ((st = check_weight(w_q, "w_q")) || (st = check_weight(w_e, "w_e"))) return st;
  if ((st = check_opt_align(r, "r")) || (st = check_opt_align(dH_score, "dH_score"))) return st;
  if ((st = check_alias({br, bs}, {bd, bwq, bwe}, nullptr, nullptr))) return st;
  if (prod({s.b, s.H, s.M}) >= kMaxIndex) return fail(DART_ERR_SHAPE, "b * H * M is too large for one launch");
  if (r == nullptr && dH_score == nullptr) return DART_OK;
  return hip_status(dart::launch_chunk_rms(s, dtype == DART_BF16, eps, dH, w_q, w_e, r, dH_score,
                                           (hipStream_t)stream),
                    "dart_chunk_rms");
}

int dart_chunk_states_rms(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                          const float* A, float eps, const float* w_q, const float* w_e, void* dH,
                          float* r, void* dH_score, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  if (!(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bx{X, prod({s.b, s.L, s.H, s.P}) * es, "X"};
  const Buf bb{B, prod({s.b, s.L, s.G, s.N}) * es, "B"};
  const Buf ba{A, prod({s.b, s.L, s.H}) * 4, "A"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bwq{w_q, s.N * 4, "w_q"};
  const Buf bwe{w_e, s.P * 4, "w_e"};
  const Buf br{r, prod({s.b, s.H, s.M, s.N}) * 4, "r"};
  const Buf bs{dH_score, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH_score"};
  if ((st = check_ptrs({bx, bb, ba, bd}))) return st;
  if ((st = check_weight(w_q, "w_q")) || (st = check_weight(w_e, "w_e"))) return st;
  if ((st = check_opt_align(r, "r")) || (st = check_opt_align(dH_score, "dH_score"))) return st;
  if ((st = check_alias({bd, br, bs}, {bx, bb, ba, bwq, bwe}, nullptr, nullptr))) return st;
  const int64_t tiles = (s.N * s.P + 255) / 256;
  if (prod({s.b, s.H, s.M, tiles}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H * M is too large for one launch");
  hipStream_t strm = (hipStream_t)stream;
  const bool bf16 = dtype == DART_BF16;
  if (use_mfma(dtype, dims))  // r and the score memory come from the same kernel's epilogue
    return hip_status(dart::launch_chunk_states_mfma(s, X, B, A, dH, strm, eps, w_q, w_e, r, dH_score),
                      "dart_chunk_states_rms");
  st = hip_status(dart::launch_chunk_states_general(s, bf16, X, B, A, dH, strm), "dart_chunk_states_rms");
  if (st || (r == nullptr && dH_score == nullptr)) return st;
  return hip_status(dart::launch_chunk_rms(s, bf16, eps, dH, w_q, w_e, r, dH_score, strm),
                    "dart_chunk_states_rms");
}

size_t dart_sma_decode_workspace_bytes(const dart_dims_t* dims, int64_t max_chunks) {
  if (dims == nullptr || dims->batch < 0 || dims->nheads <= 0 || dims->d_head <= 0 || max_chunks < 0)
    return 0;
  if (prod({dims->batch, dims->nheads, max_chunks + 1, dims->d_head + 2}) < 0) return 0;
  return dart::decode_plan(dims->batch, dims->nheads, dims->d_head, max_chunks).workspace_bytes;
}

}  // extern "C"

namespace {

// dart_sma_decode, dart_sma_decode_rms (rms: r_cache and the weights) and
// dart_sma_decode_noalloc (noalloc: the library's scratch instead of the
// caller's workspace).
int sma_decode_impl(const dart_dims_t* dims, int dtype, int64_t max_chunks, bool rms, float eps,
                    const void* q, const void* c, const void* e, const void* cache, const float* r_cache,
                    const int32_t* n_chunks, const float* w_q, const float* w_e, const void* y_ssm,
                    const void* gate, int gate_per_channel, void* out, float* R, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream, bool noalloc = false) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, false);
  if (st) return st;
  if (rms && !(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  if (max_chunks < 0) return fail(DART_ERR_SHAPE, "max_chunks = %lld < 0", (long long)max_chunks);
  if (max_chunks >= kMaxIndex) return fail(DART_ERR_SHAPE, "max_chunks must be < 2^31");
  dart::Shape s = make_shape(dims);
  s.L = 1;
  s.S = 1;
  s.M = max_chunks;
  if (s.b == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const int gpc = gate_per_channel ? 1 : 0;
  const Buf bq{q, prod({s.b, s.G, s.N}) * es, "q"};
  const Buf bc{c, prod({s.b, s.G, s.N}) * es, "c"};
  const Buf be{e, prod({s.b, s.G, s.P}) * es, "e"};
  const Buf bk{cache, prod({s.b, s.H, max_chunks, s.P, s.N}) * es, "cache"};
  const Buf by{y_ssm, prod({s.b, s.H, s.P}) * es, "y_ssm"};
  const Buf bg{gate, prod({s.b, s.H, gpc ? s.P : 1}) * es, "gate"};
  const Buf bo{out, prod({s.b, s.H, s.P}) * es, "out"};
  const Buf br{R, prod({s.b, s.H, s.P}) * 4, "R"};
  const Buf bl{lse, prod({s.b, s.H}) * 4, "lse"};
  const dart::DecodePlan plan = dart::decode_plan(s.b, s.H, s.P, max_chunks);
  const Buf bw{workspace, (int64_t)plan.workspace_bytes, "workspace"};
  const Buf brc{r_cache, prod({s.b, s.H, max_chunks, s.N}) * 4, "r_cache"};
  const Buf bwq{w_q, s.N * 4, "w_q"};
  const Buf bwe{w_e, s.P * 4, "w_e"};
  if (max_chunks > 0 && cache == nullptr) return fail(DART_ERR_NULL, "cache is NULL");
  if (rms && max_chunks > 0 && r_cache == nullptr) return fail(DART_ERR_NULL, "r_cache is NULL");
  if (rms && ((st = check_opt_align(r_cache, "r_cache")) || (st = check_weight(w_q, "w_q")) ||
              (st = check_weight(w_e, "w_e"))))
    return st;
  // a scalar gate is read one element at a time: its element's alignment suffices
  if ((st = check_ptrs({bq, bc, be, by}))) return st;
  if (gpc && (st = check_ptrs({bg}))) return st;
  if (!gpc) {
    if (gate == nullptr) return fail(DART_ERR_NULL, "gate is NULL");
    if (((uintptr_t)gate % (uintptr_t)es) != 0)
      return fail(DART_ERR_ALIGN, "gate is not aligned to its element size");
  }
  if ((st = check_ptrs({bo}))) return st;
  if ((st = check_opt_align(cache, "cache")) || (st = check_opt_align(R, "R")) ||
      (st = check_opt_align(lse, "lse")) || (st = check_opt_align(n_chunks, "n_chunks")))
    return st;
  if (noalloc) {
    if (plan.workspace_bytes > DART_DECODE_SCRATCH_BYTES)
      return fail(DART_ERR_WORKSPACE, "the split partials need %zu bytes, more than the %zu-byte scratch of "
                  "dart_sma_decode_noalloc; use dart_sma_decode with a workspace", plan.workspace_bytes,
                  (size_t)DART_DECODE_SCRATCH_BYTES);
  } else {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes)
      return fail(DART_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                  plan.workspace_bytes);
    if ((st = check_opt_align(workspace, "workspace"))) return st;
  }
  const Buf bn{n_chunks, s.b * 4, "n_chunks"};
  if ((st = check_alias({bo, br, bl, bw}, {bq, bc, be, bk, by, bg, bn, brc, bwq, bwe}, out, y_ssm))) return st;
  if (prod({s.b, s.H, plan.splits}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H is too large for one launch");
  if (noalloc) {
    float* scratch = nullptr;
    if ((st = hip_status(dart::decode_scratch(&scratch), "dart_sma_decode_noalloc scratch"))) return st;
    workspace = scratch;
  }
  hipStream_t strm = (hipStream_t)stream;
  if (rms && use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_decode_mfma(s, max_chunks, plan, q, c, e, cache, n_chunks, y_ssm, gate,
                                                   gpc, out, R, lse, (float*)workspace, r_cache, w_q, w_e,
                                                   eps, strm),
                      "dart_sma_decode_rms");
  if (rms)
    return hip_status(dart::launch_sma_decode_rms_general(s, dtype == DART_BF16, max_chunks, eps, q, c, e,
                                                          cache, r_cache, n_chunks, w_q, w_e, y_ssm, gate,
                                                          gpc, out, R, lse, strm),
                      "dart_sma_decode_rms");
  if (use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_decode_mfma(s, max_chunks, plan, q, c, e, cache, n_chunks, y_ssm,
                                                   gate, gpc, out, R, lse, (float*)workspace, nullptr,
                                                   nullptr, nullptr, 0.f, strm),
                      "dart_sma_decode");
  return hip_status(dart::launch_sma_decode_general(s, dtype == DART_BF16, max_chunks, q, c, e, cache,
                                                    n_chunks, y_ssm, gate, gpc, out, R, lse, strm),
                    "dart_sma_decode");
}

}  // namespace

extern "C" {

int dart_sma_decode(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                    const void* c, const void* e, const void* cache, const int32_t* n_chunks,
                    const void* y_ssm, const void* gate, int gate_per_channel, void* out,
                    float* R, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return sma_decode_impl(dims, dtype, max_chunks, false, 0.f, q, c, e, cache, nullptr, n_chunks, nullptr,
                         nullptr, y_ssm, gate, gate_per_channel, out, R, lse, workspace, workspace_bytes,
                         stream);
}

int dart_sma_decode_noalloc(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                            const void* c, const void* e, const void* cache, const int32_t* n_chunks,
                            const void* y_ssm, const void* gate, int gate_per_channel, void* out,
                            float* R, float* lse, void* stream) {
  return sma_decode_impl(dims, dtype, max_chunks, false, 0.f, q, c, e, cache, nullptr, n_chunks, nullptr,
                         nullptr, y_ssm, gate, gate_per_channel, out, R, lse, nullptr, 0, stream, true);
}

int dart_sma_decode_rms(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                        const void* c, const void* e, const void* cache, const float* r_cache,
                        const int32_t* n_chunks, const void* y_ssm, const void* gate,
                        int gate_per_channel, float eps, const float* w_q, const float* w_e,
                        void* out, float* R, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return sma_decode_impl(dims, dtype, max_chunks, true, eps, q, c, e, cache, r_cache, n_chunks, w_q, w_e,
                         y_ssm, gate, gate_per_channel, out, R, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int decode_update_impl(const dart_dims_t* dims, int dtype, int64_t max_chunks, bool rms, float eps,
                       const void* x, const void* B, const float* a, float* state, const int32_t* pos,
                       void* cache, float* r_cache, int32_t* n_chunks, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, false);
  if (st) return st;
  if (rms && !(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  if (dims->chunk <= 0) return fail(DART_ERR_SHAPE, "chunk = %lld must be > 0", (long long)dims->chunk);
  if (max_chunks < 0) return fail(DART_ERR_SHAPE, "max_chunks = %lld < 0", (long long)max_chunks);
  if (max_chunks >= kMaxIndex) return fail(DART_ERR_SHAPE, "max_chunks must be < 2^31");
  dart::Shape s = make_shape(dims);
  s.L = 1;
  s.S = dims->chunk;
  s.M = max_chunks;
  if (s.b == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bx{x, prod({s.b, s.H, s.P}) * es, "x"};
  const Buf bb{B, prod({s.b, s.G, s.N}) * es, "B"};
  const Buf ba{a, prod({s.b, s.H}) * 4, "a"};
  const Buf bs{state, prod({s.b, s.H, s.P, s.N}) * 4, "state"};
  const Buf bp{pos, s.b * 4, "pos"};
  const Buf bk{cache, prod({s.b, s.H, max_chunks, s.P, s.N}) * es, "cache"};
  const Buf bn{n_chunks, s.b * 4, "n_chunks"};
  const Buf brc{r_cache, prod({s.b, s.H, max_chunks, s.N}) * 4, "r_cache"};
  // x, B, a, pos are read element by element: per-token slices of larger
  // tensors are accepted at element alignment; state and cache are accessed
  // in 16-byte vectors.
  for (const Buf& e : {bx, bb, ba, bp}) {
    if (e.p == nullptr) return fail(DART_ERR_NULL, "%s is NULL", e.name);
    const uintptr_t al = (e.p == x || e.p == B) ? (uintptr_t)es : 4u;
    if (((uintptr_t)e.p & (al - 1)) != 0)
      return fail(DART_ERR_ALIGN, "%s is not %d-byte aligned", e.name, (int)al);
  }
  if ((st = check_ptrs({bs}))) return st;
  if (max_chunks > 0 && cache == nullptr) return fail(DART_ERR_NULL, "cache is NULL");
  if ((st = check_opt_align(cache, "cache"))) return st;
  if (rms && max_chunks > 0 && r_cache == nullptr) return fail(DART_ERR_NULL, "r_cache is NULL");
  if (rms && (st = check_opt_align(r_cache, "r_cache"))) return st;
  if (n_chunks != nullptr && ((uintptr_t)n_chunks & 3u) != 0)
    return fail(DART_ERR_ALIGN, "n_chunks is not 4-byte aligned");
  if ((st = check_alias({bs, bk, bn, rms ? brc : Buf{nullptr, 0, ""}}, {bx, bb, ba, bp}, nullptr, nullptr)))
    return st;
  if (prod({s.b, s.H}) >= kMaxIndex) return fail(DART_ERR_SHAPE, "b * H is too large for one launch");
  return hip_status(dart::launch_decode_update(s, dtype == DART_BF16, max_chunks, x, B, a, state, pos,
                                               cache, n_chunks, rms ? r_cache : nullptr, eps,
                                               (hipStream_t)stream),
                    rms ? "dart_decode_state_update_rms" : "dart_decode_state_update");
}

}  // namespace

extern "C" {

int dart_decode_state_update(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* x,
                             const void* B, const float* a, float* state, const int32_t* pos,
                             void* cache, int32_t* n_chunks, void* stream) {
  return decode_update_impl(dims, dtype, max_chunks, false, 0.f, x, B, a, state, pos, cache, nullptr,
                            n_chunks, stream);
}

int dart_decode_state_update_rms(const dart_dims_t* dims, int dtype, int64_t max_chunks, float eps,
                                 const void* x, const void* B, const float* a, float* state,
                                 const int32_t* pos, void* cache, float* r_cache, int32_t* n_chunks,
                                 void* stream) {
  return decode_update_impl(dims, dtype, max_chunks, true, eps, x, B, a, state, pos, cache, r_cache,
                            n_chunks, stream);
}

size_t dart_ssd_fwd_workspace_bytes(const dart_dims_t* dims, int dtype) {
  t_err[0] = '\0';
  if (dims == nullptr || check_dims(dims, dtype, true) != DART_OK) return 0;
  const dart::Shape s = make_shape(dims);
  if (prod({s.b, s.H, s.M, s.P, s.N, 4}) < 0) return 0;
  return dart::ssd_workspace_bytes(s, dtype == DART_BF16);
}

int dart_ssd_fwd(const dart_dims_t* dims, int dtype, const void* X, const void* B, const void* C,
                 const float* A, const float* H0, void* Y, void* dH, float* H_final, void* workspace,
                 size_t workspace_bytes, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bx{X, prod({s.b, s.L, s.H, s.P}) * es, "X"};
  const Buf bb{B, prod({s.b, s.L, s.G, s.N}) * es, "B"};
  const Buf bc{C, prod({s.b, s.L, s.G, s.N}) * es, "C"};
  const Buf ba{A, prod({s.b, s.L, s.H}) * 4, "A"};
  const Buf b0{H0, prod({s.b, s.H, s.P, s.N}) * 4, "H0"};
  const Buf by{Y, prod({s.b, s.L, s.H, s.P}) * es, "Y"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bf{H_final, prod({s.b, s.H, s.P, s.N}) * 4, "H_final"};
  const size_t need = dart::ssd_workspace_bytes(s, dtype == DART_BF16);
  const Buf bw{workspace, (int64_t)need, "workspace"};
  if ((st = check_ptrs({bx, bb, bc, ba, by, bd}))) return st;
  if ((st = check_opt_align(H0, "H0")) || (st = check_opt_align(H_final, "H_final"))) return st;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DART_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((st = check_opt_align(workspace, "workspace"))) return st;
  if ((st = check_alias({by, bd, bf, bw}, {bx, bb, bc, ba, b0}, nullptr, nullptr))) return st;
  if (prod({s.b, s.H, s.M, (s.N * s.P + 255) / 256}) >= kMaxIndex || prod({s.b, s.H, (s.L + 3) / 4}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "problem is too large for one launch");
  return hip_status(dart::launch_ssd_fwd(s, dtype == DART_BF16, use_mfma(dtype, dims), X, B, C, A, H0, Y, dH,
                                         H_final, workspace, (hipStream_t)stream),
                    "dart_ssd_fwd");
}

size_t dart_sma_bwd_workspace_bytes(const dart_dims_t* dims) {
  t_err[0] = '\0';
  if (dims == nullptr || check_dims(dims, DART_F32, true) != DART_OK) return 0;
  const dart::Shape s = make_shape(dims);
  if (prod({2, s.b, s.H, s.M, s.L}) < 0 || prod({s.b, s.L, s.H, 2 * s.N + s.P}) < 0) return 0;
  return bwd_workspace(s);
}

int dart_sma_bwd(const dart_dims_t* dims, int dtype, const void* Q, const void* C, const void* E,
                 const void* dH, const void* gate, int gate_per_channel, const float* R,
                 const float* lse, const void* dout, float* dQ, float* dC, float* dE, float* d_dH,
                 float* dgate, void* workspace, size_t workspace_bytes, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const int gpc = gate_per_channel ? 1 : 0;
  const Buf bq{Q, prod({s.b, s.L, s.G, s.N}) * es, "Q"};
  const Buf bc{C, prod({s.b, s.L, s.G, s.N}) * es, "C"};
  const Buf be{E, prod({s.b, s.L, s.G, s.P}) * es, "E"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bg{gate, prod({s.b, s.L, s.H, gpc ? s.P : 1}) * es, "gate"};
  const Buf br{R, prod({s.b, s.L, s.H, s.P}) * 4, "R"};
  const Buf bl{lse, prod({s.b, s.H, s.L}) * 4, "lse"};
  const Buf bo{dout, prod({s.b, s.L, s.H, s.P}) * es, "dout"};
  const Buf gq{dQ, prod({s.b, s.L, s.G, s.N}) * 4, "dQ"};
  const Buf gc{dC, prod({s.b, s.L, s.G, s.N}) * 4, "dC"};
  const Buf ge{dE, prod({s.b, s.L, s.G, s.P}) * 4, "dE"};
  const Buf gd{d_dH, prod({s.b, s.H, s.M, s.P, s.N}) * 4, "d_dH"};
  const Buf gg{dgate, prod({s.b, s.L, s.H, gpc ? s.P : 1}) * 4, "dgate"};
  const size_t need = bwd_workspace(s);
  const Buf bw{workspace, (int64_t)need, "workspace"};
  if ((st = check_ptrs({bq, bc, be, bd, bg, br, bl, bo, gq, gc, ge, gd}))) return st;
  if ((st = check_opt_align(dgate, "dgate"))) return st;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DART_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((st = check_opt_align(workspace, "workspace"))) return st;
  if ((st = check_alias({gq, gc, ge, gd, gg, bw}, {bq, bc, be, bd, bg, br, bl, bo}, nullptr, nullptr)))
    return st;
  if (prod({s.b, s.H, s.M, (s.N * s.P + 255) / 256}) >= kMaxIndex || prod({s.b, s.H, (s.L + 3) / 4}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H * M or b * H * L is too large for one launch");
  hipStream_t strm = (hipStream_t)stream;
  if (use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_bwd_mfma(s, Q, C, E, dH, gate, gpc, R, lse, dout, dQ, dC, dE, d_dH,
                                                dgate, workspace, strm),
                      "dart_sma_bwd");
  return hip_status(dart::launch_sma_bwd_general(s, dtype == DART_BF16, Q, C, E, dH, gate, gpc, R, lse,
                                                 dout, dQ, dC, dE, d_dH, dgate, (float*)workspace, strm),
                    "dart_sma_bwd");
}

size_t dart_sma_bwd_rms_workspace_bytes(const dart_dims_t* dims) {
  t_err[0] = '\0';
  if (dims == nullptr || check_dims(dims, DART_F32, true) != DART_OK) return 0;
  const dart::Shape s = make_shape(dims);
  if (prod({2, s.b, s.H, s.M, s.L}) < 0 || prod({3, s.b, s.L, s.H, s.N + s.P}) < 0 ||
      prod({2, s.b, s.H, s.M, s.P, s.N}) < 0)
    return 0;
  const size_t g = dart::sma_bwd_rms_workspace_bytes(s), m = dart::sma_bwd_rms_mfma_workspace_bytes(s);
  return g > m ? g : m;
}

int dart_sma_bwd_rms(const dart_dims_t* dims, int dtype, const void* Q, const void* C,
                     const void* E, const void* dH, const void* dH_score, const void* gate,
                     int gate_per_channel, float eps, const float* w_q, const float* w_e,
                     const float* R, const float* lse, const void* dout, float* dQ, float* dC,
                     float* dE, float* d_dH, float* dgate, float* dw_q, float* dw_e,
                     void* workspace, size_t workspace_bytes, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  if (!(eps >= 0.f && eps < INFINITY)) return fail(DART_ERR_SHAPE, "eps must be finite and >= 0");
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const int gpc = gate_per_channel ? 1 : 0;
  const Buf bq{Q, prod({s.b, s.L, s.G, s.N}) * es, "Q"};
  const Buf bc{C, prod({s.b, s.L, s.G, s.N}) * es, "C"};
  const Buf be{E, prod({s.b, s.L, s.G, s.P}) * es, "E"};
  const Buf bd{dH, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH"};
  const Buf bs{dH_score, prod({s.b, s.H, s.M, s.P, s.N}) * es, "dH_score"};
  const Buf bg{gate, prod({s.b, s.L, s.H, gpc ? s.P : 1}) * es, "gate"};
  const Buf bwq{w_q, s.N * 4, "w_q"};
  const Buf bwe{w_e, s.P * 4, "w_e"};
  const Buf br{R, prod({s.b, s.L, s.H, s.P}) * 4, "R"};
  const Buf bl{lse, prod({s.b, s.H, s.L}) * 4, "lse"};
  const Buf bo{dout, prod({s.b, s.L, s.H, s.P}) * es, "dout"};
  const Buf gq{dQ, prod({s.b, s.L, s.G, s.N}) * 4, "dQ"};
  const Buf gc{dC, prod({s.b, s.L, s.G, s.N}) * 4, "dC"};
  const Buf ge{dE, prod({s.b, s.L, s.G, s.P}) * 4, "dE"};
  const Buf gd{d_dH, prod({s.b, s.H, s.M, s.P, s.N}) * 4, "d_dH"};
  const Buf gg{dgate, prod({s.b, s.L, s.H, gpc ? s.P : 1}) * 4, "dgate"};
  const Buf gwq{dw_q, s.N * 4, "dw_q"};
  const Buf gwe{dw_e, s.P * 4, "dw_e"};
  const size_t gneed = dart::sma_bwd_rms_workspace_bytes(s), mneed = dart::sma_bwd_rms_mfma_workspace_bytes(s);
  const size_t need = gneed > mneed ? gneed : mneed;
  const Buf bw{workspace, (int64_t)need, "workspace"};
  if ((st = check_ptrs({bq, bc, be, bd, bs, bg, br, bl, bo, gq, gc, ge, gd}))) return st;
  if ((st = check_opt_align(dgate, "dgate"))) return st;
  if ((st = check_weight(w_q, "w_q")) || (st = check_weight(w_e, "w_e")) || (st = check_weight(dw_q, "dw_q")) ||
      (st = check_weight(dw_e, "dw_e")))
    return st;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DART_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((st = check_opt_align(workspace, "workspace"))) return st;
  if ((st = check_alias({gq, gc, ge, gd, gg, gwq, gwe, bw}, {bq, bc, be, bd, bs, bg, bwq, bwe, br, bl, bo},
                        nullptr, nullptr)))
    return st;
  if (prod({s.b, s.H, s.M, (s.N * s.P + 255) / 256}) >= kMaxIndex || prod({s.b, s.H, (s.L + 3) / 4}) >= kMaxIndex ||
      prod({s.b, s.H, s.M}) >= kMaxIndex || prod({s.b, s.H, s.M, s.N}) / 256 >= kMaxIndex ||
      prod({s.b, s.L, s.G}) / 4 >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "b * H * M or b * H * L is too large for one launch");
  if (use_mfma(dtype, dims))
    return hip_status(dart::launch_sma_bwd_rms_mfma(s, eps, Q, C, E, dH, dH_score, w_q, w_e, gate, gpc, R, lse,
                                                    dout, dQ, dC, dE, d_dH, dgate, dw_q, dw_e, workspace,
                                                    (hipStream_t)stream),
                      "dart_sma_bwd_rms");
  return hip_status(dart::launch_sma_bwd_rms_general(s, dtype == DART_BF16, eps, Q, C, E, dH, dH_score, w_q,
                                                     w_e, gate, gpc, R, lse, dout, dQ, dC, dE, d_dH, dgate,
                                                     dw_q, dw_e, (float*)workspace, (hipStream_t)stream),
                    "dart_sma_bwd_rms");
}

size_t dart_chunk_states_bwd_workspace_bytes(const dart_dims_t* dims) {
  t_err[0] = '\0';
  if (dims == nullptr || check_dims(dims, DART_F32, true) != DART_OK) return 0;
  const dart::Shape s = make_shape(dims);
  if (prod({2, s.b, s.H, s.L}) < 0 || prod({s.b, s.L, s.H, s.N}) < 0) return 0;
  return dart::chunk_states_bwd_workspace_bytes(s);
}

int dart_chunk_states_bwd(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                          const float* A, const float* d_dH, float* dX, float* dB, float* dA,
                          void* workspace, size_t workspace_bytes, void* stream) {
  t_err[0] = '\0';
  int st = check_dims(dims, dtype, true);
  if (st) return st;
  const dart::Shape s = make_shape(dims);
  if (s.b == 0 || s.L == 0) return DART_OK;
  const int64_t es = dtype == DART_BF16 ? 2 : 4;
  const Buf bx{X, prod({s.b, s.L, s.H, s.P}) * es, "X"};
  const Buf bb{B, prod({s.b, s.L, s.G, s.N}) * es, "B"};
  const Buf ba{A, prod({s.b, s.L, s.H}) * 4, "A"};
  const Buf bd{d_dH, prod({s.b, s.H, s.M, s.P, s.N}) * 4, "d_dH"};
  const Buf gx{dX, prod({s.b, s.L, s.H, s.P}) * 4, "dX"};
  const Buf gb{dB, prod({s.b, s.L, s.G, s.N}) * 4, "dB"};
  const Buf ga{dA, prod({s.b, s.L, s.H}) * 4, "dA"};
  const size_t need = dart::chunk_states_bwd_workspace_bytes(s);
  const Buf bw{workspace, (int64_t)need, "workspace"};
  if ((st = check_ptrs({bx, bb, ba, bd, gx, gb, ga}))) return st;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DART_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if ((st = check_opt_align(workspace, "workspace"))) return st;
  if ((st = check_alias({gx, gb, ga, bw}, {bx, bb, ba, bd}, nullptr, nullptr))) return st;
  if (prod({s.b, s.H, s.M}) >= kMaxIndex || prod({s.b, s.L, s.G, s.N}) >= kMaxIndex)
    return fail(DART_ERR_SHAPE, "problem is too large for one launch");
  hipStream_t strm = (hipStream_t)stream;
  return hip_status(dart::launch_chunk_states_bwd_general(s, dtype == DART_BF16, use_mfma(dtype, dims), X, B,
                                                          A, d_dH, dX, dB, dA, (float*)workspace, strm),
                    "dart_chunk_states_bwd");
}

}  // extern "C"
