/*
 * dart.h -- C ABI of the DART hot path on AMD Instinct MI355X (gfx950).
 *
 * The library computes the data-parallel hot path of
 *   "DART: Decoded Attention over Recurrent States for Efficient Long-Context
 *    Sequence Modeling" (arXiv 2608.02032):
 *   - chunk state memories            dart_chunk_states   [§3 Eq. 5; App. A Eq. 20]
 *   - state-memory attention (SMA)    dart_sma_fwd        [§3 Eq. 8-11; §4 Algorithm 1]
 *     with the gated residual
 *   - SMA for one new token against   dart_sma_decode     [§4 "Inference Cache"]
 *     a cache of chunk memories
 *   - decode-side cache maintenance   dart_decode_state_update  [§2 Eq. 2; §4]
 *   - gradients of the SMA branch     dart_sma_bwd        [§4 "Efficient Training";
 *     and of the chunk states         dart_chunk_states_bwd   App. C Eq. 33-35]
 *   - the SSM branch output by the    dart_ssd_fwd        [§2 Eq. 2; App. A Eq. 15-24]
 *     Mamba-2 chunked scan, with the
 *     chunk memories alongside
 *   - the RMS-normalised score        dart_chunk_states_rms, dart_chunk_rms,
 *     branch                          dart_sma_fwd_rms, dart_sma_decode_rms,
 *                                     dart_decode_state_update_rms
 *                                     [§3 text after Eq. 10; App. B.1 Eq. 25-27]
 *
 * Notation: b = batch, L = sequence length, H = heads, G = projection groups
 * (B, C, Q, E are shared by the H/G consecutive heads of a group; head h reads
 * group h / (H/G)) [§3 Fig. 2 caption; App. B.2], S = chunk size,
 * M = ceil(L/S) chunks, N = state size (key axis), P = head dim (value axis).
 * Tokens and chunks are 0-based: token t lies in chunk t / S.
 *
 * Memory layouts (all tensors dense, C order, innermost index last):
 *   X, Y_ssm, out           [b][L][H][P]      (dtype)
 *   R (optional)            [b][L][H][P]      float32
 *   B, C, Q                 [b][L][G][N]      (dtype)
 *   E                       [b][L][G][P]      (dtype)
 *   A (decay a_t)           [b][L][H]         float32, values in [0, 1]
 *   gate                    [b][L][H][P] if gate_per_channel, else [b][L][H]   (dtype)
 *   lse (optional)          [b][H][L]         float32
 *   dH (chunk memories)     [b][H][M][P][N]   (dtype)
 *       dH[b][h][c][p][n] holds entry (n, p) of the paper's N x P matrix
 *       dH_[c]: each memory is stored with its key axis N innermost.
 *
 * Ownership and execution:
 *   - Every data pointer is a device pointer on the current HIP device; the
 *     caller owns every buffer.  The library never allocates, frees or
 *     synchronises.
 *   - Every call validates its arguments on the host before any HIP call,
 *     then enqueues its kernels on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream) and returns without waiting.
 *   - Inputs are read only.  Outputs (including the optional R and lse) are
 *     fully overwritten.  `out` may alias `Y_ssm` (same pointer, same layout);
 *     no other aliasing is allowed.
 *   - Every pointer must be 16-byte aligned (dart_decode_state_update
 *     relaxes this for its per-token inputs, and the decode calls for a
 *     scalar gate; see there).
 *
 * Errors:
 *   - Calls return DART_OK (0) or a negative dart_status_t.  On failure the
 *     call launches nothing (argument errors) or stops at the failed launch
 *     (DART_ERR_HIP), and dart_last_error() returns a message for this
 *     thread's last failing call.
 *   - Faults inside a kernel surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.  The library keeps no global
 *     state beyond thread-local error text and path selection, so calls from
 *     several threads are safe.
 *
 * Supported shapes: dtype float32 or bfloat16 (all arithmetic in float32),
 * 1 <= N <= 256, 1 <= P <= 256, any S >= 1, any L (L % S != 0 allowed).
 * bfloat16 with N = 128 and P = 64 runs the MFMA kernels (for at most 4096
 * heads and groups and fewer than 2^28 tokens per sequence, bounds that keep
 * their 32-bit buffer offsets in range); every other case runs the general
 * kernels.  b = 0 or L = 0 is a valid empty call.
 */
#ifndef DART_H_
#define DART_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DART_ABI_VERSION 1

typedef enum { DART_F32 = 0, DART_BF16 = 1 } dart_dtype_t;

typedef enum {
  DART_OK = 0,
  DART_ERR_NULL = -1,        /* a required pointer is NULL */
  DART_ERR_SHAPE = -2,       /* a dimension is negative, zero where it must not be, or inconsistent */
  DART_ERR_UNSUPPORTED = -3, /* dtype or (N, P) outside the supported set */
  DART_ERR_WORKSPACE = -4,   /* decode workspace missing or too small */
  DART_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  DART_ERR_ALIGN = -6        /* a pointer is not 16-byte aligned */
} dart_status_t;

typedef struct {
  int64_t batch;   /* b */
  int64_t seqlen;  /* L */
  int64_t nheads;  /* H */
  int64_t ngroups; /* G, divides H */
  int64_t d_state; /* N */
  int64_t d_head;  /* P */
  int64_t chunk;   /* S */
} dart_dims_t;

/* Kernel selection for this thread: DART_PATH_AUTO picks the MFMA kernels
 * where supported; DART_PATH_GENERAL forces the general kernels everywhere
 * (used to cross-check the two on the GPU).  Returns the previous value. */
#define DART_PATH_AUTO 0
#define DART_PATH_GENERAL 1
int dart_set_path(int path);

/* Chunk state memories [§3 Eq. 5; App. A Eq. 20]:
 *   dH_[c] = sum_{s in chunk c} A_{s+1:e(c)} B_s^T X_s,
 *   A_{s+1:e(c)} = prod_{k=s+1}^{e(c)} a_k  (1 for the chunk's last token),
 * where e(c) is the last token actually in chunk c (a partial last chunk
 * decays to token L-1).  Accumulates in float32 and rounds once to dtype.
 *   X [b][L][H][P], B [b][L][G][N], A [b][L][H] -> dH [b][H][M][P][N]. */
int dart_chunk_states(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                      const float* A, void* dH, void* stream);

/* State-memory attention with the gated residual [§3 Eq. 8-11; §4 Algorithm 1]:
 * for every token t and every chunk c < chunk(t)
 *   V = C_t dH_c,  K = dH_c E_t,  l = Q_t K / sqrt(N),
 *   R_t = sum_c softmax_c(l) V  (R_t = 0 when chunk(t) = 0),
 *   lse_t = log sum_c exp(l)    (-inf when chunk(t) = 0),
 *   out_t = Y_ssm_t + g_t * R_t, g given after its activation.
 * R and lse are optional outputs (NULL skips them).  out is rounded once
 * from float32 to dtype. */
int dart_sma_fwd(const dart_dims_t* dims, int dtype, const void* Q, const void* C, const void* E,
                 const void* dH, const void* Y_ssm, const void* gate, int gate_per_channel,
                 void* out, float* R, float* lse, void* stream);

/* SMA for one new token per batch row against a chunk-memory cache
 * [§4 "Inference Cache"; §3 Eq. 8-11].  Every cached chunk 0..n_b-1 is
 * visible to the new token.  dims->seqlen and dims->chunk are ignored.
 *   q, c [b][G][N], e [b][G][P] (dtype)
 *   cache [b][H][max_chunks][P][N] (dtype; the dH layout above)
 *   n_chunks [b] int32 on the device, number of valid cached chunks per row,
 *            clamped to [0, max_chunks]; NULL means max_chunks for every row
 *   y_ssm, out [b][H][P] (dtype); gate [b][H][P] or [b][H] (dtype)
 *   R [b][H][P] float32 (optional), lse [b][H] float32 (optional)
 *   workspace: device scratch of at least dart_sma_decode_workspace_bytes()
 *              bytes; contents on entry are ignored.
 * A scalar gate ([b][H]) needs only its element's alignment, so the gate of
 * one token sliced from a [b][L][H] tensor is accepted as it is.
 * n_b = 0 gives R = 0, lse = -inf, out = y_ssm. */
int dart_sma_decode(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                    const void* c, const void* e, const void* cache, const int32_t* n_chunks,
                    const void* y_ssm, const void* gate, int gate_per_channel, void* out,
                    float* R, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dart_sma_decode needs for these dims and max_chunks
 * (0 on invalid dims; dtype does not matter). */
size_t dart_sma_decode_workspace_bytes(const dart_dims_t* dims, int64_t max_chunks);

/* dart_sma_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, results and kernels, without the workspace.  The
 * split partials go to a scratch array of DART_DECODE_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (its device
 * address is looked up once per device, on the first call there).  The call
 * allocates and frees nothing.
 *   Limit: dart_sma_decode_workspace_bytes(dims, max_chunks) must not exceed
 *   DART_DECODE_SCRATCH_BYTES (4 MiB: b * H up to about 15800 rows and heads
 *   at P = 64); larger problems fail with DART_ERR_WORKSPACE before any HIP
 *   call.
 *   Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *   that may overlap on one GPU (different streams, or threads without
 *   ordering between them) race; order them on one stream or use
 *   dart_sma_decode with a workspace each. */
#define DART_DECODE_SCRATCH_BYTES ((size_t)4 << 20)
int dart_sma_decode_noalloc(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                            const void* c, const void* e, const void* cache, const int32_t* n_chunks,
                            const void* y_ssm, const void* gate, int gate_per_channel, void* out,
                            float* R, float* lse, void* stream);

/* Decode-side cache maintenance, one new token per batch row [§2 Eq. 2
 * restricted to the current chunk; §3 Eq. 5 / App. A Eq. 20; §4 "Inference
 * Cache"].  For the token at absolute position pos[b] (chunk size S =
 * dims->chunk; dims->seqlen is ignored), every head of row b updates its
 * in-progress chunk memory
 *   state <- a * state + B^T x
 * and, when the token closes its chunk (pos % S == S - 1), writes the state,
 * rounded to dtype, to cache chunk pos / S and restarts the state from zero.
 * After the update n_chunks[b] = min((pos + 1) / S, max_chunks): the number of
 * complete chunks the next token's dart_sma_decode sees.
 *   x [b][H][P] (dtype)          B [b][G][N] (dtype)          a [b][H] float32
 *   state [b][H][P][N] float32   in/out; zero before a sequence's first token
 *   pos [b] int32 (device)       rows with pos < 0 are left untouched
 *   cache [b][H][max_chunks][P][N] (dtype)   written only at a chunk close;
 *                                a chunk index >= max_chunks is not written
 *   n_chunks [b] int32 (device)  written; NULL skips it
 * Alignment: state and cache 16 bytes; x, B, a, pos and n_chunks only their
 * element size (per-token slices of larger tensors are accepted). */
int dart_decode_state_update(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* x,
                             const void* B, const float* a, float* state, const int32_t* pos,
                             void* cache, int32_t* n_chunks, void* stream);

/* SMA backward with the gated residual [§3 Eq. 8-11 differentiated; §4
 * "Efficient Training"; App. C "Recomputation", Eq. 33-35].  For the loss
 * gradient dout of out = Y_ssm + g * R, every logit is recomputed and the
 * chunk weights are recovered from the forward's lse as p = exp(l - lse):
 *   dR_t = g_t * dout_t,  D_t = dR_t . R_t,  dl = p (dR_t . V_tc - D_t),
 *   dQ_t = sum_c dl dH_c E_t / sqrt(N),   dE_t = sum_c dl dH_c^T Q_t / sqrt(N),
 *   dC_t = sum_c p dH_c dR_t,
 *   d_dH_c = sum_{t: chunk(t) > c} p C_t^T dR_t + dl Q_t^T E_t / sqrt(N),
 *   dgate = dout * R (per channel) or sum_p dout * R (one gate per token).
 * The gradient of Y_ssm is dout itself and is not written.
 *   Inputs: the forward's Q, C, E, dH, gate (as for dart_sma_fwd), its
 *           outputs R [b][L][H][P] and lse [b][H][L] (float32), and
 *           dout [b][L][H][P] (dtype).
 *   Outputs, float32, fully overwritten: dQ, dC [b][L][G][N] and
 *           dE [b][L][G][P] (summed over the heads of a group); d_dH in the
 *           dH layout [b][H][M][P][N] (the last chunk, never read, gets 0);
 *           dgate shaped like gate (NULL skips it).
 *   workspace: device scratch of at least dart_sma_bwd_workspace_bytes()
 *           bytes; contents on entry are ignored. */
int dart_sma_bwd(const dart_dims_t* dims, int dtype, const void* Q, const void* C, const void* E,
                 const void* dH, const void* gate, int gate_per_channel, const float* R,
                 const float* lse, const void* dout, float* dQ, float* dC, float* dE, float* d_dH,
                 float* dgate, void* workspace, size_t workspace_bytes, void* stream);
size_t dart_sma_bwd_workspace_bytes(const dart_dims_t* dims);

/* Chunk-state backward [§3 Eq. 5 differentiated].  For d_dH (float32, the dH
 * layout [b][H][M][P][N]) and w_s = A_{s+1:e(c)}:
 *   dX_s = w_s B_s d_dH_c,   dB_s = w_s d_dH_c X_s^T (summed over the heads
 *   of a group),   dA_k = sum_{s<k in chunk(k)} (B_s d_dH_c X_s^T) dw_s/da_k,
 * which is 0 at a chunk's first token.
 *   Outputs, float32, fully overwritten: dX [b][L][H][P], dB [b][L][G][N],
 *   dA [b][L][H].  workspace: at least dart_chunk_states_bwd_workspace_bytes(). */
int dart_chunk_states_bwd(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                          const float* A, const float* d_dH, float* dX, float* dB, float* dA,
                          void* workspace, size_t workspace_bytes, void* stream);
size_t dart_chunk_states_bwd_workspace_bytes(const dart_dims_t* dims);

/* ---- RMS-normalised score branch [§3 text after Eq. 10; App. B.1 Eq. 25-27].
 * Only the logits change:
 *   l_tc = RMSNorm(Q_t) . (r_c * (dH_c RMSNorm(E_t))) / sqrt(N),
 *   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * w   (w: optional per-channel
 *                weight, w_q [N] for Q and w_e [P] for E, float32; NULL = 1),
 *   r_c[n] = (mean_p dH_c[n][p]^2 + eps)^(-1/2)   (inverse RMS of each key
 *                row of a chunk memory along the value axis, Eq. 26);
 * V = C_t dH_c, the softmax over chunks, lse and the gated residual are those
 * of dart_sma_fwd / dart_sma_decode.  One eps serves the two RMSNorms and r_c
 * (eps >= 0; with eps = 0 an all-zero key row gives r = inf).
 *
 * The forward consumes the chunk side of the normalisation precomputed once
 * per chunk, the score memory
 *   dHs_c[p][n] = w_e[p] * dH_c[p][n] * r_c[n] * w_q[n]    (dH layout),
 * stored in float16 for bfloat16 inputs (|entries| <= sqrt(P) max|w_q| max|w_e|,
 * and float16 keeps three more mantissa bits than bfloat16) and in float32
 * for float32 inputs.  Decode reads r_c from the cache instead. */

/* Chunk state memories as dart_chunk_states, plus r [b][H][M][N] float32 and
 * the score memory dH_score [b][H][M][P][N] (float16 or float32, see above),
 * both computed from dH as stored (after its rounding to dtype).  r and
 * dH_score are optional (NULL skips them); w_q [N] and w_e [P] are the
 * RMSNorm weights folded into dH_score (NULL = 1; 4-byte alignment). */
int dart_chunk_states_rms(const dart_dims_t* dims, int dtype, const void* X, const void* B,
                          const float* A, float eps, const float* w_q, const float* w_e, void* dH,
                          float* r, void* dH_score, void* stream);

/* r and the score memory of given chunk memories (any source, e.g. a cache
 * filled elsewhere): dims->seqlen and dims->chunk give M = ceil(L/S) memories
 * per (b, h) as for dart_chunk_states.  dH [b][H][M][P][N] (dtype) in,
 * r [b][H][M][N] float32 and dH_score out (either may be NULL). */
int dart_chunk_rms(const dart_dims_t* dims, int dtype, const void* dH, float eps, const float* w_q,
                   const float* w_e, float* r, void* dH_score, void* stream);

/* SMA forward with the normalised score branch and the gated residual.
 * Arguments as dart_sma_fwd, plus dH_score from dart_chunk_states_rms (with
 * the RMSNorm weights already folded in) and eps for the RMSNorm of Q_t and
 * E_t. */
int dart_sma_fwd_rms(const dart_dims_t* dims, int dtype, const void* Q, const void* C,
                     const void* E, const void* dH, const void* dH_score, const void* Y_ssm,
                     const void* gate, int gate_per_channel, float eps, void* out, float* R,
                     float* lse, void* stream);

/* Decode with the normalised score branch.  Arguments as dart_sma_decode,
 * plus r_cache [b][H][max_chunks][N] float32 (r_c of every cached chunk, as
 * written by dart_decode_state_update_rms or dart_chunk_states_rms), eps and
 * the RMSNorm weights w_q [N], w_e [P] (NULL = 1; 4-byte alignment).  The
 * workspace is sized by dart_sma_decode_workspace_bytes. */
int dart_sma_decode_rms(const dart_dims_t* dims, int dtype, int64_t max_chunks, const void* q,
                        const void* c, const void* e, const void* cache, const float* r_cache,
                        const int32_t* n_chunks, const void* y_ssm, const void* gate,
                        int gate_per_channel, float eps, const float* w_q, const float* w_e,
                        void* out, float* R, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream);

/* dart_decode_state_update, and for every chunk it closes also
 * r_cache[b][h][chunk][n] = r_c[n] of the memory as cached (float32,
 * [b][H][max_chunks][N], 16-byte aligned). */
int dart_decode_state_update_rms(const dart_dims_t* dims, int dtype, int64_t max_chunks, float eps,
                                 const void* x, const void* B, const float* a, float* state,
                                 const int32_t* pos, void* cache, float* r_cache, int32_t* n_chunks,
                                 void* stream);

/* Backward of the normalised score branch with the gated residual [App. B.1
 * Eq. 25-27 differentiated; §4 "Efficient Training"; App. C Eq. 33-35].  The
 * logits are recomputed from dH_score exactly as dart_sma_fwd_rms forms them,
 * p = exp(l - lse), and with dR_t = g_t * dout_t, D_t = dR_t . R_t,
 * qn = RMSNorm(Q_t) (weighted), en = RMSNorm(E_t) (weighted):
 *   dl     = p (dR_t . V_tc - D_t)                     (as dart_sma_bwd)
 *   dqn_t  = sum_c dl r_c * (dH_c en_t) / sqrt(N)
 *   den_t  = sum_c dl dH_c^T (r_c * qn_t) / sqrt(N)
 *   dC_t   = sum_c p dH_c dR_t
 *   dS_c   = sum_t dl qn_t en_t^T / sqrt(N)
 *   d_dH_c = sum_t p C_t^T dR_t + r_c * dS_c - (r_c^3 / P) dH_c * sum_p (dS_c * dH_c)
 *   dQ_t, dE_t: the RMSNorm backward of dqn_t * w_q, den_t * w_e,
 *   dw_q = sum over tokens and heads of dqn_t * Q_t / rms(Q_t)   (dw_e alike),
 * with r_c recomputed from dH as stored.
 *   Inputs: the forward's Q, C, E, dH, dH_score (from dart_chunk_states_rms
 *           or dart_chunk_rms with the same w_q, w_e, eps), gate, its outputs
 *           R and lse (float32), dout (dtype); eps and the RMSNorm weights
 *           w_q [N], w_e [P] (float32, NULL = 1, 4-byte alignment).
 *   Outputs, float32, fully overwritten: dQ, dC, dE, d_dH and dgate as for
 *           dart_sma_bwd; dw_q [N] and dw_e [P], each the gradient with
 *           respect to the weight at its value (1 where w_q or w_e is NULL);
 *           NULL skips dgate, dw_q or dw_e.  4-byte alignment for dw_q, dw_e.
 *   workspace: at least dart_sma_bwd_rms_workspace_bytes() bytes, 16-byte
 *           aligned; contents on entry are ignored.
 * Every result is deterministic: sums over heads, tokens and chunks run in a
 * fixed order. */
int dart_sma_bwd_rms(const dart_dims_t* dims, int dtype, const void* Q, const void* C,
                     const void* E, const void* dH, const void* dH_score, const void* gate,
                     int gate_per_channel, float eps, const float* w_q, const float* w_e,
                     const float* R, const float* lse, const void* dout, float* dQ, float* dC,
                     float* dE, float* d_dH, float* dgate, float* dw_q, float* dw_e,
                     void* workspace, size_t workspace_bytes, void* stream);
size_t dart_sma_bwd_rms_workspace_bytes(const dart_dims_t* dims);

/* The SSM branch of the block by the Mamba-2 chunked scan [§2 Eq. 2; App. A
 * Eq. 15-24]:  Y_t = C_t H_t,  H_t = a_t H_{t-1} + B_t^T X_t,  H_{-1} = H0,
 * computed per chunk c as the chunk state memory dH_[c] (Eq. 20, exactly
 * what dart_chunk_states writes), the boundary states
 * H_[c] = A_{a_c:b_c} H_[c-1] + dH_[c] (Eq. 17-18) and
 * Y_t = sum_{s in c, s <= t} C_t A_{s+1:t} B_s^T X_s + C_t A_{a_c:t} H_[c-1]
 * (Eq. 19-22).  Y is the Y_ssm input of dart_sma_fwd; dH its chunk memories.
 *   X [b][L][H][P], B, C [b][L][G][N] (dtype), A [b][L][H] float32
 *   H0 [b][H][P][N] float32 (state before the first token, NULL = 0; the
 *      same [P][N] orientation as dH)
 *   Y [b][L][H][P] (dtype), dH [b][H][M][P][N] (dtype)
 *   H_final [b][H][P][N] float32: the state after the last token (NULL skips it)
 *   workspace: at least dart_ssd_fwd_workspace_bytes(dims, dtype) bytes
 *      (chunk decays and the state entering every chunk, stored in dtype).
 * Arithmetic in float32; the state entering each chunk is rounded to dtype
 * once before it is read back. */
int dart_ssd_fwd(const dart_dims_t* dims, int dtype, const void* X, const void* B, const void* C,
                 const float* A, const float* H0, void* Y, void* dH, float* H_final, void* workspace,
                 size_t workspace_bytes, void* stream);
size_t dart_ssd_fwd_workspace_bytes(const dart_dims_t* dims, int dtype);

const char* dart_status_string(int status);
/* Message for this thread's last failing call ("" if none). */
const char* dart_last_error(void);
int dart_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DART_H_ */
