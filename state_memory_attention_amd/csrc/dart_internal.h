// Internal interface between the C ABI layer (api.cpp) and the kernel files.
// Host-side launchers only; every launcher enqueues on `stream` and returns
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dart {

struct Shape {
  int64_t b, L, H, G, N, P, S, M;  // M = ceil(L / S)
};

// ---- general kernels (any N, P <= 256; float32 or bfloat16) ---------------
hipError_t launch_chunk_states_general(const Shape& s, bool bf16, const void* X, const void* B,
                                       const float* A, void* dH, hipStream_t st);
hipError_t launch_sma_fwd_general(const Shape& s, bool bf16, const void* Q, const void* C,
                                  const void* E, const void* dH, const void* Y, const void* gate,
                                  int gate_pc, void* out, float* R, float* lse, hipStream_t st);
hipError_t launch_sma_decode_general(const Shape& s, bool bf16, int64_t max_chunks, const void* q,
                                     const void* c, const void* e, const void* cache,
                                     const int32_t* n_chunks, const void* y, const void* gate,
                                     int gate_pc, void* out, float* R, float* lse, hipStream_t st);

// ---- decode-side cache maintenance (any N, P) -----------------------------
// r_cache (nullable): inverse RMS of every chunk closed by the call
hipError_t launch_decode_update(const Shape& s, bool bf16, int64_t max_chunks, const void* x,
                                const void* B, const float* a, float* state, const int32_t* pos,
                                void* cache, int32_t* n_chunks, float* r_cache, float eps,
                                hipStream_t st);

// ---- RMS-normalised score branch (general kernels; r and the score memory
// from dH as stored: float16 score memory for bfloat16, float32 otherwise) --
hipError_t launch_chunk_rms(const Shape& s, bool bf16, float eps, const void* dH, const float* wq,
                            const float* we, float* r, void* dHs, hipStream_t st);
hipError_t launch_sma_fwd_rms_general(const Shape& s, bool bf16, float eps, const void* Q,
                                      const void* C, const void* E, const void* dH, const void* dHs,
                                      const void* Y, const void* gate, int gate_pc, void* out,
                                      float* R, float* lse, hipStream_t st);
hipError_t launch_sma_decode_rms_general(const Shape& s, bool bf16, int64_t max_chunks, float eps,
                                         const void* q, const void* c, const void* e,
                                         const void* cache, const float* r_cache,
                                         const int32_t* n_chunks, const float* wq, const float* we,
                                         const void* y, const void* gate, int gate_pc, void* out,
                                         float* R, float* lse, hipStream_t st);

// ---- backward of the normalised score branch (general kernels; dHs as the
// forward consumed it; dwq, dwe nullable) -------------------------------------
size_t sma_bwd_rms_workspace_bytes(const Shape& s);
hipError_t launch_sma_bwd_rms_general(const Shape& s, bool bf16, float eps, const void* Q, const void* C,
                                      const void* E, const void* dH, const void* dHs, const float* wq,
                                      const float* we, const void* gate, int gate_pc, const float* R,
                                      const float* lse, const void* dout, float* dQ, float* dC, float* dE,
                                      float* ddH, float* dgate, float* dwq, float* dwe, float* ws,
                                      hipStream_t st);

// Column sums out[k] = sum_r in[r][k] in a fixed order (two passes through
// part, col_sum_split(rows) * K floats).
int64_t col_sum_split(int64_t rows);
hipError_t launch_col_sum(const float* in, float* part, float* out, int64_t rows, int K, hipStream_t st);

// The same on the matrix core (bf16, N = 128, P = 64).
size_t sma_bwd_rms_mfma_workspace_bytes(const Shape& s);
hipError_t launch_sma_bwd_rms_mfma(const Shape& s, float eps, const void* Q, const void* C, const void* E,
                                   const void* dH, const void* dHs, const float* wq, const float* we,
                                   const void* gate, int gate_pc, const float* R, const float* lse,
                                   const void* dout, float* dQ, float* dC, float* dE, float* ddH, float* dgate,
                                   float* dwq, float* dwe, void* ws, hipStream_t st);

// ---- backward, general kernels -------------------------------------------
size_t sma_bwd_workspace_bytes(const Shape& s);
hipError_t launch_sma_bwd_general(const Shape& s, bool bf16, const void* Q, const void* C,
                                  const void* E, const void* dH, const void* gate, int gate_pc,
                                  const float* R, const float* lse, const void* dout, float* dQ,
                                  float* dC, float* dE, float* ddH, float* dgate, float* ws,
                                  hipStream_t st);
size_t chunk_states_bwd_workspace_bytes(const Shape& s);
// mfma: dX, dB and dw on the matrix core (bfloat16, N = 128, P = 64); the
// decay recurrence and the group sums are shared.
hipError_t launch_chunk_states_bwd_general(const Shape& s, bool bf16, bool mfma, const void* X,
                                           const void* B, const float* A, const float* ddH, float* dX,
                                           float* dB, float* dA, float* ws, hipStream_t st);
hipError_t launch_chunk_states_bwd_mfma(const Shape& s, const void* X, const void* B, const float* A,
                                        const float* ddH, float* dX, float* dB, int db_heads,
                                        float* wsw, float* wsdw, hipStream_t st);

// ---- MFMA kernels (bfloat16, N = 128, P = 64) -----------------------------
// With r or dHs (the RMS-normalised score branch) the epilogue also writes
// the inverse RMS of every key row and the float16 score memory.
hipError_t launch_chunk_states_mfma(const Shape& s, const void* X, const void* B, const float* A,
                                    void* dH, hipStream_t st, float eps = 0.f,
                                    const float* wq = nullptr, const float* we = nullptr,
                                    float* r = nullptr, void* dHs = nullptr);
hipError_t launch_sma_fwd_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                               const void* dH, const void* Y, const void* gate, int gate_pc,
                               void* out, float* R, float* lse, hipStream_t st);

// RMS-normalised forward on the matrix core (float16 score memory)
hipError_t launch_sma_fwd_rms_mfma(const Shape& s, float eps, const void* Q, const void* C,
                                   const void* E, const void* dH, const void* dHs, const void* Y,
                                   const void* gate, int gate_pc, void* out, float* R, float* lse,
                                   hipStream_t st);

// Backward on the matrix core: pass A (recompute, p and dl, dE, dgate, dR),
// pass BC (dQ, dC), pass D (d_dH); per-head partials summed over groups.
size_t sma_bwd_mfma_workspace_bytes(const Shape& s);
hipError_t launch_sma_bwd_a_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                                 const void* dH, const void* gate, int gate_pc, const void* dout,
                                 const float* R, const float* lse, float* dE, int dE_heads,
                                 float* pd, void* dR, float* dgate, hipStream_t st);
// Pass BC modes: both gradients from dH; the Q side only, from the float16
// score memory of the normalised branch (rho: [b][L][G][2] RMSNorm factors;
// Q_norm: Q when each group has one head, and dQ then goes through the
// RMSNorm backward in the epilogue, else NULL); the C side only.  memT: the
// memories transposed by launch_mem_transpose ([b][H][M][N][P]).
constexpr int kBcBoth = 0, kBcScoreQ = 1, kBcC = 2;
hipError_t launch_sma_bwd_bc_mfma(const Shape& s, int mode, const void* E, const void* dR, const void* memT,
                                  const float* pd, const float* rho, const void* Q_norm, float* dQ, float* dC,
                                  int out_heads, hipStream_t st);
// out[m][n][p] = in[m][p][n] for `count` memories of P = 64 rows of N = 128
// two-byte entries (16-byte aligned)
hipError_t launch_mem_transpose(const void* in, void* out, int64_t count, hipStream_t st);
// byte offset of the transposed memories in the MFMA backward's workspace
size_t sma_bwd_memt_offset(const Shape& s);
// ddH_score: nullptr (both terms into ddH) or a buffer for the score term
hipError_t launch_sma_bwd_d_mfma(const Shape& s, const void* dR, const void* E, const void* C,
                                 const void* Q, const float* pd, float* ddH, float* ddH_score,
                                 hipStream_t st);
hipError_t launch_sma_bwd_mfma(const Shape& s, const void* Q, const void* C, const void* E,
                               const void* dH, const void* gate, int gate_pc, const float* R,
                               const float* lse, const void* dout, float* dQ, float* dC, float* dE,
                               float* ddH, float* dgate, void* ws, hipStream_t st);
// out[r][g][k] = sum over the hpg heads of group g of in[r][h][k]
hipError_t launch_group_sum(const float* in, float* out, int64_t rows, int64_t G, int64_t hpg,
                            int64_t K, hipStream_t st);

// ---- SSM branch by the chunked scan (chunk states, chunk decays, scan over
// chunks, outputs); mfma: bfloat16, N = 128, P = 64 ------------------------
size_t ssd_workspace_bytes(const Shape& s, bool bf16);
hipError_t launch_ssd_fwd(const Shape& s, bool bf16, bool mfma, const void* X, const void* B, const void* C,
                          const float* A, const float* H0, void* Y, void* dH, float* Hfin, void* ws,
                          hipStream_t st);

// Split-chunk decode: per (b, h, split) partial softmax states in the
// workspace, then a fixed-order combine.
struct DecodePlan {
  int64_t splits;           // chunk ranges per (b, h)
  int64_t chunks_per_split;
  size_t workspace_bytes;
};
DecodePlan decode_plan(int64_t b, int64_t H, int64_t P, int64_t max_chunks);
// Device address, on the current device, of the library's decode scratch
// (DART_DECODE_SCRATCH_BYTES per GPU, for dart_sma_decode_noalloc); looked up
// once per device.
hipError_t decode_scratch(float** ptr);
// r_cache non-null selects the RMS-normalised score branch (weights nullable)
hipError_t launch_sma_decode_mfma(const Shape& s, int64_t max_chunks, const DecodePlan& plan,
                                  const void* q, const void* c, const void* e, const void* cache,
                                  const int32_t* n_chunks, const void* y, const void* gate,
                                  int gate_pc, void* out, float* R, float* lse, float* ws,
                                  const float* r_cache, const float* wq, const float* we, float eps,
                                  hipStream_t st);

}  // namespace dart
