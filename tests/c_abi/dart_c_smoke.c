/* A plain C consumer of libdart.so: device memory from the HIP runtime, the
 * library called through include/dart.h only (no Python, no torch).
 *
 * On a small bfloat16 problem (b = 1, L = 600, H = 2, G = 1, N = 128,
 * P = 64, S = 128) it checks properties that follow from the definitions
 * (DART paper §3 Eq. 5, 8-11; §4 "Inference Cache"), on the matrix-core and
 * on the general kernels:
 *   - gate = 0 gives out == Y_ssm bit for bit (the residual adds nothing);
 *   - gate = 1 gives out == bf16(Y_ssm + R) bit for bit;
 *   - tokens of chunk 0 see no chunk: R = 0 and lse = -inf;
 *   - two launches give identical outputs;
 *   - the two families' chunk memories agree to the bf16 bar (2e-2 of the
 *     largest), each rounding its own float32 sums;
 *   - decode of the last token against the chunk memories before it equals
 *     the forward's row of that token (R, lse within 1e-3);
 *   - on the same memories the two families agree on R within 1e-3;
 *   - backward with gate = 0: dQ, dC, dE, d_dH exactly 0, dgate = dout * R;
 *     the chunk-state backward of d_dH = 0 exactly 0; with gate = 1 the two
 *     kernel families agree on dQ and dC at the bf16 bar (2e-2);
 *   - a NULL input is refused with DART_ERR_NULL and a message naming it.
 * Prints "c abi smoke ok" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dart.h"

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      exit(1);                            \
    }                                     \
  } while (0)

enum { B = 1, L = 600, H = 2, G = 1, N = 128, P = 64, S = 128, M = (L + S - 1) / S };

static uint64_t lcg = 0x9e3779b97f4a7c15ull;
static float uniform(void) { /* [-1, 1) */
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((lcg >> 40) & 0xffffff) / 8388608.0f - 1.0f;
}
static uint16_t to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint16_t* bf16_array(size_t n, float scale) {
  uint16_t* a = (uint16_t*)malloc(n * 2);
  for (size_t i = 0; i < n; ++i) a[i] = to_bf16(uniform() * scale);
  return a;
}
static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}
static void* dev_alloc(size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  return d;
}
static void to_host(void* host, const void* dev, size_t bytes) {
  CHECK_HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
}

int main(void) {
  int ndev = 0;
  CHECK_HIP(hipGetDeviceCount(&ndev));
  CHECK(ndev > 0, "no GPU");
  CHECK(dart_abi_version() == DART_ABI_VERSION, "ABI version %d", dart_abi_version());

  const size_t nx = (size_t)B * L * H * P, nq = (size_t)B * L * G * N, ne = (size_t)B * L * G * P;
  const size_t na = (size_t)B * L * H, nh = (size_t)B * H * M * P * N, nl = (size_t)B * H * L;
  const float sp = 1.7320508f / sqrtf((float)P), sn = 1.7320508f / sqrtf((float)N);
  uint16_t *hX = bf16_array(nx, sp), *hB = bf16_array(nq, sn), *hC = bf16_array(nq, sn);
  uint16_t *hQ = bf16_array(nq, 3.0f * sn), *hE = bf16_array(ne, sp), *hY = bf16_array(nx, 1.7320508f);
  float* hA = (float*)malloc(na * 4);
  for (size_t i = 0; i < na; ++i) hA[i] = 0.75f + 0.25f * uniform(); /* decays in [0.5, 1) */
  uint16_t* hzero = (uint16_t*)calloc(nx, 2);
  uint16_t* hone = (uint16_t*)malloc(nx * 2);
  for (size_t i = 0; i < nx; ++i) hone[i] = to_bf16(1.0f);

  void *X = dev_copy(hX, nx * 2), *Bm = dev_copy(hB, nq * 2), *C = dev_copy(hC, nq * 2);
  void *Q = dev_copy(hQ, nq * 2), *E = dev_copy(hE, ne * 2), *Y = dev_copy(hY, nx * 2);
  float* A = (float*)dev_copy(hA, na * 4);
  void *g0 = dev_copy(hzero, nx * 2), *g1 = dev_copy(hone, nx * 2);
  void *dH = dev_alloc(nh * 2), *out = dev_alloc(nx * 2), *out2 = dev_alloc(nx * 2);
  float *R = (float*)dev_alloc(nx * 4), *lse = (float*)dev_alloc(nl * 4);

  const dart_dims_t dims = {B, L, H, G, N, P, S};
  uint16_t* ho = (uint16_t*)malloc(nx * 2);
  uint16_t* ho2 = (uint16_t*)malloc(nx * 2);
  float* hR = (float*)malloc(nx * 4);
  float* hR_mfma = (float*)malloc(nx * 4);
  float* hl = (float*)malloc(nl * 4);

  /* chunk memories from both kernel families: each rounds its float32 sums
   * to bf16, so they agree to the bf16 bar, not bit for bit; the forward
   * calls below both read the matrix-core memories */
  void* dHg = dev_alloc(nh * 2);
  dart_set_path(DART_PATH_GENERAL);
  CHECK(dart_chunk_states(&dims, DART_BF16, X, Bm, A, dHg, NULL) == DART_OK, "chunk states: %s", dart_last_error());
  dart_set_path(DART_PATH_AUTO);
  CHECK(dart_chunk_states(&dims, DART_BF16, X, Bm, A, dH, NULL) == DART_OK, "chunk states: %s", dart_last_error());
  CHECK_HIP(hipDeviceSynchronize());
  {
    uint16_t *h1 = (uint16_t*)malloc(nh * 2), *h2 = (uint16_t*)malloc(nh * 2);
    to_host(h1, dH, nh * 2);
    to_host(h2, dHg, nh * 2);
    float dmax = 0.f, hmax = 0.f;
    for (size_t i = 0; i < nh; ++i) {
      dmax = fmaxf(dmax, fabsf(from_bf16(h1[i]) - from_bf16(h2[i])));
      hmax = fmaxf(hmax, fabsf(from_bf16(h1[i])));
    }
    CHECK(hmax > 0.f && dmax <= 2e-2f * hmax, "chunk memories of the two families differ by %g of %g", dmax, hmax);
    free(h1);
    free(h2);
  }

  for (int path = DART_PATH_AUTO; path <= DART_PATH_GENERAL; ++path) {
    dart_set_path(path);
    /* gate = 0: out is Y bit for bit */
    CHECK(dart_sma_fwd(&dims, DART_BF16, Q, C, E, dH, Y, g0, 1, out, NULL, NULL, NULL) == DART_OK, "fwd: %s",
          dart_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    to_host(ho, out, nx * 2);
    CHECK(memcmp(ho, hY, nx * 2) == 0, "path %d: gate 0 does not give out == Y", path);
    /* gate = 1, with R and lse, twice */
    CHECK(dart_sma_fwd(&dims, DART_BF16, Q, C, E, dH, Y, g1, 1, out, R, lse, NULL) == DART_OK, "fwd: %s",
          dart_last_error());
    CHECK(dart_sma_fwd(&dims, DART_BF16, Q, C, E, dH, Y, g1, 1, out2, NULL, NULL, NULL) == DART_OK, "fwd: %s",
          dart_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    to_host(ho, out, nx * 2);
    to_host(ho2, out2, nx * 2);
    to_host(hR, R, nx * 4);
    to_host(hl, lse, nl * 4);
    CHECK(memcmp(ho, ho2, nx * 2) == 0, "path %d: two launches differ", path);
    size_t bad = 0;
    for (size_t i = 0; i < nx; ++i)
      if (ho[i] != to_bf16(fmaf(1.0f, hR[i], from_bf16(hY[i])))) ++bad;
    CHECK(bad == 0, "path %d: %zu outputs differ from bf16(Y + R)", path, bad);
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < S; ++t) {
        CHECK(isinf(hl[h * L + t]) && hl[h * L + t] < 0.f, "path %d: lse of chunk-0 token %d is %g", path, t,
              hl[h * L + t]);
        for (int p = 0; p < P; ++p)
          CHECK(hR[((size_t)t * H + h) * P + p] == 0.f, "path %d: R of chunk-0 token %d is not 0", path, t);
      }
    if (path == DART_PATH_AUTO) {
      memcpy(hR_mfma, hR, nx * 4);
    } else {
      float dmax = 0.f, rmax = 0.f;
      for (size_t i = 0; i < nx; ++i) {
        dmax = fmaxf(dmax, fabsf(hR[i] - hR_mfma[i]));
        rmax = fmaxf(rmax, fabsf(hR[i]));
      }
      CHECK(dmax <= 1e-3f * rmax, "general and matrix-core R differ by %g of %g", dmax, rmax);
    }
  }
  dart_set_path(DART_PATH_AUTO);

  /* decode of the last token against the chunk memories before it */
  const int t = L - 1;
  const int32_t nb = t / S;
  uint16_t *hq = (uint16_t*)malloc(G * N * 2), *hc = (uint16_t*)malloc(G * N * 2), *he = (uint16_t*)malloc(G * P * 2);
  uint16_t* hy = (uint16_t*)malloc(H * P * 2);
  memcpy(hq, hQ + (size_t)t * G * N, G * N * 2);
  memcpy(hc, hC + (size_t)t * G * N, G * N * 2);
  memcpy(he, hE + (size_t)t * G * P, G * P * 2);
  memcpy(hy, hY + (size_t)t * H * P, H * P * 2);
  void *q = dev_copy(hq, G * N * 2), *c = dev_copy(hc, G * N * 2), *e = dev_copy(he, G * P * 2);
  void *y = dev_copy(hy, H * P * 2), *gd = dev_copy(hone, H * P * 2), *od = dev_alloc(H * P * 2);
  int32_t* nch = (int32_t*)dev_copy(&nb, 4);
  float *Rd = (float*)dev_alloc(H * P * 4), *ld = (float*)dev_alloc(H * 4);
  const size_t wsb = dart_sma_decode_workspace_bytes(&dims, M);
  void* ws = dev_alloc(wsb ? wsb : 16);
  CHECK(dart_sma_decode(&dims, DART_BF16, M, q, c, e, dH, nch, y, gd, 1, od, Rd, ld, ws, wsb, NULL) == DART_OK,
        "decode: %s", dart_last_error());
  CHECK_HIP(hipDeviceSynchronize());
  float hRd[H * P], hld[H];
  to_host(hRd, Rd, sizeof(hRd));
  to_host(hld, ld, sizeof(hld));
  float dmax = 0.f, rmax = 0.f;
  for (int h = 0; h < H; ++h) {
    for (int p = 0; p < P; ++p) {
      const float r = hR_mfma[((size_t)t * H + h) * P + p];
      dmax = fmaxf(dmax, fabsf(hRd[h * P + p] - r));
      rmax = fmaxf(rmax, fabsf(r));
    }
  }
  CHECK(dmax <= 1e-3f * rmax, "decode R differs from the forward row by %g of %g", dmax, rmax);
  for (int h = 0; h < H; ++h)
    CHECK(fabsf(hld[h] - hl[h * L + t]) <= 1e-3f * fabsf(hl[h * L + t]), "decode lse %g, forward %g", hld[h],
          hl[h * L + t]);

  /* backward [§4 "Efficient Training"; App. C Eq. 33-35]: with gate = 0,
   * dR = g * dout = 0, so dQ, dC, dE and d_dH are exactly 0 and
   * dgate = dout * R; the chunk-state backward of d_dH = 0 is exactly 0.
   * With gate = 1 the two kernel families agree on dQ and dC at the bf16
   * bar (the matrix-core passes round their scaled operands to bf16). */
  {
    const size_t nqf = nq, nef = ne, nhf = nh;
    uint16_t* hd = bf16_array(nx, 1.0f);
    void* dout = dev_copy(hd, nx * 2);
    float *dQ = (float*)dev_alloc(nqf * 4), *dC = (float*)dev_alloc(nqf * 4), *dE = (float*)dev_alloc(nef * 4);
    float *ddH = (float*)dev_alloc(nhf * 4), *dg = (float*)dev_alloc(nx * 4);
    const size_t wb = dart_sma_bwd_workspace_bytes(&dims);
    void* wsb = dev_alloc(wb);
    CHECK(dart_sma_bwd(&dims, DART_BF16, Q, C, E, dH, g0, 1, R, lse, dout, dQ, dC, dE, ddH, dg, wsb, wb, NULL) ==
              DART_OK,
          "bwd: %s", dart_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    float* hb = (float*)malloc(nhf * 4);
    const struct { float* d; size_t n; const char* name; } zeros[] = {
        {dQ, nqf, "dQ"}, {dC, nqf, "dC"}, {dE, nef, "dE"}, {ddH, nhf, "d_dH"}};
    for (int z = 0; z < 4; ++z) {
      to_host(hb, zeros[z].d, zeros[z].n * 4);
      for (size_t i = 0; i < zeros[z].n; ++i) CHECK(hb[i] == 0.f, "gate 0: %s[%zu] = %g", zeros[z].name, i, hb[i]);
    }
    float* hR = (float*)malloc(nx * 4);
    to_host(hR, R, nx * 4);
    to_host(hb, dg, nx * 4);
    float gmax = 0.f, gerr = 0.f;
    for (size_t i = 0; i < nx; ++i) {
      const float ref = from_bf16(hd[i]) * hR[i];
      gmax = fmaxf(gmax, fabsf(ref));
      gerr = fmaxf(gerr, fabsf(hb[i] - ref));
    }
    CHECK(gmax > 0.f && gerr <= 1e-6f * gmax, "dgate differs from dout * R by %g of %g", gerr, gmax);

    const size_t cwb = dart_chunk_states_bwd_workspace_bytes(&dims);
    void* cws = dev_alloc(cwb ? cwb : 16);
    float *dX = (float*)dev_alloc(nx * 4), *dB = (float*)dev_alloc(nqf * 4), *dA = (float*)dev_alloc(na * 4);
    CHECK(dart_chunk_states_bwd(&dims, DART_BF16, X, Bm, A, ddH, dX, dB, dA, cws, cwb, NULL) == DART_OK,
          "chunk states bwd: %s", dart_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    const struct { float* d; size_t n; const char* name; } czeros[] = {{dX, nx, "dX"}, {dB, nqf, "dB"}, {dA, na, "dA"}};
    for (int z = 0; z < 3; ++z) {
      to_host(hb, czeros[z].d, czeros[z].n * 4);
      for (size_t i = 0; i < czeros[z].n; ++i) CHECK(hb[i] == 0.f, "d_dH 0: %s[%zu] = %g", czeros[z].name, i, hb[i]);
    }

    float* h2 = (float*)malloc(nqf * 4);
    float* hgen = (float*)malloc(nqf * 4);
    for (int which = 0; which < 2; ++which) {
      float* gout = which == 0 ? dQ : dC;
      for (int path = DART_PATH_AUTO; path <= DART_PATH_GENERAL; ++path) {
        dart_set_path(path);
        CHECK(dart_sma_bwd(&dims, DART_BF16, Q, C, E, dH, g1, 1, R, lse, dout, dQ, dC, dE, ddH, NULL, wsb, wb,
                           NULL) == DART_OK,
              "bwd: %s", dart_last_error());
        CHECK_HIP(hipDeviceSynchronize());
        to_host(path == DART_PATH_AUTO ? h2 : hgen, gout, nqf * 4);
      }
      dart_set_path(DART_PATH_AUTO);
      float dmax = 0.f, vmax = 0.f;
      for (size_t i = 0; i < nqf; ++i) {
        dmax = fmaxf(dmax, fabsf(h2[i] - hgen[i]));
        vmax = fmaxf(vmax, fabsf(hgen[i]));
      }
      CHECK(vmax > 0.f && dmax <= 2e-2f * vmax, "%s: matrix-core and general backward differ by %g of %g",
            which == 0 ? "dQ" : "dC", dmax, vmax);
    }
  }

  /* argument errors: nothing launches, the message names the argument */
  CHECK(dart_sma_fwd(&dims, DART_BF16, NULL, C, E, dH, Y, g1, 1, out, NULL, NULL, NULL) == DART_ERR_NULL,
        "NULL Q accepted");
  CHECK(strstr(dart_last_error(), "Q") != NULL, "message '%s' does not name Q", dart_last_error());

  printf("c abi smoke ok (lse of the last token %.4f / %.4f; decode - forward R %.2e of %.2e)\n", hld[0],
         hl[0 * L + t], dmax, rmax);
  return 0;
}
