/*
 * The library used from plain C99 through include/moe.h and the HIP runtime's
 * C API only (no Python, no torch): route, permute, grouped SwiGLU forward and
 * combine on a small seeded layer, then invariants of the results: every
 * status is MOE_OK, each token's K experts are distinct and in range with
 * weights summing to one, the per-expert counts add up to T*K, segment starts
 * are multiples of the alignment, row_of maps the (token, k) pairs one to one
 * onto valid rows, and the output is finite.  A rejected call must leave a
 * message in moe_last_error().  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define CHECK_HIP(x)                                                         \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                              \
    }                                                                        \
  } while (0)
#define CHECK_MOE(x)                                                         \
  do {                                                                       \
    moe_status_t s_ = (x);                                                   \
    if (s_ != MOE_OK) {                                                      \
      fprintf(stderr, "%s failed: %s (%s)\n", #x, moe_status_string(s_), moe_last_error()); \
      return 3;                                                              \
    }                                                                        \
  } while (0)
#define EXPECT(c)                                                            \
  do {                                                                       \
    if (!(c)) {                                                              \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);         \
      return 4;                                                              \
    }                                                                        \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float uniform_pm1(void) { /* xorshift64*, mapped to [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  uint64_t r = rng_state * 2685821657736338717ull;
  return (float)((r >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}
static uint16_t to_bf16(float f) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void* dalloc(size_t bytes) {
  void* p = NULL;
  if (hipMalloc(&p, bytes ? bytes : 1) != hipSuccess) return NULL;
  return p;
}

int main(void) {
  const int32_t T = 300, H = 128, E = 8, K = 2, F = 64;
  const int32_t A = moe_align();
  const int64_t M = moe_capacity_rows(T, E, K);
  EXPECT(A > 0 && M % A == 0 && M >= (int64_t)T * K);

  /* a rejected call: K > E */
  EXPECT(moe_route(T, H, E, E + 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
         MOE_ERR_INVALID_ARGUMENT);
  EXPECT(strlen(moe_last_error()) > 0);

  /* host inputs */
  uint16_t* hx = malloc((size_t)T * H * 2);
  float* hwr = malloc((size_t)H * E * 4);
  float* hb = malloc((size_t)E * 4);
  uint16_t* hw1 = malloc((size_t)E * 2 * F * H * 2);
  uint16_t* hw2 = malloc((size_t)E * H * F * 2);
  for (int64_t i = 0; i < (int64_t)T * H; ++i) hx[i] = to_bf16(uniform_pm1());
  for (int64_t i = 0; i < (int64_t)H * E; ++i) hwr[i] = 0.1f * uniform_pm1();
  for (int i = 0; i < E; ++i) hb[i] = 0.01f * uniform_pm1();
  for (int64_t i = 0; i < (int64_t)E * 2 * F * H; ++i) hw1[i] = to_bf16(0.05f * uniform_pm1());
  for (int64_t i = 0; i < (int64_t)E * H * F; ++i) hw2[i] = to_bf16(0.05f * uniform_pm1());

  /* device buffers (caller-owned, as the ABI requires) */
  uint16_t* x = dalloc((size_t)T * H * 2);
  float* wr = dalloc((size_t)H * E * 4);
  float* b = dalloc((size_t)E * 4);
  uint16_t* w1 = dalloc((size_t)E * 2 * F * H * 2);
  uint16_t* w2 = dalloc((size_t)E * H * F * 2);
  int32_t* idx = dalloc((size_t)T * K * 4);
  float* tw = dalloc((size_t)T * K * 4);
  float* ts = dalloc((size_t)T * K * 4);
  const size_t rws = moe_route_workspace_bytes(T, H, E), pws = moe_permute_workspace_bytes(T, E, K);
  void* rw = dalloc(rws);
  void* pw = dalloc(pws);
  int32_t* counts = dalloc((size_t)E * 4);
  int32_t* offsets = dalloc((size_t)(E + 1) * 4);
  int32_t* row_of = dalloc((size_t)T * K * 4);
  int32_t* src = dalloc((size_t)M * 4);
  int32_t* tile_expert = dalloc((size_t)(M / A) * 4);
  uint16_t* x_rows = dalloc((size_t)M * H * 2);
  uint16_t* act = dalloc((size_t)M * 2 * F * 2);
  uint16_t* h = dalloc((size_t)M * F * 2);
  uint16_t* y_rows = dalloc((size_t)M * H * 2);
  uint16_t* y = dalloc((size_t)T * H * 2);
  EXPECT(x && wr && b && w1 && w2 && idx && tw && ts && rw && pw && counts && offsets &&
         row_of && src && tile_expert && x_rows && act && h && y_rows && y);
  CHECK_HIP(hipMemcpy(x, hx, (size_t)T * H * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(wr, hwr, (size_t)H * E * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(b, hb, (size_t)E * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w1, hw1, (size_t)E * 2 * F * H * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(w2, hw2, (size_t)E * H * F * 2, hipMemcpyHostToDevice));

  CHECK_MOE(moe_route(T, H, E, K, x, wr, b, idx, tw, ts, NULL, rw, rws, NULL));
  CHECK_MOE(moe_permute(T, H, E, K, A, idx, x, M, counts, offsets, row_of, src, tile_expert,
                        x_rows, pw, pws, NULL));
  CHECK_MOE(moe_grouped_swiglu_fwd(E, M, H, F, offsets, counts, tile_expert, x_rows, w1, w2, act,
                                   h, y_rows, NULL));
  CHECK_MOE(moe_combine(T, H, K, y_rows, row_of, tw, NULL, y, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  int32_t* hidx = malloc((size_t)T * K * 4);
  float* htw = malloc((size_t)T * K * 4);
  int32_t hcounts[8], hoff[9];
  int32_t* hrow = malloc((size_t)T * K * 4);
  int32_t* hsrc = malloc((size_t)M * 4);
  uint16_t* hy = malloc((size_t)T * H * 2);
  CHECK_HIP(hipMemcpy(hidx, idx, (size_t)T * K * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(htw, tw, (size_t)T * K * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hcounts, counts, sizeof(hcounts), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hoff, offsets, sizeof(hoff), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hrow, row_of, (size_t)T * K * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hsrc, src, (size_t)M * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hy, y, (size_t)T * H * 2, hipMemcpyDeviceToHost));
  int32_t check[4];
  CHECK_HIP(hipMemcpy(check, pw, sizeof(check), hipMemcpyDeviceToHost));
  CHECK_MOE(moe_permute_check(check)); /* moe_route's ids: nothing rejected */

  int64_t total = 0;
  for (int e = 0; e < E; ++e) {
    total += hcounts[e];
    EXPECT(hoff[e] % A == 0);
    EXPECT(hoff[e + 1] - hoff[e] == (hcounts[e] + A - 1) / A * A);
  }
  EXPECT(total == (int64_t)T * K && hoff[0] == 0 && hoff[E] <= M);
  for (int t = 0; t < T; ++t) {
    double wsum = 0.0;
    for (int k = 0; k < K; ++k) {
      const int e = hidx[t * K + k];
      EXPECT(e >= 0 && e < E);
      for (int j = 0; j < k; ++j) EXPECT(hidx[t * K + j] != e);
      wsum += htw[t * K + k];
      const int r = hrow[t * K + k];
      EXPECT(r >= hoff[e] && r < hoff[e] + hcounts[e]);
      EXPECT(hsrc[r] == t);
    }
    EXPECT(fabs(wsum - 1.0) < 1e-5);
  }
  for (int64_t i = 0; i < (int64_t)T * H; ++i) EXPECT(isfinite(from_bf16(hy[i])));
  printf("c-abi ok: T=%d H=%d E=%d K=%d F=%d, %lld routed rows in %d padded rows\n", T, H, E, K,
         F, (long long)total, hoff[E]);
  return 0;
}
