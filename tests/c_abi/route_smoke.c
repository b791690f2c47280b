/*
 * Plain-C user of libmoe_route: no torch, only the HIP runtime and the C ABI
 * of include/moe_route.h.  Runs mask -> indices -> dispatch (bf16, MXFP4)
 * -> combine on a small seeded problem and checks what the definitions fix:
 * the masked rows, restore inverting token_expert_order, stable expert
 * groups, dispatched rows equal to their source rows, identical MXFP4 copies
 * of one token, and combine with a single weight-1 slot reproducing the row.
 * Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_route.h"

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); return 2; } } while (0)
#define CHECK_MOE(x) do { int s_ = (x); if (s_ != MOE_OK) { \
  fprintf(stderr, "%s failed: %s\n", #x, moe_error_string(s_)); return 3; } } while (0)
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 4; } } while (0)

static uint32_t lcg(uint64_t* s) { *s = *s * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(*s >> 33); }

int main(void) {
  const int64_t N = 1000, R = 900;
  const int32_t K = 4, E = 64, H = 256;
  const int64_t S = N * K;
  uint64_t seed = 12345;

  int32_t* ids = malloc(S * sizeof(int32_t));
  uint16_t* x = malloc(N * H * sizeof(uint16_t));
  float* w = malloc(S * sizeof(float));
  for (int64_t t = 0; t < N; ++t)
    for (int32_t j = 0; j < K; ++j) ids[t * K + j] = (int32_t)(lcg(&seed) % (E + 2)) - 1;
  for (int64_t i = 0; i < N * H; ++i) x[i] = (uint16_t)(0x3C00 + (lcg(&seed) & 0x3FF)) ^ (uint16_t)((lcg(&seed) & 1) << 15);
  for (int64_t i = 0; i < S; ++i) w[i] = 0.0f;
  for (int64_t t = 0; t < N; ++t) w[t * K] = 1.0f;  /* only slot 0 of each token counts */

  int32_t *d_ids, *d_cnt, *d_eids;
  uint16_t *d_x, *d_disp, *d_out;
  uint8_t *d_q, *d_s, *d_ws;
  uint32_t *d_teo, *d_esi, *d_res, *d_stats;
  float* d_w;
  hipStream_t st;
  size_t wsb = moe_create_indices_workspace_bytes(S, E);
  EXPECT(wsb > 0);
  CHECK_HIP(hipStreamCreate(&st));
  CHECK_HIP(hipMalloc((void**)&d_ids, S * 4));
  CHECK_HIP(hipMalloc((void**)&d_cnt, 4));
  CHECK_HIP(hipMalloc((void**)&d_x, N * H * 2));
  CHECK_HIP(hipMalloc((void**)&d_w, S * 4));
  CHECK_HIP(hipMalloc((void**)&d_teo, S * 4));
  CHECK_HIP(hipMalloc((void**)&d_res, S * 4));
  CHECK_HIP(hipMalloc((void**)&d_esi, (E + 1) * 4));
  CHECK_HIP(hipMalloc((void**)&d_eids, E * 4));
  CHECK_HIP(hipMalloc((void**)&d_stats, 8));
  CHECK_HIP(hipMalloc((void**)&d_ws, wsb));
  CHECK_HIP(hipMalloc((void**)&d_disp, S * H * 2));
  CHECK_HIP(hipMalloc((void**)&d_q, S * H / 2));
  CHECK_HIP(hipMalloc((void**)&d_s, S * H / 32));
  CHECK_HIP(hipMalloc((void**)&d_out, N * H * 2));
  CHECK_HIP(hipMemset(d_ws, 0, wsb));
  CHECK_HIP(hipMemcpy(d_ids, ids, S * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_cnt, &(int32_t){(int32_t)R}, 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, N * H * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w, S * 4, hipMemcpyHostToDevice));

  CHECK_MOE(moe_mask_padding(d_ids, N, K, d_cnt, 0, st));
  CHECK_MOE(moe_create_indices(d_ids, S, E, d_teo, d_esi, d_res, d_eids, d_stats, NULL, 0, d_ws, wsb, st));
  CHECK_MOE(moe_dispatch(d_x, N, H, K, d_res, d_disp, S, st));
  CHECK_MOE(moe_dispatch_mxfp4(d_x, N, H, K, d_res, d_q, d_s, S, 0, st));
  /* combine over y = the dispatched rows: with weight 1 on slot 0 only, row t comes back */
  CHECK_MOE(moe_combine(d_disp, S, d_w, d_res, N, H, K, d_out, st));
  CHECK_HIP(hipStreamSynchronize(st));

  int32_t* m = malloc(S * 4);
  uint32_t *teo = malloc(S * 4), *res = malloc(S * 4), *esi = malloc((E + 1) * 4), stats[2];
  uint16_t *disp = malloc(S * H * 2), *out = malloc(N * H * 2);
  uint8_t *q = malloc(S * H / 2), *sc = malloc(S * H / 32);
  CHECK_HIP(hipMemcpy(m, d_ids, S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(teo, d_teo, S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(res, d_res, S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(esi, d_esi, (E + 1) * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(stats, d_stats, 8, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(disp, d_disp, S * H * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(q, d_q, S * H / 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(sc, d_s, S * H / 32, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out, d_out, N * H * 2, hipMemcpyDeviceToHost));

  int64_t v = 0;
  for (int64_t i = 0; i < S; ++i) {
    const int64_t t = i / K;
    if (t >= R) EXPECT(m[i] == -1); else EXPECT(m[i] == ids[i]);
    if (m[i] >= 0 && m[i] < E) ++v;
  }
  EXPECT(esi[stats[1]] == (uint32_t)v);
  for (int64_t p = 0; p < v; ++p) {
    const uint32_t i = teo[p];
    EXPECT(i < S && res[i] == (uint32_t)p);
    if (p > 0) EXPECT(m[teo[p - 1]] < m[i] || (m[teo[p - 1]] == m[i] && teo[p - 1] < i));
    EXPECT(memcmp(disp + (int64_t)p * H, x + (int64_t)(i / K) * H, H * 2) == 0);
  }
  for (int64_t p = v; p < S; ++p) EXPECT(teo[p] == MOE_SENTINEL);
  for (int64_t t = 0; t < N; ++t) {
    uint32_t first = MOE_SENTINEL;
    for (int32_t j = 0; j < K; ++j) {
      const uint32_t p = res[t * K + j];
      if (p == MOE_SENTINEL) continue;
      if (first == MOE_SENTINEL) first = p;
      EXPECT(memcmp(q + (int64_t)p * H / 2, q + (int64_t)first * H / 2, H / 2) == 0);
      EXPECT(memcmp(sc + (int64_t)p * H / 32, sc + (int64_t)first * H / 32, H / 32) == 0);
    }
    const uint32_t p0 = res[t * K];
    for (int32_t c = 0; c < H; ++c) {
      const uint16_t want = p0 == MOE_SENTINEL ? 0 : x[t * H + c];
      const uint16_t got = out[t * H + c];
      /* +0 and -0 both read back as a zero sum: -0 * 1 + 0 = +0 */
      EXPECT(got == want || (want == 0x8000 && got == 0));
    }
  }
  printf("c-abi ok: N=%lld routed=%lld active=%u max=%u\n", (long long)N, (long long)v, stats[1], stats[0]);
  return 0;
}
