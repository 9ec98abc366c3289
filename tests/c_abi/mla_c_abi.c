/*
 * A plain C client of the library (test infrastructure): no Python, no torch.
 * It allocates device memory with the HIP runtime, calls mla_rope_rmsnorm_quant
 * through include/pkv.h on a small ragged batch (fp8 cache, per-tensor scale),
 * runs the CPU oracle on the same host arrays and compares: q within 1 bf16
 * ulp, cache codes within 1 step, at most 3 values of each differing, every
 * byte outside the new rows unchanged.  Then the same batch through
 * mla_rope_rmsnorm_inplace on a bf16 cache that holds the latent rows at the
 * new tokens' slots, against the oracle's in-place form.  Between the two,
 * the batch through pkv_token_plan + mla_rope_rmsnorm_quant_planned on a fresh
 * copy of the fp8 pool, which must write the batch form's bytes exactly.
 * Exit status 0 = pass.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"
#include "pkv_oracle.h" /* the oracle's entry points (liboracle.so) */

enum { B = 3, H = 5, R = 64, DN = 512, W = DN + R, S = 8, L = 2, LAYER = 1, MAXSEQ = 32 };

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}
/* a finite bf16 pattern with magnitude in [2^-4, 2^3) */
static uint16_t rand_bf16(void) {
  const uint32_t r = next32();
  const uint16_t sign = (uint16_t)((r & 1u) << 15);
  const uint16_t exp = (uint16_t)(127 - 4 + (r >> 1) % 7);
  return (uint16_t)(sign | (exp << 7) | ((r >> 8) & 0x7F));
}

#define CHECK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
      return 2;                                                         \
    }                                                                   \
  } while (0)

static long ord16(uint16_t u) { return (u & 0x8000) ? -(long)(u & 0x7FFF) : (long)(u & 0x7FFF); }
static long ord8(uint8_t u) { return (u & 0x80) ? -(long)(u & 0x7F) : (long)(u & 0x7F); }

int main(void) {
  const uint32_t new_len[B] = {3, 0, 5}, prior[B] = {2, 7, 11};
  uint32_t offsets[B + 1] = {0};
  for (int b = 0; b < B; ++b) offsets[b + 1] = offsets[b] + new_len[b];
  const int T = (int)offsets[B];
  enum { PT_STRIDE = 2, P = B * PT_STRIDE + 1 };
  uint32_t page_table[B * PT_STRIDE];
  for (int i = 0; i < B * PT_STRIDE; ++i) page_table[i] = (uint32_t)(P - 1 - i);  /* reversed */

  uint16_t* q = malloc(sizeof(uint16_t) * T * H * R);
  uint16_t* latent = malloc(sizeof(uint16_t) * T * W);
  uint16_t gamma[DN];
  float* freqs = malloc(sizeof(float) * MAXSEQ * R);
  const size_t cache_bytes = (size_t)L * P * S * W;
  uint8_t* cache0 = malloc(cache_bytes);
  for (int i = 0; i < T * H * R; ++i) q[i] = rand_bf16();
  for (int i = 0; i < T * W; ++i) latent[i] = rand_bf16();
  for (int i = 0; i < DN; ++i) gamma[i] = (uint16_t)(0x3F80 + (next32() % 64) - 32); /* ~1 */
  for (int p = 0; p < MAXSEQ; ++p)
    for (int i = 0; i < R / 2; ++i) {
      const double ang = p * pow(10000.0, -2.0 * i / R);
      freqs[p * R + 2 * i] = (float)cos(ang);
      freqs[p * R + 2 * i + 1] = (float)sin(ang);
    }
  for (size_t i = 0; i < cache_bytes; ++i) {
    uint8_t v = (uint8_t)next32();
    if ((v & 0x7F) == 0x7F) v ^= 1; /* no NaN codes */
    cache0[i] = v;
  }
  const float scale = 0.05f;
  const float eps = 1e-6f;

  /* device copies */
  void *d_q, *d_qo, *d_lat, *d_gamma, *d_freqs, *d_cache, *d_off, *d_len, *d_pt, *d_scale;
  CHECK(hipMalloc(&d_q, sizeof(uint16_t) * T * H * R));
  CHECK(hipMalloc(&d_qo, sizeof(uint16_t) * T * H * R));
  CHECK(hipMalloc(&d_lat, sizeof(uint16_t) * T * W));
  CHECK(hipMalloc(&d_gamma, sizeof gamma));
  CHECK(hipMalloc(&d_freqs, sizeof(float) * MAXSEQ * R));
  CHECK(hipMalloc(&d_cache, cache_bytes));
  CHECK(hipMalloc(&d_off, sizeof offsets));
  CHECK(hipMalloc(&d_len, sizeof prior));
  CHECK(hipMalloc(&d_pt, sizeof page_table));
  CHECK(hipMalloc(&d_scale, sizeof scale));
  CHECK(hipMemcpy(d_q, q, sizeof(uint16_t) * T * H * R, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_lat, latent, sizeof(uint16_t) * T * W, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_gamma, gamma, sizeof gamma, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_freqs, freqs, sizeof(float) * MAXSEQ * R, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_cache, cache0, cache_bytes, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_off, offsets, sizeof offsets, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_len, prior, sizeof prior, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_pt, page_table, sizeof page_table, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_scale, &scale, sizeof scale, hipMemcpyHostToDevice));

  pkv_paged_cache c;
  memset(&c, 0, sizeof c);
  c.data = d_cache;
  c.dtype = PKV_DTYPE_FP8_E4M3FN;
  c.num_layers = L;
  c.num_pages = P;
  c.page_size = S;
  c.num_heads = 1;
  c.head_dim = W;
  c.layer_stride = (int64_t)P * S * W;
  c.page_stride = (int64_t)S * W;
  c.slot_stride = W;
  c.head_stride = W;
  c.cache_lengths = d_len;
  c.page_table = d_pt;
  c.page_table_stride = PT_STRIDE;
  c.scale_mode = PKV_SCALE_PER_TENSOR;
  c.scales = d_scale;
  c.error_count = NULL;

  const int st = mla_rope_rmsnorm_quant(d_qo, (int64_t)H * R, R, d_q, (int64_t)H * R, R, d_lat, W,
                                        d_off, B, (uint32_t)T, H, R, DN, d_freqs, MAXSEQ, d_gamma,
                                        eps, &c, LAYER, NULL, NULL);
  if (st != PKV_OK) {
    fprintf(stderr, "mla_rope_rmsnorm_quant: %s\n", pkv_status_string(st));
    return 1;
  }
  CHECK(hipDeviceSynchronize());
  uint16_t* q_gpu = malloc(sizeof(uint16_t) * T * H * R);
  uint8_t* cache_gpu = malloc(cache_bytes);
  CHECK(hipMemcpy(q_gpu, d_qo, sizeof(uint16_t) * T * H * R, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(cache_gpu, d_cache, cache_bytes, hipMemcpyDeviceToHost));

  uint16_t* q_ref = malloc(sizeof(uint16_t) * T * H * R);
  uint8_t* cache_ref = malloc(cache_bytes);
  memcpy(cache_ref, cache0, cache_bytes);
  const int orc = oracle_mla_rope_rmsnorm_quant(q_ref, 0, q, 0, latent, offsets, prior, B,
                                                page_table, PT_STRIDE, freqs, 2, MAXSEQ, gamma,
                                                0, eps, H, R, DN, cache_ref, 0 /* fp8 */, L, P,
                                                S, LAYER, 1 /* per-tensor */, scale, NULL);
  if (orc != 0) {
    fprintf(stderr, "oracle: precondition failed (%d)\n", orc);
    return 1;
  }
  long q_diff = 0, q_max = 0, c_diff = 0, c_max = 0, rows_changed = 0;
  for (int i = 0; i < T * H * R; ++i) {
    const long d = labs(ord16(q_gpu[i]) - ord16(q_ref[i]));
    q_diff += d != 0;
    if (d > q_max) q_max = d;
  }
  for (size_t i = 0; i < cache_bytes; ++i) {
    const long d = labs(ord8(cache_gpu[i]) - ord8(cache_ref[i]));
    c_diff += d != 0;
    if (d > c_max) c_max = d;
    rows_changed += cache_ref[i] != cache0[i];
  }
  printf("c-abi mla: T=%d q: %ld differ (max %ld ulp); cache: %ld differ (max %ld); "
         "oracle changed %ld bytes\n", T, q_diff, q_max, c_diff, c_max, rows_changed);
  int ok = q_max <= 1 && q_diff <= 3 && c_max <= 1 && c_diff <= 3 && rows_changed > 0;

  /* planned: this batch's token plan, then the step placed by it */
  void *d_plan, *d_cache_p, *d_qo_p;
  CHECK(hipMalloc(&d_plan, sizeof(uint32_t) * 4 * T));
  CHECK(hipMalloc(&d_cache_p, cache_bytes));
  CHECK(hipMalloc(&d_qo_p, sizeof(uint16_t) * T * H * R));
  CHECK(hipMemcpy(d_cache_p, cache0, cache_bytes, hipMemcpyHostToDevice));
  c.data = d_cache_p;
  int st3 = pkv_token_plan((uint32_t*)d_plan, d_off, B, (uint32_t)T, &c, NULL);
  if (st3 == PKV_OK)
    st3 = mla_rope_rmsnorm_quant_planned(d_qo_p, (int64_t)H * R, R, d_q, (int64_t)H * R, R,
                                         d_lat, W, (const uint32_t*)d_plan, (uint32_t)T, H, R,
                                         DN, d_freqs, MAXSEQ, d_gamma, eps, &c, LAYER,
                                         NULL, NULL);
  if (st3 != PKV_OK) {
    fprintf(stderr, "planned: %s\n", pkv_status_string(st3));
    return 1;
  }
  CHECK(hipDeviceSynchronize());
  uint16_t* q_p = malloc(sizeof(uint16_t) * T * H * R);
  uint8_t* cache_p = malloc(cache_bytes);
  CHECK(hipMemcpy(q_p, d_qo_p, sizeof(uint16_t) * T * H * R, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(cache_p, d_cache_p, cache_bytes, hipMemcpyDeviceToHost));
  const int same = memcmp(q_p, q_gpu, sizeof(uint16_t) * T * H * R) == 0 &&
                   memcmp(cache_p, cache_gpu, cache_bytes) == 0;
  printf("c-abi mla planned: %s\n", same ? "bit-identical to the batch form" : "DIFFERS");
  ok = ok && same;

  /* in place: a bf16 cache holding each new token's latent row at its slot */
  const size_t n16 = (size_t)L * P * S * W;
  uint16_t* cache16 = malloc(sizeof(uint16_t) * n16);
  for (size_t i = 0; i < n16; ++i) cache16[i] = rand_bf16();
  for (int b = 0; b < B; ++b)
    for (uint32_t j = 0; j < new_len[b]; ++j) {
      const uint32_t slot = prior[b] + j;
      const uint32_t page = page_table[b * PT_STRIDE + slot / S];
      memcpy(cache16 + (((size_t)LAYER * P + page) * S + slot % S) * W,
             latent + (size_t)(offsets[b] + j) * W, sizeof(uint16_t) * W);
    }
  void* d_cache16;
  CHECK(hipMalloc(&d_cache16, sizeof(uint16_t) * n16));
  CHECK(hipMemcpy(d_cache16, cache16, sizeof(uint16_t) * n16, hipMemcpyHostToDevice));
  c.data = d_cache16;
  c.dtype = PKV_DTYPE_BF16;
  c.scale_mode = PKV_SCALE_NONE;
  c.scales = NULL;
  /* the element types spelled out (the same as the NULL defaults) */
  const pkv_elem_types types = {PKV_DTYPE_BF16, PKV_DTYPE_BF16, PKV_DTYPE_F32, PKV_DTYPE_BF16};
  const int st2 = mla_rope_rmsnorm_inplace(d_qo, (int64_t)H * R, R, d_q, (int64_t)H * R, R, d_off,
                                           B, (uint32_t)T, H, R, DN, d_freqs, MAXSEQ, d_gamma, eps,
                                           &c, LAYER, &types, NULL);
  if (st2 != PKV_OK) {
    fprintf(stderr, "mla_rope_rmsnorm_inplace: %s\n", pkv_status_string(st2));
    return 1;
  }
  CHECK(hipDeviceSynchronize());
  uint16_t* cache16_gpu = malloc(sizeof(uint16_t) * n16);
  CHECK(hipMemcpy(q_gpu, d_qo, sizeof(uint16_t) * T * H * R, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(cache16_gpu, d_cache16, sizeof(uint16_t) * n16, hipMemcpyDeviceToHost));
  uint16_t* cache16_ref = malloc(sizeof(uint16_t) * n16);
  memcpy(cache16_ref, cache16, sizeof(uint16_t) * n16);
  if (oracle_mla_rope_rmsnorm_inplace(q_ref, 0, q, 0, offsets, prior, B, page_table, PT_STRIDE,
                                      freqs, 2, MAXSEQ, gamma, 0, eps, H, R, DN, cache16_ref, L,
                                      P, S, LAYER) != 0) {
    fprintf(stderr, "oracle (in place): precondition failed\n");
    return 1;
  }
  long q2_diff = 0, q2_max = 0, r_diff = 0, r_max = 0, changed = 0;
  for (int i = 0; i < T * H * R; ++i) {
    const long d = labs(ord16(q_gpu[i]) - ord16(q_ref[i]));
    q2_diff += d != 0;
    if (d > q2_max) q2_max = d;
  }
  for (size_t i = 0; i < n16; ++i) {
    const long d = labs(ord16(cache16_gpu[i]) - ord16(cache16_ref[i]));
    r_diff += d != 0;
    if (d > r_max) r_max = d;
    changed += cache16_ref[i] != cache16[i];
  }
  printf("c-abi mla in place: q: %ld differ (max %ld ulp); cache: %ld differ (max %ld ulp); "
         "oracle changed %ld values\n", q2_diff, q2_max, r_diff, r_max, changed);
  ok = ok && q2_max <= 1 && q2_diff <= 3 && r_max <= 1 && r_diff <= 3 && changed > 0;
  puts(ok ? "PASS" : "FAIL");
  return ok ? 0 : 1;
}
