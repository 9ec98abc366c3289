/*
 * pkv_oracle.c -- CPU oracle for the paged-KV pre-attention path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark load this library.  It shares no
 * source, header, table or helper with the HIP library; it includes nothing but
 * the C standard library and its own pkv_oracle.h.
 *
 * Style: plain scalar loops, every intermediate in IEEE binary64 (built with
 * -ffp-contract=off, no fast-math), and exactly one rounding into each output
 * type.  A bf16 value times an fp32 value is exact in binary64 (8 + 24
 * significant bits), and so is the sum of two such products unless their
 * magnitudes lie more than 2^21 apart: a rotated value is then the correctly
 * rounded value of the plain definition, exact ties included.  Values that
 * pass through the square root and divisions of the norm carry a binary64
 * error well under 2^-43 relative, so they are correctly rounded except within
 * that distance of a rounding boundary.  The fused K norm of the Q/K RoPE
 * applies r after rotating a pair whose members it both scales (the rotation
 * is linear), so that a pair which cancels keeps the exactness above.
 * (tests/exact_pins.py checks both statements against 120-digit decimal
 * arithmetic.)
 *
 * Sources (Modular MAX / Mojo API reference pages):
 *   [MLA]   "mla_fused_rope_rmsnorm_quantization" -- summary, Parameters, Args
 *   [QK]    "generic_fused_qk_rope_bshd_paged_ragged" -- summary, Parameters, Args
 *   [GRAPH] "mla_graph" module page -- Functions list
 *   [NORM]  "rms_norm_kv_cache_ragged_paged" -- description paragraphs
 *   FP8 E4M3FN follows the OCP 8-bit floating point specification (v1.0),
 *   the public format the name "E4M3FN" in [GRAPH] refers to.
 *
 * Readings taken where the pages are silent (each is also tested):
 *   - freqs_cis row p holds (cos, sin) adjacent: column 2i = cos of pair i,
 *     column 2i+1 = sin of pair i ("cis" = cos + i sin).
 *   - Rotation: x' = x cos - y sin, y' = y cos + x sin.
 *   - MLA rope style is rotate-half: pair (i, i + R/2).  In [QK], interleaved
 *     means the pair (2i, 2i+1); either way pair i uses frequency column i.
 *   - Latent row = [kv_norm_dim non-rope values | rope_dim rope values]; gamma
 *     covers the first kv_norm_dim values.
 *   - Token t of request b (t = o[b] + j) sits at position and cache slot
 *     c[b] + j, where c[b] is the request's cache length before this step;
 *     slot s lives in page page_table[b][s / page_size] at offset
 *     s mod page_size.
 *   - RMSNorm: r = 1 / sqrt(mean(x^2) + eps), mean over the normalised
 *     columns only, eps inside the root, gamma applied before any cast.
 *   - FP8: value = y / scale (scale is the dequantisation multiplier),
 *     saturating to +-448, round-to-nearest-even, subnormals and -0 kept.
 *     Per-token scale = fp32(amax / 448) over the whole row; an all-zero row
 *     gets scale 0 and codes +-0.
 *   - In [QK] with a K norm, the norm runs before the rotation and the K row
 *     is rounded to bf16 once, after both.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "pkv_oracle.h"

/* Return codes: 0 = done; negative = a precondition on the data does not hold
 * (nothing is guaranteed about the outputs then). */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_BAD_POSITION (-2)
#define ORACLE_BAD_PAGE (-3)

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_decode(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest bfloat16 to v, ties to the even significand, in a single step from
 * binary64 (no intermediate binary32 rounding).  A bf16 value has 8
 * significant bits; its smallest quantum (subnormals) is 2^-133. */
uint16_t oracle_bf16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return 0x7FC0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int e;
  frexp(a, &e);                 /* a = f * 2^e with 0.5 <= f < 1 */
  int qexp = e - 8;             /* keep 8 significant bits */
  if (qexp < -133) qexp = -133; /* subnormal range: fixed quantum */
  double n = nearbyint(ldexp(a, -qexp)); /* default mode: ties to even */
  double r = ldexp(n, qexp);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow */
  float f = (float)r;           /* exact: r has at most 9 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits; exponent field 0 holds zero and the subnormals m * 2^-24, field 31
 * the infinities (fraction 0) and NaNs. */
double oracle_f16_decode(uint16_t bits) {
  const int e = (bits >> 10) & 0x1F;
  const int m = bits & 0x3FF;
  double mag;
  if (e == 0x1F) mag = m ? NAN : INFINITY;
  else if (e == 0) mag = ldexp((double)m, -24);
  else mag = ldexp(1.0 + m / 1024.0, e - 15);
  return (bits & 0x8000u) ? -mag : mag;
}

/* Nearest binary16 to v, ties to the even significand, in one step from
 * binary64; magnitudes that round past the largest finite value (65504)
 * become infinity, as IEEE rounding to nearest prescribes. */
uint16_t oracle_f16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return 0x7E00u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
  int e;
  frexp(a, &e);                 /* a = f * 2^e with 0.5 <= f < 1 */
  int qexp = e - 11;            /* keep 11 significant bits */
  if (qexp < -24) qexp = -24;   /* subnormal range: fixed quantum 2^-24 */
  double n = nearbyint(ldexp(a, -qexp));
  double r = ldexp(n, qexp);
  if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(r, 24)); /* subnormal */
  int er;
  frexp(r, &er);
  const int E = er - 1;         /* r = 1.f * 2^E, -14 <= E <= 15 */
  const int m = (int)((ldexp(r, -E) - 1.0) * 1024.0);
  return (uint16_t)(sign | ((E + 15) << 10) | m);
}

/* Element types of the q, freqs and gamma arrays ([MLA] Parameters: dtype,
 * freq_dtype, gamma_dtype, out_rope_dtype; [QK] Parameters: dtype and
 * freq_dtype; [NORM]: the dtype of gamma and weight_offset). */
#define ORACLE_BF16 0
#define ORACLE_F32 2
#define ORACLE_F16 3

/* Element i of an array of the given type, widened exactly to binary64. */
static double elem(const void* base, int64_t i, int type) {
  if (type == ORACLE_F32) return (double)((const float*)base)[i];
  const uint16_t bits = ((const uint16_t*)base)[i];
  return type == ORACLE_F16 ? oracle_f16_decode(bits) : oracle_bf16_decode(bits);
}

/* v rounded once into element i of an array of the given type. */
static void put_elem(void* base, int64_t i, int type, double v) {
  if (type == ORACLE_F32) ((float*)base)[i] = (float)v;  /* RNE */
  else if (type == ORACLE_F16) ((uint16_t*)base)[i] = oracle_f16_encode(v);
  else ((uint16_t*)base)[i] = oracle_bf16_encode(v);
}

/* Row p of a freqs_cis table of `dim` columns as fp32 values (bf16 and fp16
 * values are exactly fp32 values): a pointer into the table itself when it
 * is fp32, else into buf, filled. */
static const float* freqs_row_at(const void* freqs, int type, int64_t p, int64_t dim,
                                 float* buf) {
  if (type == ORACLE_F32) return (const float*)freqs + p * dim;
  for (int64_t i = 0; i < dim; ++i) buf[i] = (float)elem(freqs, p * dim + i, type);
  return buf;
}

/* FP8 E4M3FN (OCP): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 0x7E = 448, exponent field
 * 0 holds subnormals m * 2^-9. */
double oracle_e4m3fn_decode(uint8_t code) {
  int sign = (code >> 7) & 1;
  int ef = (code >> 3) & 0xF;
  int m = code & 7;
  double mag;
  if (ef == 0xF && m == 7) return NAN;
  if (ef == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, ef - 7);
  return sign ? -mag : mag;
}

/* Saturating round-to-nearest-even encode of a binary64 value.  Magnitudes
 * above 448 become 448 (saturation, never NaN); -0 keeps its sign.  A NaN
 * input is outside the method's domain and maps to the NaN code. */
uint8_t oracle_e4m3fn_encode_sat(double v) {
  uint8_t sign = signbit(v) ? 0x80u : 0u;
  if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                 /* a = f * 2^e with 0.5 <= f < 1 */
  int qexp = e - 4;             /* 4 significant bits for normals */
  if (qexp < -9) qexp = -9;     /* subnormal quantum 2^-9 */
  double n = nearbyint(ldexp(a, -qexp));
  double r = ldexp(n, qexp);    /* rounded magnitude, <= 448 */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) {     /* subnormal: r = m * 2^-9, m in 1..7 */
    int m = (int)ldexp(r, 9);
    return (uint8_t)(sign | m);
  }
  int er;
  frexp(r, &er);
  int E = er - 1;               /* r = 1.mmm * 2^E, -6 <= E <= 8 */
  int m = (int)((ldexp(r, -E) - 1.0) * 8.0);
  return (uint8_t)(sign | ((E + 7) << 3) | m);
}

/* Observation of fp8 decisions, for tests.  While a probe is set, every fp8
 * code that an entry point below writes into [probe_base, probe_base + n)
 * also leaves the binary64 value it was rounded from at the same index of
 * probe_pre.  A test then knows how close each code was to a rounding
 * midpoint; nothing else changes. */
static uintptr_t probe_base;
static int64_t probe_n;
static double* probe_pre;

void oracle_set_fp8_probe(const void* base, int64_t n, double* pre) {
  probe_base = (uintptr_t)base;
  probe_n = pre ? n : 0;
  probe_pre = pre;
}

static void put_fp8(uint8_t* dst, double v) {
  *dst = oracle_e4m3fn_encode_sat(v);
  const uintptr_t a = (uintptr_t)dst;
  if (probe_pre && a >= probe_base && a - probe_base < (uintptr_t)probe_n)
    probe_pre[a - probe_base] = v;
}

/* ------------------------------------------------------------------------- */
/* Steps of the method, in binary64                                           */
/* ------------------------------------------------------------------------- */

/* RoPE over one row of `dim` values with one freqs_cis row ([MLA] Args:
 * freqs_cis holds per position the cosine/sine values, dim columns).  Pair i
 * is (i, i + dim/2) for rotate-half and (2i, 2i+1) when interleaved ([QK]
 * Parameters: interleaved); it is rotated by the angle whose cos/sin sit in
 * columns 2i and 2i+1.  x and out must not alias. */
void oracle_rope_row(const double* x, double* out, int64_t dim,
                     const float* freqs_row, int interleaved) {
  int64_t half = dim / 2;
  for (int64_t i = 0; i < half; ++i) {
    double cs = (double)freqs_row[2 * i];
    double sn = (double)freqs_row[2 * i + 1];
    int64_t ia = interleaved ? 2 * i : i;
    int64_t ib = interleaved ? 2 * i + 1 : i + half;
    double a = x[ia];
    double b = x[ib];
    out[ia] = a * cs - b * sn;
    out[ib] = b * cs + a * sn;
  }
}

/* Inverse RMS of the first n values: 1 / sqrt(sum(x^2)/n + eps). */
double oracle_inv_rms(const double* x, int64_t n, double eps) {
  double ss = 0.0;
  for (int64_t k = 0; k < n; ++k) ss += x[k] * x[k];
  return 1.0 / sqrt(ss / (double)n + eps);
}

/* RMSNorm of the first n values, y_k = x_k * r * g_k ([MLA] summary: RMSNorm
 * on the non-rope part, with gamma; [NORM]: gamma plus weight_offset). */
void oracle_rmsnorm_row(const double* x, double* y, int64_t n, const double* g,
                        double eps) {
  double r = oracle_inv_rms(x, n, eps);
  for (int64_t k = 0; k < n; ++k) y[k] = x[k] * r * g[k];
}

/* ------------------------------------------------------------------------- */
/* Ragged and paged addressing                                                */
/* ------------------------------------------------------------------------- */

/* Physical page holding cache slot `slot` of request b, or -1 when the page
 * table entry is missing or out of range. */
static int64_t page_of(const uint32_t* page_table, int64_t pt_stride,
                       int64_t num_pages, int64_t page_size, int64_t b,
                       int64_t slot) {
  int64_t col = slot / page_size;
  if (col >= pt_stride) return -1;
  uint32_t p = page_table[b * pt_stride + col];
  if ((int64_t)p >= num_pages) return -1;
  return (int64_t)p;
}

/* ------------------------------------------------------------------------- */
/* Entry points                                                               */
/* ------------------------------------------------------------------------- */

/* Scale modes of the latent cache. */
#define ORACLE_SCALE_PER_TENSOR 1
#define ORACLE_SCALE_PER_TOKEN 2
/* Latent cache element types. */
#define ORACLE_CACHE_FP8 0
#define ORACLE_CACHE_BF16 1

/*
 * Fused MLA pre-attention step ([MLA] summary and Args; [GRAPH] entry
 * fused_rope_rmsnorm_quantization_kernel: read the latent from a buffer,
 * quantise at the end, write into the cache).
 *
 * Host arrays, all dense and row-major:
 *   q_out         [T][H][R] of q_out_type (q_rope_output; out_rope_dtype)
 *   q_in          [T][H][R] of q_in_type         (q_rope; dtype)
 *   latent        bf16 bits [T][Dn + R]          (the KV latent input)
 *   row_offsets   u32 [B + 1]                    (input_row_offsets)
 *   cache_lengths u32 [B]  length of each request's cache before this step
 *   page_table    u32 [B][pt_stride]
 *   freqs         [max_seq_len][R] of freq_type  (freqs_cis; freq_dtype)
 *   gamma         [Dn] of gamma_type             (gamma_dtype)
 * Element types: ORACLE_BF16 (bits), ORACLE_F16 (bits), ORACLE_F32.
 *   cache         [L][P][S][Dn + R] of u8 (fp8 codes) or u16 (bf16 bits)
 *   token_scales  f32 [L][P][S]  (written in per-token mode only)
 * Only layer `layer_idx` and only the new tokens' slots are written.
 * latent = NULL is the in-place form (see oracle_mla_rope_rmsnorm_inplace):
 * each token's row x is read from its own slot of the bf16 cache.
 */
/* True when a token plan entry (page, offset, position, placed) is marked
 * placed and names a slot inside the pool. */
static int plan_entry_placed(const uint32_t* e, int64_t num_pages, int64_t page_size) {
  return !(e[3] == 0 || (int64_t)e[0] >= num_pages || (int64_t)e[1] >= page_size);
}

/* gamma + weight_offset of the K-cache norm, widened ([NORM]: weight_offset
 * is added to gamma). */
static void kv_norm_gamma(const void* gamma, int gamma_type, int64_t n, float weight_offset,
                          double* g) {
  for (int64_t k = 0; k < n; ++k)
    g[k] = elem(gamma, k, gamma_type) + (double)weight_offset;
}

/* One token of the fused MLA step: q of token t rotated at position pos into
 * q_out, and the token's latent row (from the buffer, or in place from cache
 * row `row`) normalised, rotated and written to cache row `row` (row counts
 * latent rows of W = Dn + R elements from the start of the cache, layer
 * included). */
static int mla_token(void* q_out, int q_out_type, const void* q_in, int q_in_type,
                     const uint16_t* latent, int64_t t, int64_t pos, int64_t row,
                     const void* freqs, int freq_type, const double* g, double eps, int64_t H,
                     int64_t R, int64_t Dn, void* cache, int cache_type, int scale_mode,
                     float tensor_scale, float* token_scales) {
  const int64_t W = Dn + R;
  double x[4096], y[4096], qa[1024], qb[1024];
  float frow[1024];
  const float* fr = freqs_row_at(freqs, freq_type, pos, R, frow);

  /* q: RoPE on every head, one rounding per value into the output type
   * ([MLA] Parameters: dtype of q_rope, out_rope_dtype of q_rope_output). */
  for (int64_t h = 0; h < H; ++h) {
    for (int64_t i = 0; i < R; ++i) qa[i] = elem(q_in, (t * H + h) * R + i, q_in_type);
    oracle_rope_row(qa, qb, R, fr, 0);
    if (q_out_type == ORACLE_F32) {
      float* dst = (float*)q_out + (t * H + h) * R;
      for (int64_t i = 0; i < R; ++i) dst[i] = (float)qb[i];  /* RNE */
    } else {
      for (int64_t i = 0; i < R; ++i) put_elem(q_out, (t * H + h) * R + i, q_out_type, qb[i]);
    }
  }

  /* latent: RMSNorm on the first Dn values, RoPE on the R-value tail;
   * the row comes from its buffer, or in place from the cache slot. */
  const uint16_t* src = latent ? latent + t * W : (const uint16_t*)cache + row * W;
  for (int64_t k = 0; k < W; ++k) x[k] = oracle_bf16_decode(src[k]);
  oracle_rmsnorm_row(x, y, Dn, g, eps);
  oracle_rope_row(x + Dn, y + Dn, R, fr, 0);

  if (cache_type == ORACLE_CACHE_BF16) {
    uint16_t* dst = (uint16_t*)cache + row * W;
    for (int64_t k = 0; k < W; ++k) dst[k] = oracle_bf16_encode(y[k]);
    return ORACLE_OK;
  }
  uint8_t* dst = (uint8_t*)cache + row * W;
  if (scale_mode == ORACLE_SCALE_PER_TENSOR) {
    const double s = (double)tensor_scale;
    for (int64_t k = 0; k < W; ++k) put_fp8(&dst[k], y[k] / s);
  } else if (scale_mode == ORACLE_SCALE_PER_TOKEN) {
    double amax = 0.0;
    for (int64_t k = 0; k < W; ++k)
      if (fabs(y[k]) > amax) amax = fabs(y[k]);
    const float st = (float)(amax / 448.0); /* stored fp32, one rounding */
    for (int64_t k = 0; k < W; ++k)
      put_fp8(&dst[k], st == 0.0f ? y[k] : y[k] / (double)st);
    token_scales[row] = st;
  } else {
    return ORACLE_BAD_ARG;
  }
  return ORACLE_OK;
}

int oracle_mla_rope_rmsnorm_quant(
    void* q_out, int q_out_type, const void* q_in, int q_in_type, const uint16_t* latent,
    const uint32_t* row_offsets, const uint32_t* cache_lengths, int64_t B,
    const uint32_t* page_table, int64_t pt_stride, const void* freqs, int freq_type,
    int64_t max_seq_len, const void* gamma, int gamma_type, float epsilon, int64_t H,
    int64_t R, int64_t Dn, void* cache, int cache_type, int64_t num_layers,
    int64_t num_pages, int64_t page_size, int64_t layer_idx, int scale_mode,
    float tensor_scale, float* token_scales) {
  if (R <= 0 || R % 2 || Dn <= 0 || H < 0 || B < 0 || layer_idx < 0 ||
      layer_idx >= num_layers || page_size <= 0)
    return ORACLE_BAD_ARG;
  if (!latent && cache_type != ORACLE_CACHE_BF16) return ORACLE_BAD_ARG;
  double g[4096];
  if (Dn + R > 4096 || R > 1024) return ORACLE_BAD_ARG;
  for (int64_t k = 0; k < Dn; ++k) g[k] = elem(gamma, k, gamma_type);
  const double eps = (double)epsilon; /* the fp32 value, widened exactly */
  int status = ORACLE_OK;

  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = row_offsets[b]; t < (int64_t)row_offsets[b + 1]; ++t) {
      const int64_t j = t - (int64_t)row_offsets[b];
      const int64_t pos = (int64_t)cache_lengths[b] + j;
      const int64_t slot = pos;
      if (pos >= max_seq_len) { status = ORACLE_BAD_POSITION; continue; }
      const int64_t page = page_of(page_table, pt_stride, num_pages,
                                   page_size, b, slot);
      if (page < 0) { status = ORACLE_BAD_PAGE; continue; }
      const int64_t off = slot % page_size;
      const int64_t row = ((layer_idx * num_pages + page) * page_size + off);
      const int rc = mla_token(q_out, q_out_type, q_in, q_in_type, latent, t, pos, row,
                               freqs, freq_type, g, eps, H, R, Dn, cache, cache_type,
                               scale_mode, tensor_scale, token_scales);
      if (rc != ORACLE_OK) return rc;
    }
  }
  return status;
}

/*
 * Placement of every new token of a ragged batch, written out once: the
 * request of token t (t = o[b] + j), its cache slot and RoPE position
 * c[b] + j, and the slot's physical page and offset (the addressing of [MLA]
 * Args: input_row_offsets, the cache's lengths and page table).
 *   plan  u32 [T][4]: (page, offset, position, 1) for a placed token;
 *         (0, 0, 0, 0) for a token no request owns (t >= o[B]) or whose
 *         slot has no page-table entry or a page id past the pool.
 * Positions are not compared with a freqs table here.
 */
int oracle_token_plan(uint32_t* plan, int64_t T, const uint32_t* row_offsets,
                      const uint32_t* cache_lengths, int64_t B, const uint32_t* page_table,
                      int64_t pt_stride, int64_t num_pages, int64_t page_size) {
  if (T < 0 || B < 0 || page_size <= 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < 4 * T; ++i) plan[i] = 0;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = row_offsets[b]; t < (int64_t)row_offsets[b + 1] && t < T; ++t) {
      const int64_t slot = (int64_t)cache_lengths[b] + (t - (int64_t)row_offsets[b]);
      const int64_t page = page_of(page_table, pt_stride, num_pages, page_size, b, slot);
      if (page < 0) continue;
      plan[4 * t] = (uint32_t)page;
      plan[4 * t + 1] = (uint32_t)(slot % page_size);
      plan[4 * t + 2] = (uint32_t)slot;
      plan[4 * t + 3] = 1;
    }
  }
  return ORACLE_OK;
}

/*
 * Fused MLA step placed by a token plan: token t is rotated at position
 * plan[t][2] and its row stored at (page plan[t][0], offset plan[t][1]) of
 * layer layer_idx.  A token whose entry is not marked placed, whose position
 * is not below max_seq_len, or whose page or offset lies outside the pool is
 * skipped (nothing written; the return value reports it).  Other arguments
 * as for oracle_mla_rope_rmsnorm_quant; latent = NULL is the in-place form on
 * a bf16 cache (each row read from the cell it is written back to).
 */
int oracle_mla_rope_rmsnorm_quant_planned(
    void* q_out, int q_out_type, const void* q_in, int q_in_type, const uint16_t* latent,
    const uint32_t* plan, int64_t T, const void* freqs, int freq_type, int64_t max_seq_len,
    const void* gamma, int gamma_type, float epsilon, int64_t H, int64_t R, int64_t Dn,
    void* cache,
    int cache_type, int64_t num_layers, int64_t num_pages, int64_t page_size,
    int64_t layer_idx, int scale_mode, float tensor_scale, float* token_scales) {
  if (R <= 0 || R % 2 || Dn <= 0 || H < 0 || T < 0 || layer_idx < 0 ||
      layer_idx >= num_layers || page_size <= 0)
    return ORACLE_BAD_ARG;
  if (!latent && cache_type != ORACLE_CACHE_BF16) return ORACLE_BAD_ARG;
  double g[4096];
  if (Dn + R > 4096 || R > 1024) return ORACLE_BAD_ARG;
  for (int64_t k = 0; k < Dn; ++k) g[k] = elem(gamma, k, gamma_type);
  const double eps = (double)epsilon;
  int status = ORACLE_OK;
  for (int64_t t = 0; t < T; ++t) {
    const uint32_t* e = plan + 4 * t;
    if (!plan_entry_placed(e, num_pages, page_size)) { status = ORACLE_BAD_PAGE; continue; }
    if ((int64_t)e[2] >= max_seq_len) { status = ORACLE_BAD_POSITION; continue; }
    const int64_t row = ((layer_idx * num_pages + e[0]) * page_size + e[1]);
    const int rc = mla_token(q_out, q_out_type, q_in, q_in_type, latent, t, (int64_t)e[2], row,
                             freqs, freq_type, g, eps, H, R, Dn, cache, cache_type, scale_mode,
                             tensor_scale, token_scales);
    if (rc != ORACLE_OK) return rc;
  }
  return status;
}

/*
 * In-place form ([GRAPH] fused_rope_rmsnorm_kernel; the fp8 prefill and
 * decode branches apply RoPE and RMSNorm to the key cache in place): the
 * latent row of every new token already sits in the bf16 cache at its slot
 * and is replaced by its normalised, rotated value; q as above.
 */
int oracle_mla_rope_rmsnorm_inplace(
    void* q_out, int q_out_type, const void* q_in, int q_in_type, const uint32_t* row_offsets,
    const uint32_t* cache_lengths, int64_t B, const uint32_t* page_table, int64_t pt_stride,
    const void* freqs, int freq_type, int64_t max_seq_len, const void* gamma, int gamma_type,
    float epsilon, int64_t H, int64_t R, int64_t Dn, uint16_t* cache, int64_t num_layers,
    int64_t num_pages, int64_t page_size, int64_t layer_idx) {
  return oracle_mla_rope_rmsnorm_quant(q_out, q_out_type, q_in, q_in_type, NULL, row_offsets,
                                       cache_lengths, B, page_table, pt_stride, freqs,
                                       freq_type, max_seq_len, gamma, gamma_type, epsilon, H,
                                       R, Dn, cache,
                                       ORACLE_CACHE_BF16, num_layers, num_pages, page_size,
                                       layer_idx, 0, 1.0f, NULL);
}

/*
 * Paged-ragged Q/K RoPE ([QK] summary, Parameters, Args).  Q is rotated out
 * of place into q_out; the K rows of the new tokens are rotated in place in
 * the bf16 cache of layer `layer_idx`.  With k_gamma non-NULL the K row of
 * every head is first RMS-normalised over its first k_norm_cols columns (the
 * optional per-head K norm), still unrounded, then rotated, then rounded once.
 *
 *   q_out, q_in   [T][Hq][D] of q_type ([QK] Parameters: dtype; bf16 or
 *                 fp16 bits, or fp32)
 *   k_cache       bf16 bits [L][P][S][Hkv][D], or fp8 codes (k_type)
 *   freqs         [max_seq_len][D] of freq_type ([QK] Parameters: freq_dtype)
 *   position_ids  u32 [T] or NULL (then position = cache length + index)
 *   k_gamma       bf16 bits [k_norm_cols] or NULL
 */
/* K row of one head, widened to binary64: bf16 bits, or fp8 code times the
 * row's scale. */
static void load_k_row(const void* k_cache, int k_type, int64_t elem, int64_t D,
                       double scale, double* a) {
  for (int64_t i = 0; i < D; ++i)
    a[i] = k_type == ORACLE_CACHE_BF16
               ? oracle_bf16_decode(((const uint16_t*)k_cache)[elem + i])
               : oracle_e4m3fn_decode(((const uint8_t*)k_cache)[elem + i]) * scale;
}

/* Write a processed K row back: bf16 round, or fp8 with the tensor scale, or
 * (per-token) with a fresh scale fp32(max|y| / 448) that is stored too.
 * Only the columns lo..hi-1 are written; the per-token statistic covers the
 * whole row (columns left as they were keep their own values, re-encoded). */
static void store_k_row(void* k_cache, int k_type, int scale_mode, int64_t elem, int64_t D,
                        const double* y, float tensor_scale, float* token_scale,
                        int64_t lo, int64_t hi) {
  if (k_type == ORACLE_CACHE_BF16) {
    for (int64_t i = lo; i < hi; ++i) ((uint16_t*)k_cache)[elem + i] = oracle_bf16_encode(y[i]);
    return;
  }
  double s = (double)tensor_scale;
  if (scale_mode == ORACLE_SCALE_PER_TOKEN) {
    double amax = 0.0;
    for (int64_t i = 0; i < D; ++i)
      if (fabs(y[i]) > amax) amax = fabs(y[i]);
    const float st = (float)(amax / 448.0);
    *token_scale = st;
    s = (double)st;
  }
  for (int64_t i = lo; i < hi; ++i)
    put_fp8(&((uint8_t*)k_cache)[elem + i], s == 0.0 ? y[i] : y[i] / s);
}

int oracle_qk_rope_paged_ragged(
    void* q_out, const void* q_in, int q_type, int64_t Hq, int64_t D,
    const uint32_t* row_offsets, const uint32_t* cache_lengths, int64_t B,
    const uint32_t* page_table, int64_t pt_stride, void* k_cache, int k_type,
    int scale_mode, float* k_scales, int64_t num_layers, int64_t num_pages,
    int64_t page_size, int64_t Hkv, int64_t layer_idx, const void* freqs, int freq_type,
    int64_t max_seq_len, const uint32_t* position_ids, const int64_t* mrope_section,
    int interleaved, const uint16_t* k_gamma, int64_t k_norm_cols, float epsilon) {
  if (D <= 0 || D % 2 || D > 1024 || layer_idx < 0 || layer_idx >= num_layers ||
      page_size <= 0 || (k_gamma && (k_norm_cols <= 0 || k_norm_cols > D)))
    return ORACLE_BAD_ARG;
  if (mrope_section && (!position_ids || mrope_section[0] < 0 || mrope_section[1] < 0 ||
                        mrope_section[2] < 0 ||
                        mrope_section[0] + mrope_section[1] + mrope_section[2] != D / 2))
    return ORACLE_BAD_ARG;
  double a[1024], r[1024], g[1024];
  int both[1024];     /* K norm: both members of the value's pair normalised */
  float frow[1024];
  float mixed[1024];  /* multimodal: per-pair cos/sin gathered from three rows */
  int64_t T = row_offsets[B];
  if (k_gamma)
    for (int64_t k = 0; k < k_norm_cols; ++k) g[k] = oracle_bf16_decode(k_gamma[k]);
  const double eps = (double)epsilon;
  int status = ORACLE_OK;

  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = row_offsets[b]; t < (int64_t)row_offsets[b + 1]; ++t) {
      const int64_t j = t - (int64_t)row_offsets[b];
      const int64_t slot = (int64_t)cache_lengths[b] + j;
      const int64_t pos = position_ids ? (int64_t)position_ids[t] : slot;
      if (pos >= max_seq_len) { status = ORACLE_BAD_POSITION; continue; }
      const int64_t page = page_of(page_table, pt_stride, num_pages,
                                   page_size, b, slot);
      if (page < 0) { status = ORACLE_BAD_PAGE; continue; }
      const int64_t off = slot % page_size;
      const float* fr = freqs_row_at(freqs, freq_type, pos, D, frow);
      if (mrope_section) {
        /* [QK] Parameters, mrope_section: pair i of section k (temporal,
         * height, width) is rotated by the angle of position row k. */
        int bad = 0;
        for (int64_t i = 0; i < D / 2; ++i) {
          const int64_t k = i < mrope_section[0] ? 0
                            : i < mrope_section[0] + mrope_section[1] ? 1 : 2;
          const int64_t pk = (int64_t)position_ids[k * T + t];
          if (pk >= max_seq_len) { bad = 1; break; }
          mixed[2 * i] = (float)elem(freqs, pk * D + 2 * i, freq_type);
          mixed[2 * i + 1] = (float)elem(freqs, pk * D + 2 * i + 1, freq_type);
        }
        if (bad) { status = ORACLE_BAD_POSITION; continue; }
        fr = mixed;
      }

      for (int64_t h = 0; h < Hq; ++h) {
        const int64_t base = (t * Hq + h) * D;
        for (int64_t i = 0; i < D; ++i) a[i] = elem(q_in, base + i, q_type);
        oracle_rope_row(a, r, D, fr, interleaved);
        for (int64_t i = 0; i < D; ++i) put_elem(q_out, base + i, q_type, r[i]);
      }
      for (int64_t h = 0; h < Hkv; ++h) {
        const int64_t head = ((layer_idx * num_pages + page) * page_size + off) * Hkv + h;
        const double ks = k_type == ORACLE_CACHE_FP8
            ? (double)(scale_mode == ORACLE_SCALE_PER_TOKEN ? k_scales[head] : k_scales[0])
            : 1.0;
        load_k_row(k_cache, k_type, head * D, D, ks, a);
        if (k_gamma) {
          /* [QK] the K norm, then the rotation.  The rotation is linear, so
           * a pair whose members are both normalised is rotated as x * gamma
           * and scaled by inv after it: the same value, and an exact
           * cancellation in the pair gives an exact zero, as the definition
           * does (scaling each member by its own rounded product first would
           * leave a binary64 residue there).  A pair with one normalised
           * member takes inv on that member before the rotation. */
          const double inv = oracle_inv_rms(a, k_norm_cols, eps);
          for (int64_t i = 0; i < D; ++i) {
            const int64_t partner = interleaved ? (i ^ 1) : (i + D / 2) % D;
            both[i] = i < k_norm_cols && partner < k_norm_cols;
            if (i < k_norm_cols) a[i] = both[i] ? a[i] * g[i] : a[i] * inv * g[i];
          }
          oracle_rope_row(a, r, D, fr, interleaved);
          for (int64_t i = 0; i < D; ++i)
            if (both[i]) r[i] *= inv;
        } else {
          oracle_rope_row(a, r, D, fr, interleaved);
        }
        store_k_row(k_cache, k_type, scale_mode, head * D, D, r,
                    k_type == ORACLE_CACHE_FP8 ? k_scales[0] : 1.0f,
                    scale_mode == ORACLE_SCALE_PER_TOKEN ? &k_scales[head] : NULL, 0, D);
      }
    }
  }
  return status;
}

/*
 * Gather of whole request contexts from the paged latent cache into a dense
 * buffer ([GRAPH] mla_prefill_branch_fp8: the latent values are copied from
 * the paged cache to a contiguous buffer and quantised to fp8 there).
 * Row kv_row_offsets[b] + j of `out` receives cache slot j of request b, for
 * j < kv_row_offsets[b+1] - kv_row_offsets[b].  Element conversions:
 *   fp8  -> fp8 : the code itself; per-token scales copied to out_scales[row]
 *   fp8  -> bf16: bf16_rne(decode(code) * scale), scale = the tensor scale or
 *                 the row's per-token scale
 *   bf16 -> bf16: the bits themselves
 *   bf16 -> fp8 : e4m3fn_sat_rne(value / out_tensor_scale)
 *
 *   out     [total_rows][W] of u8 (fp8) or u16 (bf16), dense
 *   cache   [L][P][S][W] of u8 (fp8) or u16 (bf16)
 *   cache_scales  fp8 cache: [1] (per-tensor) or [L][P][S] (per-token)
 */
int oracle_mla_gather_latent_paged(
    void* out, int out_type, float* out_scales, float out_tensor_scale,
    const uint32_t* kv_row_offsets, int64_t B, const uint32_t* page_table,
    int64_t pt_stride, const void* cache, int cache_type, int scale_mode,
    const float* cache_scales, int64_t W, int64_t num_layers, int64_t num_pages,
    int64_t page_size, int64_t layer_idx) {
  if (W <= 0 || layer_idx < 0 || layer_idx >= num_layers || page_size <= 0)
    return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t row = kv_row_offsets[b]; row < (int64_t)kv_row_offsets[b + 1]; ++row) {
      const int64_t slot = row - (int64_t)kv_row_offsets[b];
      const int64_t page = page_of(page_table, pt_stride, num_pages, page_size, b, slot);
      if (page < 0) { status = ORACLE_BAD_PAGE; continue; }
      const int64_t src_row = (layer_idx * num_pages + page) * page_size + slot % page_size;
      double scale = 1.0;
      if (cache_type == ORACLE_CACHE_FP8)
        scale = (double)(scale_mode == ORACLE_SCALE_PER_TOKEN ? cache_scales[src_row]
                                                               : cache_scales[0]);
      for (int64_t k = 0; k < W; ++k) {
        if (cache_type == ORACLE_CACHE_FP8) {
          const uint8_t code = ((const uint8_t*)cache)[src_row * W + k];
          if (out_type == ORACLE_CACHE_FP8)
            ((uint8_t*)out)[row * W + k] = code;
          else
            ((uint16_t*)out)[row * W + k] = oracle_bf16_encode(oracle_e4m3fn_decode(code) * scale);
        } else {
          const uint16_t bits = ((const uint16_t*)cache)[src_row * W + k];
          if (out_type == ORACLE_CACHE_BF16)
            ((uint16_t*)out)[row * W + k] = bits;
          else
            put_fp8(&((uint8_t*)out)[row * W + k],
                    oracle_bf16_decode(bits) / (double)out_tensor_scale);
        }
      }
      if (cache_type == ORACLE_CACHE_FP8 && out_type == ORACLE_CACHE_FP8 &&
          scale_mode == ORACLE_SCALE_PER_TOKEN && out_scales)
        out_scales[row] = cache_scales[src_row];
    }
  }
  return status;
}

/*
 * In-place RMSNorm of the new K-cache entries ([NORM] description): tokens
 * t < total_seq_len are mapped to (request, index) through row_offsets; each
 * head's first gamma_len columns are normalised with (gamma + weight_offset);
 * the other columns are left alone.  multiply_before_cast = 1 rounds once,
 * after the gamma product; = 0 rounds the normalised value to bf16 first,
 * then multiplies by (gamma + weight_offset) and rounds again.
 * per_head_norm = 1: one statistic per head; 0: one per token over all heads.
 *
 *   k_cache   bf16 bits [L][P][S][Hkv][D], or fp8 codes (k_type)
 *   gamma     [gamma_len] of gamma_type ([NORM]: the dtype of gamma and
 *             weight_offset; bf16 or fp16 bits, or fp32)
 */
/* The K-cache RMSNorm of one token whose rows sit at (page, off) of layer
 * layer_idx: every head's first gamma_len columns normalised with g (gamma
 * plus weight_offset, widened), in place. */
static void kv_norm_token(void* k_cache, int k_type, int scale_mode, float* k_scales,
                          int64_t num_pages, int64_t page_size, int64_t Hkv, int64_t D,
                          int64_t layer_idx, int64_t page, int64_t off, const double* g,
                          int64_t gamma_len, double eps, int multiply_before_cast,
                          int per_head_norm) {
  double a[1024];
  double token_inv = 0.0;
  if (!per_head_norm) {
    /* Reading of per_head_norm = False (listed on the page, not
     * described): one statistic over the first gamma_len columns of all
     * heads of the token. */
    double ss = 0.0;
    for (int64_t h = 0; h < Hkv; ++h) {
      const int64_t head = ((layer_idx * num_pages + page) * page_size + off) * Hkv + h;
      const double ks = k_type == ORACLE_CACHE_FP8
          ? (double)(scale_mode == ORACLE_SCALE_PER_TOKEN ? k_scales[head] : k_scales[0])
          : 1.0;
      load_k_row(k_cache, k_type, head * D, D, ks, a);
      for (int64_t i = 0; i < gamma_len; ++i) ss += a[i] * a[i];
    }
    token_inv = 1.0 / sqrt(ss / (double)(Hkv * gamma_len) + eps);
  }
  for (int64_t h = 0; h < Hkv; ++h) {
    const int64_t head = ((layer_idx * num_pages + page) * page_size + off) * Hkv + h;
    const double ks = k_type == ORACLE_CACHE_FP8
        ? (double)(scale_mode == ORACLE_SCALE_PER_TOKEN ? k_scales[head] : k_scales[0])
        : 1.0;
    load_k_row(k_cache, k_type, head * D, D, ks, a);
    double inv = per_head_norm ? oracle_inv_rms(a, gamma_len, eps) : token_inv;
    for (int64_t i = 0; i < gamma_len; ++i) {
      if (multiply_before_cast) {
        a[i] = a[i] * inv * g[i];
      } else {  /* bf16 only: round the normalised value, then apply gamma */
        a[i] = oracle_bf16_decode(oracle_bf16_encode(a[i] * inv)) * g[i];
      }
    }
    /* only the normalised columns are written (per-token: the fresh scale
     * covers the whole head, the other columns are re-encoded with it) */
    const int per_token = k_type == ORACLE_CACHE_FP8 && scale_mode == ORACLE_SCALE_PER_TOKEN;
    store_k_row(k_cache, k_type, scale_mode, head * D, D, a,
                k_type == ORACLE_CACHE_FP8 ? k_scales[0] : 1.0f,
                per_token ? &k_scales[head] : NULL, 0, per_token ? D : gamma_len);
  }
}

int oracle_rms_norm_kv_cache_paged(
    void* k_cache, int k_type, int scale_mode, float* k_scales, int64_t num_layers,
    int64_t num_pages, int64_t page_size, int64_t Hkv, int64_t D, int64_t layer_idx,
    const uint32_t* row_offsets, const uint32_t* cache_lengths, int64_t B,
    const uint32_t* page_table, int64_t pt_stride, const void* gamma, int gamma_type,
    int64_t gamma_len, float epsilon, float weight_offset, int64_t total_seq_len,
    int multiply_before_cast, int per_head_norm) {
  if (gamma_len <= 0 || gamma_len > D || D > 1024 || layer_idx < 0 ||
      layer_idx >= num_layers || page_size <= 0)
    return ORACLE_BAD_ARG;
  double g[1024];
  if (k_type == ORACLE_CACHE_FP8 && !multiply_before_cast) return ORACLE_BAD_ARG;
  kv_norm_gamma(gamma, gamma_type, gamma_len, weight_offset, g);
  const double eps = (double)epsilon;
  int status = ORACLE_OK;

  for (int64_t b = 0; b < B; ++b) {
    for (int64_t t = row_offsets[b]; t < (int64_t)row_offsets[b + 1]; ++t) {
      if (t >= total_seq_len) break;
      const int64_t slot = (int64_t)cache_lengths[b] + (t - (int64_t)row_offsets[b]);
      const int64_t page = page_of(page_table, pt_stride, num_pages,
                                   page_size, b, slot);
      if (page < 0) { status = ORACLE_BAD_PAGE; continue; }
      const int64_t off = slot % page_size;
      kv_norm_token(k_cache, k_type, scale_mode, k_scales, num_pages, page_size, Hkv, D,
                    layer_idx, page, off, g, gamma_len, eps, multiply_before_cast,
                    per_head_norm);
    }
  }
  return status;
}

/*
 * The K-cache RMSNorm with each token placed by a token plan
 * (oracle_token_plan): token t < total_seq_len is normalised at page
 * plan[t][0], offset plan[t][1]; an entry not marked placed, or with a page
 * or offset outside the pool, is skipped (reported by the return value).
 * Other arguments as for oracle_rms_norm_kv_cache_paged.
 */
int oracle_rms_norm_kv_cache_planned(
    void* k_cache, int k_type, int scale_mode, float* k_scales, int64_t num_layers,
    int64_t num_pages, int64_t page_size, int64_t Hkv, int64_t D, int64_t layer_idx,
    const uint32_t* plan, const void* gamma, int gamma_type, int64_t gamma_len, float epsilon,
    float weight_offset, int64_t total_seq_len, int multiply_before_cast, int per_head_norm) {
  if (gamma_len <= 0 || gamma_len > D || D > 1024 || layer_idx < 0 ||
      layer_idx >= num_layers || page_size <= 0 || total_seq_len < 0)
    return ORACLE_BAD_ARG;
  double g[1024];
  if (k_type == ORACLE_CACHE_FP8 && !multiply_before_cast) return ORACLE_BAD_ARG;
  kv_norm_gamma(gamma, gamma_type, gamma_len, weight_offset, g);
  const double eps = (double)epsilon;
  int status = ORACLE_OK;
  for (int64_t t = 0; t < total_seq_len; ++t) {
    const uint32_t* e = plan + 4 * t;
    if (!plan_entry_placed(e, num_pages, page_size)) { status = ORACLE_BAD_PAGE; continue; }
    kv_norm_token(k_cache, k_type, scale_mode, k_scales, num_pages, page_size, Hkv, D,
                  layer_idx, (int64_t)e[0], (int64_t)e[1], g, gamma_len, eps,
                  multiply_before_cast, per_head_norm);
  }
  return status;
}
