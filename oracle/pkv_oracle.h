/*
 * pkv_oracle.h -- the CPU oracle's exported functions (liboracle.so).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: declared for the oracle's own source
 * (so that the compiler checks every definition against it) and for the
 * plain C test client.  Nothing in the HIP library includes it.  The
 * functions' documentation sits with their definitions in pkv_oracle.c.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double oracle_bf16_decode(uint16_t bits);
uint16_t oracle_bf16_encode(double v);
double oracle_f16_decode(uint16_t bits);
uint16_t oracle_f16_encode(double v);
double oracle_e4m3fn_decode(uint8_t code);
uint8_t oracle_e4m3fn_encode_sat(double v);
void oracle_set_fp8_probe(const void* base, int64_t n, double* pre);
void oracle_rope_row(const double* x, double* out, int64_t dim, const float* freqs_row,
                     int interleaved);
double oracle_inv_rms(const double* x, int64_t n, double eps);
void oracle_rmsnorm_row(const double* x, double* y, int64_t n, const double* g, double eps);
int oracle_mla_rope_rmsnorm_quant(void* q_out, int q_out_type, const void* q_in, int q_in_type,
                                  const uint16_t* latent, const uint32_t* row_offsets,
                                  const uint32_t* cache_lengths, int64_t B,
                                  const uint32_t* page_table, int64_t pt_stride,
                                  const void* freqs, int freq_type, int64_t max_seq_len,
                                  const void* gamma, int gamma_type, float epsilon, int64_t H,
                                  int64_t R, int64_t Dn, void* cache, int cache_type,
                                  int64_t num_layers, int64_t num_pages, int64_t page_size,
                                  int64_t layer_idx, int scale_mode, float tensor_scale,
                                  float* token_scales);
int oracle_token_plan(uint32_t* plan, int64_t T, const uint32_t* row_offsets,
                      const uint32_t* cache_lengths, int64_t B, const uint32_t* page_table,
                      int64_t pt_stride, int64_t num_pages, int64_t page_size);
int oracle_mla_rope_rmsnorm_quant_planned(void* q_out, int q_out_type, const void* q_in,
                                          int q_in_type, const uint16_t* latent,
                                          const uint32_t* plan, int64_t T, const void* freqs,
                                          int freq_type, int64_t max_seq_len, const void* gamma,
                                          int gamma_type, float epsilon, int64_t H, int64_t R,
                                          int64_t Dn, void* cache, int cache_type,
                                          int64_t num_layers, int64_t num_pages,
                                          int64_t page_size, int64_t layer_idx, int scale_mode,
                                          float tensor_scale, float* token_scales);
int oracle_mla_rope_rmsnorm_inplace(void* q_out, int q_out_type, const void* q_in, int q_in_type,
                                    const uint32_t* row_offsets, const uint32_t* cache_lengths,
                                    int64_t B, const uint32_t* page_table, int64_t pt_stride,
                                    const void* freqs, int freq_type, int64_t max_seq_len,
                                    const void* gamma, int gamma_type, float epsilon, int64_t H,
                                    int64_t R, int64_t Dn, uint16_t* cache, int64_t num_layers,
                                    int64_t num_pages, int64_t page_size, int64_t layer_idx);
int oracle_qk_rope_paged_ragged(void* q_out, const void* q_in, int q_type, int64_t Hq, int64_t D,
                                const uint32_t* row_offsets, const uint32_t* cache_lengths,
                                int64_t B, const uint32_t* page_table, int64_t pt_stride,
                                void* k_cache, int k_type, int scale_mode, float* k_scales,
                                int64_t num_layers, int64_t num_pages, int64_t page_size,
                                int64_t Hkv, int64_t layer_idx, const void* freqs, int freq_type,
                                int64_t max_seq_len, const uint32_t* position_ids,
                                const int64_t* mrope_section, int interleaved,
                                const uint16_t* k_gamma, int64_t k_norm_cols, float epsilon);
int oracle_mla_gather_latent_paged(void* out, int out_type, float* out_scales,
                                   float out_tensor_scale, const uint32_t* kv_row_offsets,
                                   int64_t B, const uint32_t* page_table, int64_t pt_stride,
                                   const void* cache, int cache_type, int scale_mode,
                                   const float* cache_scales, int64_t W, int64_t num_layers,
                                   int64_t num_pages, int64_t page_size, int64_t layer_idx);
int oracle_rms_norm_kv_cache_paged(void* k_cache, int k_type, int scale_mode, float* k_scales,
                                   int64_t num_layers, int64_t num_pages, int64_t page_size,
                                   int64_t Hkv, int64_t D, int64_t layer_idx,
                                   const uint32_t* row_offsets, const uint32_t* cache_lengths,
                                   int64_t B, const uint32_t* page_table, int64_t pt_stride,
                                   const void* gamma, int gamma_type, int64_t gamma_len,
                                   float epsilon, float weight_offset, int64_t total_seq_len,
                                   int multiply_before_cast, int per_head_norm);
int oracle_rms_norm_kv_cache_planned(void* k_cache, int k_type, int scale_mode, float* k_scales,
                                     int64_t num_layers, int64_t num_pages, int64_t page_size,
                                     int64_t Hkv, int64_t D, int64_t layer_idx,
                                     const uint32_t* plan, const void* gamma, int gamma_type,
                                     int64_t gamma_len, float epsilon, float weight_offset,
                                     int64_t total_seq_len, int multiply_before_cast,
                                     int per_head_norm);

#ifdef __cplusplus
}
#endif

#endif /* PKV_ORACLE_H */
