// pkv_internal.h -- kernel argument blocks and launchers (host side of the
// kernels).  The C ABI in pkv_api.cpp validates arguments, fills these
// blocks and calls the launchers; nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct pkv_paged_cache;  // include/pkv.h
struct pkv_elem_types;   // include/pkv.h

namespace pkv {

// K cache element encoding of the sibling entry points.
enum class KMode : int { Bf16 = 0, Fp8PerTensor = 1, Fp8PerToken = 2 };

// Paged cache geometry of one layer, in elements of the cache type.
struct CacheView {
  void* layer_base;            // data + layer_idx * layer_stride (in bytes)
  int64_t page_stride, slot_stride, head_stride;
  uint32_t num_pages, page_size, num_heads;
  const uint32_t* cache_lengths;
  const uint32_t* page_table;
  uint32_t pt_stride;
  uint32_t* error_count;
};

// Latent row source and cache encoding of the MLA kernel: from the latent
// buffer into an fp8 (tensor / token scale) or bf16 cache, or in place on a
// bf16 cache that already holds the row.
enum class MlaOut : int { Fp8PerTensor = 0, Fp8PerToken = 1, Bf16 = 2, Bf16InPlace = 3 };

// q_rope / q_rope_output element types of the MLA kernel (a template
// parameter): bf16 or fp16 in, bf16, fp16 or fp32 out.
enum class QIO : int { B_B = 0, B_H, B_F, H_H, H_B, H_F };

struct MlaArgs {
  void* q_out;                 // of the QIO output type
  QIO qio;
  int freq_type, gamma_type;   // ElemType of freqs_cis and gamma
  int64_t qo_tok, qo_head;
  const uint16_t* q_in;        // bf16 or fp16 bits
  int64_t qi_tok, qi_head;
  const uint16_t* latent;      // unused in place
  int64_t kv_row;
  const uint32_t* offsets;
  uint32_t batch;
  uint32_t total_tokens;
  uint32_t num_heads;
  uint32_t chunks;             // waves per token (head chunks)
  uint32_t rope_dim;           // 32, 64 or 128
  uint32_t nope_chunks;        // kv_norm_dim / 8 (at most 64)
  float inv_dn;                // 1 / kv_norm_dim, rounded to fp32
  const void* freqs;           // [max_seq_len][rope_dim] of freq_type
  uint32_t max_seq_len;
  const void* gamma;           // [kv_norm_dim] of gamma_type
  float epsilon;
  const float* tensor_scale;   // per-tensor mode: device scalar
  float* token_scales;         // per-token mode: this layer's [pages][page_size][heads]
  CacheView cache;
  const uint32_t* plan;        // [total_tokens][4] (page, offset, position, placed), or
                               // null: placement from offsets, lengths and page table
};

// Heads per MLA wave for a q with `heads` heads of rope_dim values; launch_mla
// takes that value.  The rope and non-rope widths the kernel is built for.
uint32_t mla_heads_per_wave(uint32_t heads, uint32_t rope_dim);
bool mla_rope_dim_supported(uint32_t rope_dim);
bool mla_nope_dim_supported(uint32_t kv_norm_dim);
hipError_t launch_mla(const MlaArgs& a, MlaOut mode, int heads_per_wave, hipStream_t stream);

// A validated MLA launch (pkv_api.cpp): its argument block, cache encoding
// and heads per wave; `empty` when there is nothing to launch.
struct MlaLaunch {
  MlaArgs args;
  MlaOut mode;
  int heads_per_wave;
  bool empty;
};

// Per-token placement of a ragged batch (token_plan.hip).
struct PlanArgs {
  uint32_t* plan;                // [total_tokens][4] written
  const uint32_t* offsets;
  uint32_t batch;
  uint32_t total_tokens;
  const uint32_t* cache_lengths;
  const uint32_t* page_table;
  uint32_t pt_stride, num_pages, page_size;
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);

struct QkArgs {
  uint16_t* q_out;               // bf16 or fp16 bits, the type of q_in
  int64_t qo_tok, qo_head;
  const uint16_t* q_in;
  int64_t qi_tok, qi_head;
  uint32_t total_tokens, num_q_heads;
  uint32_t chunks;               // waves per token (Q head chunks)
  const uint32_t* offsets;
  uint32_t batch;
  const void* freqs;             // [max_seq_len][head_dim] of freq_type
  int freq_type;                 // ElemType
  uint32_t max_seq_len;
  const uint32_t* position_ids;  // may be null; [3][total_tokens] with mrope
  uint32_t mrope;                // 1: multimodal RoPE with the two section ends below
  uint32_t mrope_end0, mrope_end1;  // pairs [0,end0) temporal, [end0,end1) height, rest width
  const uint16_t* k_gamma;       // may be null
  uint32_t k_norm_cols;
  float inv_norm_cols;           // 1 / k_norm_cols, rounded to fp32 (0 without a norm)
  float epsilon;
  float* k_scales;               // fp8 K: tensor scale [1] or this layer's per-token scales
  CacheView cache;               // K cache
};

// Q heads one wave of the Q/K kernel handles (head_dim 64, 80, 96, 128, 256).
uint32_t qk_heads_per_wave(int head_dim);
hipError_t launch_qk_rope(const QkArgs& a, int head_dim, bool interleaved, bool q_f16,
                          KMode kmode, hipStream_t stream);

struct KvNormArgs {
  uint32_t total_tokens;
  const uint32_t* offsets;
  uint32_t batch;
  const void* gamma;             // [gamma_len] of gamma_type
  int gamma_type;                // ElemType
  uint32_t gamma_len;
  float inv_cols;                // 1 / gamma_len, rounded to fp32
  float inv_token_cols;          // 1 / (gamma_len * heads): the per-token mean
  bool per_head;                 // false: one statistic per token over all heads
  float epsilon, weight_offset;
  float* k_scales;               // fp8 K: tensor scale [1] or this layer's per-token scales
  CacheView cache;               // K cache
  uint32_t head_dim;
  const uint32_t* plan;          // [total_tokens][4] token plan, or null: placement
                                 // from offsets, lengths and page table
};

hipError_t launch_kv_norm(const KvNormArgs& a, bool multiply_before_cast, KMode kmode,
                          hipStream_t stream);

struct GatherArgs {
  void* out;
  int64_t out_row_bytes;        // output row stride in bytes
  float* out_scales;            // per-token scale copy target (may be null)
  const float* out_scale;       // bf16 -> fp8 per-tensor scale (may be null)
  const uint32_t* kv_row_offsets;
  uint32_t batch;
  uint32_t total_rows;
  uint32_t row_bytes;           // cache row size in bytes (head_dim * element size)
  const float* cache_scale;     // fp8 cache: per-tensor [1] or this layer's per-token scales
  CacheView cache;
};

enum class GatherKind : int { Fp8ToFp8 = 0, Fp8ToBf16 = 1, Bf16ToBf16 = 2, Bf16ToFp8 = 3 };

hipError_t launch_gather(const GatherArgs& a, GatherKind kind, bool per_token, hipStream_t stream);

// The planned MLA step's and the token plan's host checks, filling their
// argument blocks without launching (pkv_api.cpp); each returns the status the
// corresponding entry point would return before enqueueing anything.
int mla_prepare_planned(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                        const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                        const void* kv_latent, int64_t kv_row_stride,
                        const uint32_t* token_plan, uint32_t total_tokens, uint32_t num_heads,
                        uint32_t rope_dim, uint32_t kv_norm_dim, const void* freqs_cis,
                        uint32_t max_seq_len, const void* gamma, float epsilon,
                        const ::pkv_paged_cache* kv_cache, uint32_t layer_idx,
                        const ::pkv_elem_types* types, MlaLaunch* out);
int plan_prepare(uint32_t* token_plan, const uint32_t* input_row_offsets, uint32_t batch_size,
                 uint32_t total_tokens, const ::pkv_paged_cache* cache, PlanArgs* out);
// A launch's status code (PKV_OK or PKV_ERR_LAUNCH).
int status_of(hipError_t e);

}  // namespace pkv
