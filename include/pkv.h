/*
 * pkv.h -- C ABI of the paged-KV pre-attention library (gfx950 / MI355X).
 *
 * Ten entry points, each one stream-ordered kernel launch (but one, below):
 *
 *   mla_rope_rmsnorm_quant   fused MLA step: RoPE on q_rope, RMSNorm on the
 *                            latent row's non-rope part, RoPE on its rope tail,
 *                            FP8 E4M3FN quantisation, paged cache write.
 *                            Page "mla_fused_rope_rmsnorm_quantization"
 *                            (summary, Args) and the
 *                            fused_rope_rmsnorm_quantization_kernel entry of
 *                            the "mla_graph" module page.
 *   mla_rope_rmsnorm_inplace the same step on a bf16 cache that already
 *                            holds the latent rows, in place
 *                            (fused_rope_rmsnorm_kernel and the first two
 *                            steps of mla_prefill_branch_fp8 /
 *                            mla_decode_branch_fp8, "mla_graph" module page).
 *   pkv_token_plan           each new token's cache placement (page, offset,
 *                            position), written once per batch layout, and
 *   mla_rope_rmsnorm_quant_planned, mla_rope_rmsnorm_inplace_planned
 *                            the fused MLA step (buffer and in-place forms)
 *                            placed by such a plan (the same page's
 *                            addressing, split so that every layer of a model
 *                            step reuses it).
 *   mla_rope_rmsnorm_quant_noalloc
 *                            the planned step with its plan in a static device
 *                            array, for callers that cannot allocate (two
 *                            launches when it builds the plan).
 *   qk_rope_paged_ragged     RoPE on Q (out of place) and on the new K rows of a
 *                            paged cache (in place), optional per-head K
 *                            RMSNorm fused in front of the K rotation.
 *                            Page "generic_fused_qk_rope_bshd_paged_ragged".
 *   rms_norm_kv_cache_paged  in-place RMSNorm of the new K-cache rows, and
 *   rms_norm_kv_cache_paged_planned
 *                            the same placed by a token plan.
 *                            Page "rms_norm_kv_cache_ragged_paged".
 *   mla_gather_latent_paged  copy of whole request contexts from the paged
 *                            latent cache into a dense buffer, with fp8
 *                            dequantisation / quantisation on the way (the
 *                            paged-to-contiguous copy and fp8 quantisation
 *                            steps of mla_prefill_branch_fp8, "mla_graph"
 *                            module page).
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Pointers are DEVICE pointers unless marked (host).  Element types: bf16 and
 * fp16 are stored as their 16-bit patterns, fp8 as its byte; which type a q,
 * freqs_cis or gamma array holds is given by the call's pkv_elem_types (NULL:
 * the defaults); "stride" arguments count elements, not bytes, and the
 * innermost dimension is always contiguous.
 *
 * Ragged batch: input_row_offsets[0..batch] (device, u32) is non-decreasing
 * with input_row_offsets[0] = 0 and input_row_offsets[batch] = total tokens;
 * request b owns tokens input_row_offsets[b] .. input_row_offsets[b+1]-1.
 * Token j of request b (counted from 0) goes to cache slot
 * cache_lengths[b] + j, where cache_lengths[b] is the request's length before
 * this step; slot s lives in physical page page_table[b*stride + s/page_size]
 * at offset s % page_size.  Without explicit position ids the token's RoPE
 * position equals its slot.
 *
 * freqs_cis: [max_seq_len][dim] (fp32 unless the call's types say bf16 or
 * fp16), row p holds for pair i the cosine in column 2i and the sine in
 * column 2i+1 of the angle p * theta_i.
 *
 * Ownership: the caller allocates and frees every buffer.  The library
 * allocates nothing, keeps no state between calls (except the plan array of
 * mla_rope_rmsnorm_quant_noalloc), never synchronises and may be called from
 * several host threads.  Outputs may alias their inputs only
 * exactly (q_out == q_in); partial overlap is undefined.
 *
 * Errors: every entry point returns PKV_OK (0) or a pkv_status.  All argument
 * checks run on the host before anything is enqueued; on error nothing is
 * enqueued and no memory is touched.  PKV_ERR_LAUNCH reports a refused launch.
 * Faults inside the kernel surface at the caller's next synchronisation.
 *
 * Device-data rules the host cannot check (offsets monotone, positions below
 * max_seq_len, page-table entries below num_pages, table wide enough for every
 * slot, no two tokens mapped to one slot): the kernels check the first four
 * per token before dereferencing anything derived from them; a token that
 * fails a check is skipped entirely (no output written for it) and, when the
 * cache descriptor carries an error counter, the counter is incremented once
 * per skipped token.  Tokens sharing a slot race (undefined result).
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = 2,       /* sizes inconsistent with each other */
  PKV_ERR_DTYPE = 3,       /* element type not accepted by this entry point */
  PKV_ERR_ALIGN = 4,       /* pointer or stride breaks the 16-byte rule */
  PKV_ERR_UNSUPPORTED = 5, /* valid request that this library does not implement */
  PKV_ERR_RANGE = 6,       /* index argument out of range (e.g. layer_idx) */
  PKV_ERR_LAUNCH = 7       /* the HIP runtime refused the kernel launch */
} pkv_status;

typedef enum pkv_dtype {
  PKV_DTYPE_BF16 = 0,
  PKV_DTYPE_FP8_E4M3FN = 1, /* OCP FP8 E4M3FN: bias 7, max 448, no inf */
  PKV_DTYPE_F32 = 2,        /* IEEE binary32 */
  PKV_DTYPE_F16 = 3         /* IEEE binary16 */
} pkv_dtype;

/*
 * Element types of a call's q, q output, freqs_cis and gamma tensors (the
 * pages' dtype, out_rope_dtype, freq_dtype and gamma_dtype parameters).  A
 * NULL pointer in place of the struct means the defaults in brackets.
 *   q       q_rope of the MLA step, q_proj and the Q output of the Q/K RoPE:
 *           PKV_DTYPE_BF16 or PKV_DTYPE_F16 [BF16]
 *   q_out   q_rope_output of the MLA step: BF16, F16 or F32 [BF16]
 *           (the Q/K RoPE writes its output in the type of q)
 *   freqs   freqs_cis: F32, BF16 or F16 [F32]
 *   gamma   gamma of the MLA step and of the K-cache RMSNorm: BF16, F16 or
 *           F32 [BF16] (the Q/K RoPE's optional K-norm gamma is BF16 only)
 * Another value returns PKV_ERR_DTYPE.  The latent row is always bf16 (the
 * MLA page's latent input yields bfloat16 values).
 */
typedef struct pkv_elem_types {
  int32_t q;
  int32_t q_out;
  int32_t freqs;
  int32_t gamma;
} pkv_elem_types;

typedef enum pkv_scale_mode {
  PKV_SCALE_NONE = 0,       /* bf16 cache, no quantisation */
  PKV_SCALE_PER_TENSOR = 1, /* scales[0] (read only): one dequant multiplier */
  PKV_SCALE_PER_TOKEN = 2   /* scales[layer][page][slot][head] written per row:
                               max|row| / 448 rounded to fp32 */
} pkv_scale_mode;

/*
 * A paged cache for all layers (the collection's role on the pages: one pool
 * of pages per layer, retrieved by layer_idx).  Element (layer, page, slot,
 * head, d) sits at data + layer*layer_stride + page*page_stride +
 * slot*slot_stride + head*head_stride + d (element units, d contiguous).
 * Host struct; the pointers inside it are device pointers.
 */
typedef struct pkv_paged_cache {
  void* data;                     /* pool base, 16-byte aligned */
  int32_t dtype;                  /* pkv_dtype */
  uint32_t num_layers;
  uint32_t num_pages;             /* pages per layer */
  uint32_t page_size;             /* slots per page (> 0) */
  uint32_t num_heads;             /* heads per slot */
  uint32_t head_dim;              /* elements per head */
  int64_t layer_stride, page_stride, slot_stride, head_stride; /* elements */
  const uint32_t* cache_lengths;  /* [batch] prior length of each request */
  const uint32_t* page_table;     /* [batch][page_table_stride] page ids */
  uint32_t page_table_stride;     /* entries per request row (>= 1) */
  int32_t scale_mode;             /* pkv_scale_mode */
  float* scales;                  /* PER_TENSOR: [1]; PER_TOKEN: dense
                                     [num_layers][num_pages][page_size][num_heads] */
  uint32_t* error_count;          /* optional (may be NULL): skipped tokens */
} pkv_paged_cache;

/*
 * Fused MLA pre-attention step.  For every token t (request b, index j,
 * position p = cache_lengths[b] + j):
 *   q_rope_out[t,h,:] = RoPE_p(q_rope[t,h,:]) for every head h, rotate-half
 *                       pairs (i, i + rope_dim/2), fp32 math, one rounding
 *                       into the output type;
 *   y[0:kv_norm_dim]  = x * r * gamma,  r = 1/sqrt(mean(x^2) + epsilon),
 *                       x = kv_latent[t, 0:kv_norm_dim];
 *   y[kv_norm_dim: ]  = RoPE_p(kv_latent[t, kv_norm_dim:kv_norm_dim+rope_dim]);
 *   cache[layer_idx][page][slot][0][:] = E4M3FN_sat_rne(y / scale)  (fp8) or
 *                                        bf16_rne(y)                  (bf16).
 * Per-token scale mode writes scale = fp32(max|y| / 448) beside the row.
 *
 *   q_rope_out      [total_tokens][num_heads][rope_dim] of types->q_out (bf16,
 *                   fp16 or fp32: the pages' out_rope_dtype), strides
 *                   qo_tok_stride / qo_head_stride (elements, 16-byte
 *                   multiples)
 *   q_rope          types->q (bf16 or fp16), same shape, strides
 *                   qi_tok_stride / qi_head_stride
 *   kv_latent       bf16 [total_tokens][kv_norm_dim + rope_dim], row stride
 *                   kv_row_stride (multiple of 8)
 *   input_row_offsets u32 [batch_size + 1]
 *   total_tokens    (host) number of new tokens = input_row_offsets[batch_size]
 *   freqs_cis       [max_seq_len][rope_dim] of types->freqs (fp32, bf16, fp16)
 *   gamma           [kv_norm_dim] of types->gamma (bf16, fp16, fp32)
 *   types           (host) element types, or NULL (bf16 q and q output, fp32
 *                   freqs_cis, bf16 gamma); see pkv_elem_types
 *   kv_cache        (host) descriptor: dtype FP8_E4M3FN with scale mode
 *                   PER_TENSOR or PER_TOKEN, or BF16 with scale mode NONE;
 *                   num_heads 1, head_dim kv_norm_dim + rope_dim
 *   stream          hipStream_t to enqueue on (NULL = default stream)
 * Supported here: rope_dim 32, 64 or 128; kv_norm_dim a multiple of 8 up to
 * 512 (the pages leave both open: gamma [kv_norm_dim], q_rope [..,
 * rope_dim]); any num_heads >= 0; q head strides up to 2^27 elements.  Other
 * sizes return PKV_ERR_UNSUPPORTED.  The cache row (kv_norm_dim + rope_dim
 * elements) must keep the descriptor's strides 16-byte multiples.
 */
int mla_rope_rmsnorm_quant(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                           const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                           const void* kv_latent, int64_t kv_row_stride,
                           const uint32_t* input_row_offsets, uint32_t batch_size,
                           uint32_t total_tokens, uint32_t num_heads, uint32_t rope_dim,
                           uint32_t kv_norm_dim, const void* freqs_cis, uint32_t max_seq_len,
                           const void* gamma, float epsilon, const pkv_paged_cache* kv_cache,
                           uint32_t layer_idx, const pkv_elem_types* types, void* stream);

/*
 * Fused MLA pre-attention step in place on a bf16 latent cache ("mla_graph"
 * module page: fused_rope_rmsnorm_kernel applies RoPE to q and RMSNorm to the
 * cache; the fp8 prefill and decode branches apply RoPE and RMSNorm to the
 * key cache in place).  Identical to mla_rope_rmsnorm_quant with a BF16 cache,
 * except that x is read from the cache row the result replaces:
 *   x = cache[layer_idx][page][slot][0][:]   (bf16, written earlier by the
 *                                             caller at the token's slot)
 *   cache[layer_idx][page][slot][0][:] = bf16_rne(y)
 * Arguments as for mla_rope_rmsnorm_quant, without kv_latent / kv_row_stride;
 * kv_cache must be dtype BF16 with scale mode NONE (else PKV_ERR_DTYPE).
 * Rows of tokens that fail a device-data check are neither read nor written.
 * Same supported sizes.
 */
int mla_rope_rmsnorm_inplace(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                             const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                             const uint32_t* input_row_offsets, uint32_t batch_size,
                             uint32_t total_tokens, uint32_t num_heads, uint32_t rope_dim,
                             uint32_t kv_norm_dim, const void* freqs_cis, uint32_t max_seq_len,
                             const void* gamma, float epsilon, const pkv_paged_cache* kv_cache,
                             uint32_t layer_idx, const pkv_elem_types* types, void* stream);

/*
 * Token plan: the placement of every new token of a ragged batch, written
 * once so that the fused MLA step of every layer can read it instead of
 * resolving it again (page "mla_fused_rope_rmsnorm_quantization", Args:
 * input_row_offsets and the KV collection's cache lengths and page table;
 * every layer of a model step shares them).
 *
 *   token_plan      u32 [total_tokens][4], written, 16-byte aligned: for token
 *                   t of request b (index j) the entry (page, offset,
 *                   position, 1) with position = slot = cache_lengths[b] + j,
 *                   page = page_table[b][slot / page_size], offset =
 *                   slot % page_size.  A token that no request owns, or
 *                   whose slot has no page-table column or a page id not
 *                   below num_pages, gets (0, 0, 0, 0).
 *   input_row_offsets u32 [batch_size + 1], total_tokens (host) as for
 *                   mla_rope_rmsnorm_quant
 *   cache           (host) descriptor: cache_lengths, page_table,
 *                   page_table_stride, page_size and num_pages are read; the
 *                   pool itself and the error counter are not touched
 * Positions are not compared with a freqs table here (the planned step does
 * that).  The plan stays valid while the batch layout, the cache lengths and
 * the page table are unchanged.
 */
int pkv_token_plan(uint32_t* token_plan, const uint32_t* input_row_offsets,
                   uint32_t batch_size, uint32_t total_tokens, const pkv_paged_cache* cache,
                   void* stream);

/*
 * The fused MLA step of mla_rope_rmsnorm_quant with each token placed by a
 * token plan: token t is rotated at position token_plan[t][2] and its row
 * written at page token_plan[t][0], offset token_plan[t][1] of layer
 * layer_idx.  With the plan pkv_token_plan wrote for the same batch the
 * results equal mla_rope_rmsnorm_quant's bit for bit.  A token whose entry
 * is not marked placed (fourth word 0), whose position is not below
 * max_seq_len, or whose page or offset lies outside the pool is skipped and
 * counted like a device-data failure.
 *
 *   token_plan      u32 [total_tokens][4], 16-byte aligned
 * Other arguments as for mla_rope_rmsnorm_quant (same shapes, dtypes and
 * supported sizes); the cache descriptor's cache_lengths and page_table are
 * not read and may be NULL.
 */
int mla_rope_rmsnorm_quant_planned(void* q_rope_out, int64_t qo_tok_stride,
                                   int64_t qo_head_stride, const void* q_rope,
                                   int64_t qi_tok_stride, int64_t qi_head_stride,
                                   const void* kv_latent, int64_t kv_row_stride,
                                   const uint32_t* token_plan, uint32_t total_tokens,
                                   uint32_t num_heads, uint32_t rope_dim, uint32_t kv_norm_dim,
                                   const void* freqs_cis, uint32_t max_seq_len,
                                   const void* gamma, float epsilon,
                                   const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                                   const pkv_elem_types* types, void* stream);

/*
 * mla_rope_rmsnorm_inplace with each token placed by a token plan: the row at
 * page token_plan[t][0], offset token_plan[t][1] of layer layer_idx is read,
 * normalised, rotated at position token_plan[t][2] and written back there.
 * With the plan pkv_token_plan wrote for the same batch the results equal
 * mla_rope_rmsnorm_inplace's bit for bit.  Skipped entries as for
 * mla_rope_rmsnorm_quant_planned (their rows are neither read nor written).
 *
 *   token_plan      u32 [total_tokens][4], 16-byte aligned
 * Other arguments as for mla_rope_rmsnorm_inplace; the descriptor's
 * cache_lengths and page_table are not read and may be NULL.
 */
int mla_rope_rmsnorm_inplace_planned(void* q_rope_out, int64_t qo_tok_stride,
                                     int64_t qo_head_stride, const void* q_rope,
                                     int64_t qi_tok_stride, int64_t qi_head_stride,
                                     const uint32_t* token_plan, uint32_t total_tokens,
                                     uint32_t num_heads, uint32_t rope_dim,
                                     uint32_t kv_norm_dim, const void* freqs_cis,
                                     uint32_t max_seq_len, const void* gamma, float epsilon,
                                     const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                                     const pkv_elem_types* types, void* stream);

/*
 * mla_rope_rmsnorm_quant_planned without a caller-allocated plan, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The token plan lives in a
 * static array the library holds on every device it runs on (2^18 entries of
 * 16 bytes = 4 MiB per device, kept until the process ends); the call
 * allocates nothing and calls no allocating routine.
 *
 *   build_plan != 0  write the plan of this batch (input_row_offsets,
 *                    batch_size and the descriptor's cache_lengths and
 *                    page_table, as pkv_token_plan would) into the array of
 *                    the stream's device, then run the planned step from it:
 *                    two stream-ordered launches.
 *   build_plan == 0  run the planned step from the plan the last call with
 *                    build_plan != 0 built on that device (for the other
 *                    layers of the same batch layout); input_row_offsets and
 *                    batch_size are not read.  PKV_ERR_SHAPE when that plan
 *                    has fewer tokens than total_tokens (or none was built).
 * Results equal mla_rope_rmsnorm_quant_planned's with the plan pkv_token_plan
 * writes for the same batch, bit for bit.  Other arguments, shapes and
 * supported sizes as for mla_rope_rmsnorm_quant.  total_tokens above 2^18
 * returns PKV_ERR_UNSUPPORTED.  A call with total_tokens = 0 enqueues nothing
 * but resolves the array's address on the stream's device, so that a caller
 * can make it before capturing a graph.
 * Every call on one device shares that device's array and it keeps the last
 * build's contents: calls that overlap on one device (other streams, other
 * host threads) race, and a build_plan == 0 call reads whatever the last
 * build on that device wrote.
 */
int mla_rope_rmsnorm_quant_noalloc(void* q_rope_out, int64_t qo_tok_stride,
                                   int64_t qo_head_stride, const void* q_rope,
                                   int64_t qi_tok_stride, int64_t qi_head_stride,
                                   const void* kv_latent, int64_t kv_row_stride,
                                   const uint32_t* input_row_offsets, uint32_t batch_size,
                                   uint32_t total_tokens, uint32_t num_heads, uint32_t rope_dim,
                                   uint32_t kv_norm_dim, const void* freqs_cis,
                                   uint32_t max_seq_len, const void* gamma, float epsilon,
                                   const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                                   const pkv_elem_types* types, int build_plan, void* stream);

/*
 * Paged-ragged fused Q/K RoPE.  Q is rotated into q_out; the K rows of the
 * new tokens (slot cache_lengths[b] + j) are rotated in place for every KV
 * head.  Position = position_ids[t] when position_ids != NULL, else the slot.
 * Multimodal RoPE (mrope_section != NULL, three host values summing to
 * head_dim/2: temporal, height, width pair counts): position_ids is
 * [3][total_tokens] and pair i is rotated by the angle of the row of its
 * section (page "generic_fused_qk_rope_bshd_paged_ragged", Parameters, names
 * mrope_section but gives no position layout: the three-row layout, and the
 * sections taken in that order over the pairs, are the reading taken).
 * interleaved != 0 rotates adjacent pairs (2i, 2i+1), otherwise pairs
 * (i, i + head_dim/2); pair i always uses freqs_cis columns 2i, 2i+1.
 * With k_norm_gamma != NULL, each K head's first k_norm_cols columns are
 * first RMS-normalised with gamma (fp32, unrounded), then the row is
 * rotated and rounded to bf16 once.
 *
 *   q_out, q_proj   types->q (bf16 or fp16) [total_tokens][num_q_heads]
 *                   [head_dim] with strides
 *   k_cache         (host) descriptor, head_dim == the q head_dim: dtype
 *                   BF16 with scale mode NONE, or FP8_E4M3FN with
 *                   PER_TENSOR (K = code * scales[0], re-encoded with the
 *                   same scale) or PER_TOKEN (K = code * the slot/head
 *                   scale; after the rotation the head's scale is replaced
 *                   by max|y| / 448 and the head re-encoded with it)
 *   freqs_cis       [max_seq_len][head_dim] of types->freqs (fp32, bf16, fp16)
 *   position_ids    u32 [total_tokens] or NULL ([3][total_tokens] with
 *                   mrope_section)
 *   mrope_section   (host) u32 [3] or NULL
 *   k_norm_gamma    bf16 [k_norm_cols] or NULL; 0 < k_norm_cols <= head_dim
 *   types           (host) element types or NULL (bf16 q, fp32 freqs_cis);
 *                   types->q_out must equal types->q, and types->gamma must
 *                   be bf16 when k_norm_gamma is given (PKV_ERR_DTYPE
 *                   otherwise)
 * Supported here: head_dim 64, 80, 96, 128 or 256; q and K head strides up
 * to 2^27 elements (else PKV_ERR_UNSUPPORTED).
 */
int qk_rope_paged_ragged(void* q_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                         const void* q_proj, int64_t qi_tok_stride, int64_t qi_head_stride,
                         uint32_t total_tokens, uint32_t num_q_heads, uint32_t head_dim,
                         const uint32_t* input_row_offsets, uint32_t batch_size,
                         const pkv_paged_cache* k_cache, uint32_t layer_idx,
                         const void* freqs_cis, uint32_t max_seq_len,
                         const uint32_t* position_ids, const uint32_t* mrope_section,
                         int interleaved, const void* k_norm_gamma, uint32_t k_norm_cols,
                         float epsilon, const pkv_elem_types* types, void* stream);

/*
 * In-place RMSNorm of the new K-cache rows.  Tokens t < total_seq_len (host
 * value) are mapped to (request, index) through input_row_offsets; for every
 * head the first gamma_len columns become x * r * (gamma + weight_offset)
 * with r = 1/sqrt(mean over those columns of x^2 + epsilon); the remaining
 * columns are not written.  multiply_before_cast != 0 rounds to bf16 once,
 * after the gamma product; 0 rounds x * r to bf16, then multiplies by
 * (gamma + weight_offset) and rounds again.
 *
 *   k_cache        (host) descriptor: BF16 + NONE, or FP8_E4M3FN with
 *                  PER_TENSOR (normalised columns re-encoded with the tensor
 *                  scale) or PER_TOKEN (the head's scale becomes max|y| / 448
 *                  and the whole head is re-encoded with it); fp8 caches
 *                  need multiply_before_cast != 0
 *   gamma          [gamma_len] of types->gamma (bf16, fp16, fp32),
 *                  0 < gamma_len <= head_dim
 *   types          (host) element types or NULL; only types->gamma is read
 *   per_head_norm  non-zero: one statistic per head; 0: one statistic per
 *                  token over the first gamma_len columns of all its heads
 *                  (the page lists the flag without describing it; this is
 *                  the reading taken)
 * Supported here: head_dim 64, 80, 96, 128 or 256, any number of heads with
 * either statistic.
 */
int rms_norm_kv_cache_paged(const pkv_paged_cache* k_cache, uint32_t layer_idx,
                            const void* gamma, uint32_t gamma_len, float epsilon,
                            float weight_offset, uint32_t total_seq_len,
                            const uint32_t* input_row_offsets, uint32_t batch_size,
                            int per_head_norm, int multiply_before_cast,
                            const pkv_elem_types* types, void* stream);

/*
 * rms_norm_kv_cache_paged with each token placed by a token plan (see
 * pkv_token_plan): token t < total_seq_len is normalised in the rows at page
 * token_plan[t][0], offset token_plan[t][1] of layer layer_idx.  With the plan
 * pkv_token_plan wrote for the same batch the result equals
 * rms_norm_kv_cache_paged's bit for bit.  An entry not marked placed, or whose
 * page or offset lies outside the pool, is skipped and counted.
 *
 *   token_plan      u32 [>= total_seq_len][4], 16-byte aligned
 * Other arguments as for rms_norm_kv_cache_paged; the descriptor's
 * cache_lengths and page_table are not read and may be NULL.  Same supported
 * sizes.
 */
int rms_norm_kv_cache_paged_planned(const pkv_paged_cache* k_cache, uint32_t layer_idx,
                                    const void* gamma, uint32_t gamma_len, float epsilon,
                                    float weight_offset, uint32_t total_seq_len,
                                    const uint32_t* token_plan, int per_head_norm,
                                    int multiply_before_cast, const pkv_elem_types* types,
                                    void* stream);

/*
 * Gather of request contexts from the paged latent cache.  For request b and
 * j < kv_row_offsets[b+1] - kv_row_offsets[b], row kv_row_offsets[b] + j of
 * out receives cache slot j of request b (layer layer_idx), converted:
 *   fp8 cache  -> fp8 out : the codes; with per-token cache scales the row's
 *                           scale is also written to out_scales[row]
 *   fp8 cache  -> bf16 out: bf16_rne(decode(code) * scale), scale = the
 *                           tensor scale or the row's per-token scale
 *   bf16 cache -> bf16 out: the bits
 *   bf16 cache -> fp8 out : E4M3FN_sat_rne(value / out_scale[0])
 *
 *   out             [total_rows][head_dim] of out_dtype, row stride
 *                   out_row_stride (elements; 16-byte multiple)
 *   out_dtype       PKV_DTYPE_FP8_E4M3FN or PKV_DTYPE_BF16
 *   out_scales      fp32 [total_rows], written for fp8 -> fp8 with per-token
 *                   scales; may be NULL otherwise
 *   out_scale       fp32 [1], read for bf16 -> fp8; may be NULL otherwise
 *   kv_row_offsets  u32 [batch_size + 1], prefix sums of context lengths
 *   total_rows      (host) kv_row_offsets[batch_size]
 *   cache           (host) latent cache descriptor, one head; its
 *                   cache_lengths field is not used
 * Rows whose slot has no valid page are skipped (not written) and counted.
 * Supported here: head_dim * element size a multiple of 16 bytes, at most
 * 1 KiB (fp8) / 2 KiB (bf16).
 */
int mla_gather_latent_paged(void* out, int32_t out_dtype, int64_t out_row_stride,
                            float* out_scales, const float* out_scale,
                            const uint32_t* kv_row_offsets, uint32_t batch_size,
                            uint32_t total_rows, const pkv_paged_cache* cache,
                            uint32_t layer_idx, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
