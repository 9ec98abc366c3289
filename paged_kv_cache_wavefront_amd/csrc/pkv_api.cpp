// pkv_api.cpp -- the exported C ABI (include/pkv.h): host-side argument
// validation, kernel selection and launch.  Every check runs before anything
// is enqueued; no entry point allocates, synchronises or keeps state.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace {

using pkv::CacheView;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Head strides the kernels add to per-lane 32-bit byte offsets (up to 7
// heads away, 4-byte elements): at most 2^27 elements.
constexpr int64_t kMaxHeadStride = int64_t(1) << 27;
bool mult(int64_t v, int64_t k) { return v >= 0 && v % k == 0; }

size_t elem_bytes(int32_t dtype) { return dtype == PKV_DTYPE_BF16 ? 2 : 1; }

// Checks common to every cache descriptor; fills the per-layer view.
int check_cache(const pkv_paged_cache* c, uint32_t layer_idx, uint32_t batch_size,
                CacheView* view, bool need_lengths = true) {
  if (c == nullptr) return PKV_ERR_NULL;
  if (c->dtype != PKV_DTYPE_BF16 && c->dtype != PKV_DTYPE_FP8_E4M3FN) return PKV_ERR_DTYPE;
  if (c->num_layers == 0 || c->num_pages == 0 || c->page_size == 0 || c->num_heads == 0 ||
      c->head_dim == 0 || c->page_table_stride == 0)
    return PKV_ERR_SHAPE;
  if (layer_idx >= c->num_layers) return PKV_ERR_RANGE;
  if (batch_size > 0 && ((need_lengths && c->cache_lengths == nullptr) || c->page_table == nullptr))
    return PKV_ERR_NULL;
  if (c->data == nullptr) return PKV_ERR_NULL;
  // Every 16-byte vector access stays aligned when the pool base and every
  // stride are multiples of 16 bytes.
  const int64_t per16 = 16 / (int64_t)elem_bytes(c->dtype);
  if (!aligned16(c->data) || !mult(c->layer_stride, per16) || !mult(c->page_stride, per16) ||
      !mult(c->slot_stride, per16) || !mult(c->head_stride, per16))
    return PKV_ERR_ALIGN;
  view->layer_base = static_cast<char*>(c->data) +
                     (int64_t)layer_idx * c->layer_stride * (int64_t)elem_bytes(c->dtype);
  view->page_stride = c->page_stride;
  view->slot_stride = c->slot_stride;
  view->head_stride = c->head_stride;
  view->num_pages = c->num_pages;
  view->page_size = c->page_size;
  view->num_heads = c->num_heads;
  view->cache_lengths = c->cache_lengths;
  view->page_table = c->page_table;
  view->pt_stride = c->page_table_stride;
  view->error_count = c->error_count;
  return PKV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

// A call's element types, NULL standing for the defaults.
pkv_elem_types types_or_default(const pkv_elem_types* t) {
  if (t != nullptr) return *t;
  return pkv_elem_types{PKV_DTYPE_BF16, PKV_DTYPE_BF16, PKV_DTYPE_F32, PKV_DTYPE_BF16};
}
bool is_16bit_float(int32_t t) { return t == PKV_DTYPE_BF16 || t == PKV_DTYPE_F16; }
bool is_float(int32_t t) { return is_16bit_float(t) || t == PKV_DTYPE_F32; }

// The MLA kernel's q input / output pair; false if it is not one it is built for.
bool qio_of(int32_t q, int32_t q_out, pkv::QIO* out) {
  if (!is_16bit_float(q) || !is_float(q_out)) return false;
  const bool h = q == PKV_DTYPE_F16;
  if (q_out == PKV_DTYPE_BF16) *out = h ? pkv::QIO::H_B : pkv::QIO::B_B;
  else if (q_out == PKV_DTYPE_F16) *out = h ? pkv::QIO::H_H : pkv::QIO::B_H;
  else *out = h ? pkv::QIO::H_F : pkv::QIO::B_F;
  return true;
}

// Head dims the Q/K RoPE and K-norm kernels are built for.
bool sibling_head_dim(uint32_t d) { return d == 64 || d == 80 || d == 96 || d == 128 || d == 256; }

// Element encoding of a K cache for the sibling entry points; false if the
// dtype / scale-mode pair is not one of bf16 + none, fp8 + tensor / token.
bool k_mode_of(const pkv_paged_cache* c, pkv::KMode* km) {
  if (c->dtype == PKV_DTYPE_BF16 && c->scale_mode == PKV_SCALE_NONE) {
    *km = pkv::KMode::Bf16;
  } else if (c->dtype == PKV_DTYPE_FP8_E4M3FN && c->scale_mode == PKV_SCALE_PER_TENSOR) {
    *km = pkv::KMode::Fp8PerTensor;
  } else if (c->dtype == PKV_DTYPE_FP8_E4M3FN && c->scale_mode == PKV_SCALE_PER_TOKEN) {
    *km = pkv::KMode::Fp8PerToken;
  } else {
    return false;
  }
  return true;
}

// fp8 K scales: the tensor scale, or this layer's per-token (slot, head) block.
float* k_scales_of(const pkv_paged_cache* c, uint32_t layer_idx, pkv::KMode km) {
  if (km == pkv::KMode::Fp8PerToken)
    return c->scales + (int64_t)layer_idx * c->num_pages * c->page_size * c->num_heads;
  return c->scales;
}

// The latent row comes from kv_latent, or (in_place) from the bf16 cache row
// it is written back to.
// Both MLA entry points and the planned form: placement from the ragged
// batch (input_row_offsets, the cache's lengths and page table) or, when
// `planned`, from token_plan alone.
// With `prepared` set, the call only validates and fills *prepared (no launch).
int mla_entry(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
              const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
              const void* kv_latent, int64_t kv_row_stride, bool in_place, bool planned,
              const uint32_t* token_plan,
              const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t total_tokens,
              uint32_t num_heads, uint32_t rope_dim, uint32_t kv_norm_dim,
              const void* freqs_cis, uint32_t max_seq_len, const void* gamma, float epsilon,
              const pkv_paged_cache* kv_cache, uint32_t layer_idx, const pkv_elem_types* types,
              void* stream, pkv::MlaLaunch* prepared = nullptr) {
  if (prepared != nullptr) prepared->empty = true;
  if (kv_cache == nullptr) return PKV_ERR_NULL;
  const pkv_elem_types ty = types_or_default(types);
  pkv::QIO qio;
  if (!qio_of(ty.q, ty.q_out, &qio) || !is_float(ty.freqs) || !is_float(ty.gamma))
    return PKV_ERR_DTYPE;
  const int64_t qo_align = ty.q_out == PKV_DTYPE_F32 ? 4 : 8;  // 16 bytes in elements
  if (rope_dim == 0 || rope_dim % 2 != 0 || kv_norm_dim == 0) return PKV_ERR_SHAPE;
  if (kv_cache->num_heads != 1 || kv_cache->head_dim != kv_norm_dim + rope_dim)
    return PKV_ERR_SHAPE;
  if (!pkv::mla_rope_dim_supported(rope_dim) || !pkv::mla_nope_dim_supported(kv_norm_dim))
    return PKV_ERR_UNSUPPORTED;
  pkv::MlaOut mode;
  if (kv_cache->dtype == PKV_DTYPE_FP8_E4M3FN && kv_cache->scale_mode == PKV_SCALE_PER_TENSOR)
    mode = pkv::MlaOut::Fp8PerTensor;
  else if (kv_cache->dtype == PKV_DTYPE_FP8_E4M3FN && kv_cache->scale_mode == PKV_SCALE_PER_TOKEN)
    mode = pkv::MlaOut::Fp8PerToken;
  else if (kv_cache->dtype == PKV_DTYPE_BF16 && kv_cache->scale_mode == PKV_SCALE_NONE)
    mode = in_place ? pkv::MlaOut::Bf16InPlace : pkv::MlaOut::Bf16;
  else
    return PKV_ERR_DTYPE;
  if (in_place && mode != pkv::MlaOut::Bf16InPlace) return PKV_ERR_DTYPE;
  if (!planned && total_tokens > 0 && batch_size == 0) return PKV_ERR_SHAPE;
  if (max_seq_len == 0) return PKV_ERR_SHAPE;
  CacheView view{};
  // the planned form reads neither the cache lengths nor the page table
  int st = check_cache(kv_cache, layer_idx, planned ? 0u : batch_size, &view);
  if (st != PKV_OK) return st;
  if (total_tokens == 0) return PKV_OK;

  if ((planned ? token_plan == nullptr : input_row_offsets == nullptr) ||
      freqs_cis == nullptr || gamma == nullptr || (!in_place && kv_latent == nullptr))
    return PKV_ERR_NULL;
  if (planned && !aligned16(token_plan)) return PKV_ERR_ALIGN;
  if (num_heads > 0 && (q_rope == nullptr || q_rope_out == nullptr)) return PKV_ERR_NULL;
  const bool fp8 = mode == pkv::MlaOut::Fp8PerTensor || mode == pkv::MlaOut::Fp8PerToken;
  if (fp8 && kv_cache->scales == nullptr) return PKV_ERR_NULL;
  if (!aligned16(q_rope) || !aligned16(q_rope_out) || !aligned16(gamma) ||
      !aligned16(freqs_cis) || !mult(qo_tok_stride, qo_align) ||
      !mult(qo_head_stride, qo_align) || !mult(qi_tok_stride, 8) || !mult(qi_head_stride, 8))
    return PKV_ERR_ALIGN;
  if (!in_place && (!aligned16(kv_latent) || !mult(kv_row_stride, 8))) return PKV_ERR_ALIGN;
  if (qi_head_stride > kMaxHeadStride || qo_head_stride > kMaxHeadStride)
    return PKV_ERR_UNSUPPORTED;

  pkv::MlaArgs a{};
  a.q_out = q_rope_out;
  a.qio = qio;
  a.freq_type = ty.freqs;
  a.gamma_type = ty.gamma;
  a.qo_tok = qo_tok_stride;
  a.qo_head = qo_head_stride;
  a.q_in = static_cast<const uint16_t*>(q_rope);
  a.qi_tok = qi_tok_stride;
  a.qi_head = qi_head_stride;
  a.latent = in_place ? nullptr : static_cast<const uint16_t*>(kv_latent);
  a.kv_row = in_place ? 0 : kv_row_stride;
  a.offsets = planned ? nullptr : input_row_offsets;
  a.batch = planned ? 0u : batch_size;
  a.plan = planned ? token_plan : nullptr;
  a.total_tokens = total_tokens;
  a.num_heads = num_heads;
  const int hpw = (int)pkv::mla_heads_per_wave(num_heads, rope_dim);
  a.chunks = num_heads == 0 ? 1u : (num_heads + (uint32_t)hpw - 1) / (uint32_t)hpw;
  a.rope_dim = rope_dim;
  a.nope_chunks = kv_norm_dim / 8;
  a.inv_dn = (float)(1.0 / (double)kv_norm_dim);
  a.freqs = freqs_cis;
  a.max_seq_len = max_seq_len;
  a.gamma = gamma;
  a.epsilon = epsilon;
  a.tensor_scale = kv_cache->scales;
  a.token_scales = nullptr;
  if (mode == pkv::MlaOut::Fp8PerToken)
    a.token_scales = kv_cache->scales + (int64_t)layer_idx * kv_cache->num_pages *
                                            kv_cache->page_size * kv_cache->num_heads;
  a.cache = view;
  if (prepared != nullptr) {
    *prepared = pkv::MlaLaunch{a, mode, hpw, false};
    return PKV_OK;
  }
  return launch_status(pkv::launch_mla(a, mode, hpw, static_cast<hipStream_t>(stream)));
}

// pkv_token_plan's checks; fills *out.
int plan_entry(uint32_t* token_plan, const uint32_t* input_row_offsets, uint32_t batch_size,
               uint32_t total_tokens, const pkv_paged_cache* cache, pkv::PlanArgs* out) {
  if (cache == nullptr) return PKV_ERR_NULL;
  if (cache->num_pages == 0 || cache->page_size == 0 || cache->page_table_stride == 0)
    return PKV_ERR_SHAPE;
  if (total_tokens > 0 && batch_size == 0) return PKV_ERR_SHAPE;
  *out = pkv::PlanArgs{};
  if (total_tokens == 0) return PKV_OK;
  if (token_plan == nullptr || input_row_offsets == nullptr || cache->cache_lengths == nullptr ||
      cache->page_table == nullptr)
    return PKV_ERR_NULL;
  if (!aligned16(token_plan)) return PKV_ERR_ALIGN;
  out->plan = token_plan;
  out->offsets = input_row_offsets;
  out->batch = batch_size;
  out->total_tokens = total_tokens;
  out->cache_lengths = cache->cache_lengths;
  out->page_table = cache->page_table;
  out->pt_stride = cache->page_table_stride;
  out->num_pages = cache->num_pages;
  out->page_size = cache->page_size;
  return PKV_OK;
}

}  // namespace

namespace pkv {

int mla_prepare_planned(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                        const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                        const void* kv_latent, int64_t kv_row_stride,
                        const uint32_t* token_plan, uint32_t total_tokens, uint32_t num_heads,
                        uint32_t rope_dim, uint32_t kv_norm_dim, const void* freqs_cis,
                        uint32_t max_seq_len, const void* gamma, float epsilon,
                        const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                        const pkv_elem_types* types, MlaLaunch* out) {
  return mla_entry(q_rope_out, qo_tok_stride, qo_head_stride, q_rope, qi_tok_stride,
                   qi_head_stride, kv_latent, kv_row_stride, false, true, token_plan, nullptr,
                   0, total_tokens, num_heads, rope_dim, kv_norm_dim, freqs_cis, max_seq_len,
                   gamma, epsilon, kv_cache, layer_idx, types, nullptr, out);
}

int plan_prepare(uint32_t* token_plan, const uint32_t* input_row_offsets, uint32_t batch_size,
                 uint32_t total_tokens, const pkv_paged_cache* cache, PlanArgs* out) {
  return plan_entry(token_plan, input_row_offsets, batch_size, total_tokens, cache, out);
}

int status_of(hipError_t e) { return launch_status(e); }

}  // namespace pkv

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_NULL: return "PKV_ERR_NULL: a required pointer is NULL";
    case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE: inconsistent sizes";
    case PKV_ERR_DTYPE: return "PKV_ERR_DTYPE: element type not accepted";
    case PKV_ERR_ALIGN: return "PKV_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: not implemented for these sizes";
    case PKV_ERR_RANGE: return "PKV_ERR_RANGE: index argument out of range";
    case PKV_ERR_LAUNCH: return "PKV_ERR_LAUNCH: kernel launch refused";
    default: return "unknown pkv status";
  }
}

int mla_rope_rmsnorm_quant(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                           const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                           const void* kv_latent, int64_t kv_row_stride,
                           const uint32_t* input_row_offsets, uint32_t batch_size,
                           uint32_t total_tokens, uint32_t num_heads, uint32_t rope_dim,
                           uint32_t kv_norm_dim, const void* freqs_cis, uint32_t max_seq_len,
                           const void* gamma, float epsilon, const pkv_paged_cache* kv_cache,
                           uint32_t layer_idx, const pkv_elem_types* types, void* stream) {
  return mla_entry(q_rope_out, qo_tok_stride, qo_head_stride, q_rope, qi_tok_stride,
                   qi_head_stride, kv_latent, kv_row_stride, false, false, nullptr,
                   input_row_offsets, batch_size, total_tokens, num_heads, rope_dim,
                   kv_norm_dim, freqs_cis, max_seq_len, gamma, epsilon, kv_cache, layer_idx,
                   types, stream);
}

int pkv_token_plan(uint32_t* token_plan, const uint32_t* input_row_offsets,
                   uint32_t batch_size, uint32_t total_tokens, const pkv_paged_cache* cache,
                   void* stream) {
  pkv::PlanArgs a;
  const int st = plan_entry(token_plan, input_row_offsets, batch_size, total_tokens, cache, &a);
  if (st != PKV_OK || total_tokens == 0) return st;
  return launch_status(pkv::launch_plan(a, static_cast<hipStream_t>(stream)));
}

int mla_rope_rmsnorm_inplace_planned(void* q_rope_out, int64_t qo_tok_stride,
                                     int64_t qo_head_stride, const void* q_rope,
                                     int64_t qi_tok_stride, int64_t qi_head_stride,
                                     const uint32_t* token_plan, uint32_t total_tokens,
                                     uint32_t num_heads, uint32_t rope_dim,
                                     uint32_t kv_norm_dim, const void* freqs_cis,
                                     uint32_t max_seq_len, const void* gamma, float epsilon,
                                     const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                                     const pkv_elem_types* types, void* stream) {
  return mla_entry(q_rope_out, qo_tok_stride, qo_head_stride, q_rope, qi_tok_stride,
                   qi_head_stride, nullptr, 0, true, true, token_plan, nullptr, 0, total_tokens,
                   num_heads, rope_dim, kv_norm_dim, freqs_cis, max_seq_len, gamma, epsilon,
                   kv_cache, layer_idx, types, stream);
}

int mla_rope_rmsnorm_quant_planned(void* q_rope_out, int64_t qo_tok_stride,
                                   int64_t qo_head_stride, const void* q_rope,
                                   int64_t qi_tok_stride, int64_t qi_head_stride,
                                   const void* kv_latent, int64_t kv_row_stride,
                                   const uint32_t* token_plan, uint32_t total_tokens,
                                   uint32_t num_heads, uint32_t rope_dim, uint32_t kv_norm_dim,
                                   const void* freqs_cis, uint32_t max_seq_len,
                                   const void* gamma, float epsilon,
                                   const pkv_paged_cache* kv_cache, uint32_t layer_idx,
                                   const pkv_elem_types* types, void* stream) {
  return mla_entry(q_rope_out, qo_tok_stride, qo_head_stride, q_rope, qi_tok_stride,
                   qi_head_stride, kv_latent, kv_row_stride, false, true, token_plan, nullptr,
                   0, total_tokens, num_heads, rope_dim, kv_norm_dim, freqs_cis, max_seq_len,
                   gamma, epsilon, kv_cache, layer_idx, types, stream);
}

int mla_rope_rmsnorm_inplace(void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                             const void* q_rope, int64_t qi_tok_stride, int64_t qi_head_stride,
                             const uint32_t* input_row_offsets, uint32_t batch_size,
                             uint32_t total_tokens, uint32_t num_heads, uint32_t rope_dim,
                             uint32_t kv_norm_dim, const void* freqs_cis, uint32_t max_seq_len,
                             const void* gamma, float epsilon, const pkv_paged_cache* kv_cache,
                             uint32_t layer_idx, const pkv_elem_types* types, void* stream) {
  return mla_entry(q_rope_out, qo_tok_stride, qo_head_stride, q_rope, qi_tok_stride,
                   qi_head_stride, nullptr, 0, true, false, nullptr, input_row_offsets,
                   batch_size, total_tokens, num_heads, rope_dim, kv_norm_dim, freqs_cis,
                   max_seq_len, gamma, epsilon, kv_cache, layer_idx, types, stream);
}

int qk_rope_paged_ragged(void* q_out, int64_t qo_tok_stride, int64_t qo_head_stride,
                         const void* q_proj, int64_t qi_tok_stride, int64_t qi_head_stride,
                         uint32_t total_tokens, uint32_t num_q_heads, uint32_t head_dim,
                         const uint32_t* input_row_offsets, uint32_t batch_size,
                         const pkv_paged_cache* k_cache, uint32_t layer_idx,
                         const void* freqs_cis, uint32_t max_seq_len,
                         const uint32_t* position_ids, const uint32_t* mrope_section,
                         int interleaved, const void* k_norm_gamma, uint32_t k_norm_cols,
                         float epsilon, const pkv_elem_types* types, void* stream) {
  if (k_cache == nullptr) return PKV_ERR_NULL;
  const pkv_elem_types ty = types_or_default(types);
  if (!is_16bit_float(ty.q) || ty.q_out != ty.q || !is_float(ty.freqs) ||
      (k_norm_gamma != nullptr && ty.gamma != PKV_DTYPE_BF16))
    return PKV_ERR_DTYPE;
  if (mrope_section != nullptr &&
      (uint64_t)mrope_section[0] + mrope_section[1] + mrope_section[2] != head_dim / 2)
    return PKV_ERR_SHAPE;
  if (head_dim == 0 || head_dim % 2 != 0 || k_cache->head_dim != head_dim) return PKV_ERR_SHAPE;
  pkv::KMode km;
  if (!k_mode_of(k_cache, &km)) return PKV_ERR_DTYPE;
  if (k_norm_gamma != nullptr && (k_norm_cols == 0 || k_norm_cols > head_dim))
    return PKV_ERR_SHAPE;
  if (!sibling_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (total_tokens > 0 && batch_size == 0) return PKV_ERR_SHAPE;
  if (max_seq_len == 0) return PKV_ERR_SHAPE;
  CacheView view{};
  int st = check_cache(k_cache, layer_idx, batch_size, &view);
  if (st != PKV_OK) return st;
  if (total_tokens == 0) return PKV_OK;
  if (input_row_offsets == nullptr || freqs_cis == nullptr) return PKV_ERR_NULL;
  if (num_q_heads > 0 && (q_proj == nullptr || q_out == nullptr)) return PKV_ERR_NULL;
  if (km != pkv::KMode::Bf16 && k_cache->scales == nullptr) return PKV_ERR_NULL;
  if (mrope_section != nullptr && position_ids == nullptr) return PKV_ERR_NULL;
  if (!aligned16(q_proj) || !aligned16(q_out) || !aligned16(freqs_cis) ||
      !aligned16(k_norm_gamma) || !mult(qo_tok_stride, 8) || !mult(qo_head_stride, 8) ||
      !mult(qi_tok_stride, 8) || !mult(qi_head_stride, 8))
    return PKV_ERR_ALIGN;
  if (qi_head_stride > kMaxHeadStride || qo_head_stride > kMaxHeadStride ||
      k_cache->head_stride > kMaxHeadStride)
    return PKV_ERR_UNSUPPORTED;

  pkv::QkArgs a{};
  a.q_out = static_cast<uint16_t*>(q_out);
  a.qo_tok = qo_tok_stride;
  a.qo_head = qo_head_stride;
  a.q_in = static_cast<const uint16_t*>(q_proj);
  a.qi_tok = qi_tok_stride;
  a.qi_head = qi_head_stride;
  a.total_tokens = total_tokens;
  a.num_q_heads = num_q_heads;
  const uint32_t qhpw = pkv::qk_heads_per_wave((int)head_dim);
  a.chunks = num_q_heads == 0 ? 1u : (num_q_heads + qhpw - 1) / qhpw;
  a.offsets = input_row_offsets;
  a.batch = batch_size;
  a.freqs = freqs_cis;
  a.freq_type = ty.freqs;
  a.max_seq_len = max_seq_len;
  a.position_ids = position_ids;
  a.mrope = mrope_section != nullptr;
  if (a.mrope) {
    a.mrope_end0 = mrope_section[0];
    a.mrope_end1 = mrope_section[0] + mrope_section[1];
  }
  a.k_gamma = static_cast<const uint16_t*>(k_norm_gamma);
  a.k_norm_cols = k_norm_gamma ? k_norm_cols : 0;
  a.inv_norm_cols = k_norm_gamma ? (float)(1.0 / (double)k_norm_cols) : 0.0f;
  a.epsilon = epsilon;
  a.k_scales = k_scales_of(k_cache, layer_idx, km);
  a.cache = view;
  return launch_status(pkv::launch_qk_rope(a, (int)head_dim, interleaved != 0,
                                           ty.q == PKV_DTYPE_F16, km,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Both K-norm entry points: placement from the ragged batch or, when
// `planned`, from token_plan alone.
int kv_norm_entry(const pkv_paged_cache* k_cache, uint32_t layer_idx, const void* gamma,
                  uint32_t gamma_len, float epsilon, float weight_offset,
                  uint32_t total_seq_len, bool planned, const uint32_t* token_plan,
                  const uint32_t* input_row_offsets, uint32_t batch_size, int per_head_norm,
                  int multiply_before_cast, const pkv_elem_types* types, void* stream) {
  if (k_cache == nullptr) return PKV_ERR_NULL;
  const int32_t gamma_type = types_or_default(types).gamma;
  if (!is_float(gamma_type)) return PKV_ERR_DTYPE;
  pkv::KMode km;
  if (!k_mode_of(k_cache, &km)) return PKV_ERR_DTYPE;
  if (gamma_len == 0 || gamma_len > k_cache->head_dim) return PKV_ERR_SHAPE;
  if (km != pkv::KMode::Bf16 && !multiply_before_cast) return PKV_ERR_UNSUPPORTED;
  if (!sibling_head_dim(k_cache->head_dim))
    return PKV_ERR_UNSUPPORTED;
  if (!planned && total_seq_len > 0 && batch_size == 0) return PKV_ERR_SHAPE;
  CacheView view{};
  int st = check_cache(k_cache, layer_idx, planned ? 0u : batch_size, &view);
  if (st != PKV_OK) return st;
  if (total_seq_len == 0) return PKV_OK;
  if (gamma == nullptr || (planned ? token_plan == nullptr : input_row_offsets == nullptr))
    return PKV_ERR_NULL;
  if (km != pkv::KMode::Bf16 && k_cache->scales == nullptr) return PKV_ERR_NULL;
  if (!aligned16(gamma) || (planned && !aligned16(token_plan))) return PKV_ERR_ALIGN;

  pkv::KvNormArgs a{};
  a.total_tokens = total_seq_len;
  a.offsets = planned ? nullptr : input_row_offsets;
  a.batch = planned ? 0u : batch_size;
  a.plan = planned ? token_plan : nullptr;
  a.gamma = gamma;
  a.gamma_type = gamma_type;
  a.gamma_len = gamma_len;
  a.inv_cols = (float)(1.0 / (double)gamma_len);
  a.inv_token_cols = (float)(1.0 / ((double)gamma_len * (double)k_cache->num_heads));
  a.per_head = per_head_norm != 0;
  a.epsilon = epsilon;
  a.weight_offset = weight_offset;
  a.k_scales = k_scales_of(k_cache, layer_idx, km);
  a.cache = view;
  a.head_dim = k_cache->head_dim;
  return launch_status(pkv::launch_kv_norm(a, multiply_before_cast != 0, km,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rms_norm_kv_cache_paged(const pkv_paged_cache* k_cache, uint32_t layer_idx,
                            const void* gamma, uint32_t gamma_len, float epsilon,
                            float weight_offset, uint32_t total_seq_len,
                            const uint32_t* input_row_offsets, uint32_t batch_size,
                            int per_head_norm, int multiply_before_cast,
                            const pkv_elem_types* types, void* stream) {
  return kv_norm_entry(k_cache, layer_idx, gamma, gamma_len, epsilon, weight_offset,
                       total_seq_len, false, nullptr, input_row_offsets, batch_size,
                       per_head_norm, multiply_before_cast, types, stream);
}

int rms_norm_kv_cache_paged_planned(const pkv_paged_cache* k_cache, uint32_t layer_idx,
                                    const void* gamma, uint32_t gamma_len, float epsilon,
                                    float weight_offset, uint32_t total_seq_len,
                                    const uint32_t* token_plan, int per_head_norm,
                                    int multiply_before_cast, const pkv_elem_types* types,
                                    void* stream) {
  return kv_norm_entry(k_cache, layer_idx, gamma, gamma_len, epsilon, weight_offset,
                       total_seq_len, true, token_plan, nullptr, 0, per_head_norm,
                       multiply_before_cast, types, stream);
}

int mla_gather_latent_paged(void* out, int32_t out_dtype, int64_t out_row_stride,
                            float* out_scales, const float* out_scale,
                            const uint32_t* kv_row_offsets, uint32_t batch_size,
                            uint32_t total_rows, const pkv_paged_cache* cache,
                            uint32_t layer_idx, void* stream) {
  if (cache == nullptr) return PKV_ERR_NULL;
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_FP8_E4M3FN) return PKV_ERR_DTYPE;
  const bool in_fp8 = cache->dtype == PKV_DTYPE_FP8_E4M3FN;
  const bool out_fp8 = out_dtype == PKV_DTYPE_FP8_E4M3FN;
  if (in_fp8 && cache->scale_mode != PKV_SCALE_PER_TENSOR && cache->scale_mode != PKV_SCALE_PER_TOKEN)
    return PKV_ERR_DTYPE;
  if (cache->dtype == PKV_DTYPE_BF16 && cache->scale_mode != PKV_SCALE_NONE) return PKV_ERR_DTYPE;
  if (cache->num_heads != 1) return PKV_ERR_SHAPE;
  const uint64_t in_eb = in_fp8 ? 1 : 2, out_eb = out_fp8 ? 1 : 2;
  const uint64_t row_bytes = (uint64_t)cache->head_dim * in_eb;
  if (row_bytes % 16 != 0 || ((uint64_t)cache->head_dim * out_eb) % 8 != 0) return PKV_ERR_ALIGN;
  if (cache->head_dim > 1024) return PKV_ERR_UNSUPPORTED;
  if (out_row_stride < (int64_t)cache->head_dim) return PKV_ERR_SHAPE;
  if (total_rows > 0 && batch_size == 0) return PKV_ERR_SHAPE;
  CacheView view{};
  int st = check_cache(cache, layer_idx, batch_size, &view, /*need_lengths=*/false);
  if (st != PKV_OK) return st;
  if (total_rows == 0) return PKV_OK;
  if (out == nullptr || kv_row_offsets == nullptr) return PKV_ERR_NULL;
  if (in_fp8 && cache->scales == nullptr) return PKV_ERR_NULL;
  if (in_fp8 && out_fp8 && cache->scale_mode == PKV_SCALE_PER_TOKEN && out_scales == nullptr)
    return PKV_ERR_NULL;
  if (!in_fp8 && out_fp8 && out_scale == nullptr) return PKV_ERR_NULL;
  if (!aligned16(out) || ((uint64_t)out_row_stride * out_eb) % 16 != 0) return PKV_ERR_ALIGN;

  pkv::GatherArgs a{};
  a.out = out;
  a.out_row_bytes = out_row_stride * (int64_t)out_eb;
  a.out_scales = out_scales;
  a.out_scale = out_scale;
  a.kv_row_offsets = kv_row_offsets;
  a.batch = batch_size;
  a.total_rows = total_rows;
  a.row_bytes = (uint32_t)row_bytes;
  const bool per_token = in_fp8 && cache->scale_mode == PKV_SCALE_PER_TOKEN;
  a.cache_scale = cache->scales;
  if (per_token)
    a.cache_scale = cache->scales + (int64_t)layer_idx * cache->num_pages * cache->page_size *
                                        cache->num_heads;
  a.cache = view;
  const pkv::GatherKind kind = in_fp8 ? (out_fp8 ? pkv::GatherKind::Fp8ToFp8 : pkv::GatherKind::Fp8ToBf16)
                                      : (out_fp8 ? pkv::GatherKind::Bf16ToFp8 : pkv::GatherKind::Bf16ToBf16);
  return launch_status(pkv::launch_gather(a, kind, per_token, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
