// Host-side unit test of the C ABI's argument handling (test infrastructure):
// pkv_api.cpp is linked against stand-in launchers that record the argument
// block instead of launching, and the whole binary is built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  It checks that valid calls reach a launcher
// with the right derived fields (layer base, scale blocks, chunk counts, flags),
// that refused calls reach none, and that zero-token calls launch nothing.
#include <cstdio>
#include <cstring>

#include "pkv.h"
#include "../../paged_kv_cache_wavefront_amd/csrc/pkv_internal.h"

namespace pkv {
namespace {
int g_calls = 0;
MlaArgs g_mla;
MlaOut g_mla_mode;
int g_mla_hpw;
QkArgs g_qk;
int g_qk_dim;
bool g_qk_inter;
KMode g_qk_mode;
KvNormArgs g_norm;
bool g_norm_mbc;
KMode g_norm_mode;
GatherArgs g_gather;
GatherKind g_gather_kind;
bool g_gather_per_token;
}  // namespace

uint32_t mla_heads_per_wave(uint32_t heads) { return heads > 16 ? 32 : 16; }
hipError_t launch_mla(const MlaArgs& a, MlaOut mode, int hpw, hipStream_t) {
  ++g_calls; g_mla = a; g_mla_mode = mode; g_mla_hpw = hpw;
  return hipSuccess;
}
static uint32_t lanes_per_head(uint32_t head_dim) {
  uint32_t p = 1;
  while (p < head_dim / 8) p *= 2;
  return p;
}
uint32_t qk_heads_per_wave(int head_dim) { return 4u * (64u / lanes_per_head((uint32_t)head_dim)); }
hipError_t launch_qk_rope(const QkArgs& a, int head_dim, bool inter, KMode km, hipStream_t) {
  ++g_calls; g_qk = a; g_qk_dim = head_dim; g_qk_inter = inter; g_qk_mode = km;
  return hipSuccess;
}
uint32_t kv_norm_max_heads(uint32_t head_dim) { return 4u * (64u / lanes_per_head(head_dim)); }
hipError_t launch_kv_norm(const KvNormArgs& a, bool mbc, KMode km, hipStream_t) {
  ++g_calls; g_norm = a; g_norm_mbc = mbc; g_norm_mode = km;
  return hipSuccess;
}
hipError_t launch_gather(const GatherArgs& a, GatherKind kind, bool per_token, hipStream_t) {
  ++g_calls; g_gather = a; g_gather_kind = kind; g_gather_per_token = per_token;
  return hipSuccess;
}
}  // namespace pkv

static int failures = 0, checks = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    ++checks;                                                              \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      std::fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond);     \
    }                                                                      \
  } while (0)

// 16-byte aligned stand-ins for device pointers (never dereferenced here).
alignas(16) static unsigned char arena[1 << 16];
static void* P(size_t off) { return arena + off; }

static pkv_paged_cache latent_cache(int32_t dtype, int32_t mode, uint32_t pages) {
  pkv_paged_cache c;
  std::memset(&c, 0, sizeof c);
  c.data = P(0);
  c.dtype = dtype;
  c.num_layers = 2;
  c.num_pages = pages;
  c.page_size = 16;
  c.num_heads = 1;
  c.head_dim = 576;
  c.layer_stride = (int64_t)pages * 16 * 576;
  c.page_stride = 16 * 576;
  c.slot_stride = 576;
  c.head_stride = 576;
  c.cache_lengths = static_cast<const uint32_t*>(P(4096));
  c.page_table = static_cast<const uint32_t*>(P(8192));
  c.page_table_stride = 4;
  c.scale_mode = mode;
  c.scales = static_cast<float*>(P(12288));
  return c;
}

static pkv_paged_cache k_cache(int32_t dtype, int32_t mode, uint32_t heads, uint32_t dim) {
  pkv_paged_cache c;
  std::memset(&c, 0, sizeof c);
  c.data = P(0);
  c.dtype = dtype;
  c.num_layers = 3;
  c.num_pages = 10;
  c.page_size = 8;
  c.num_heads = heads;
  c.head_dim = dim;
  c.head_stride = dim;
  c.slot_stride = (int64_t)heads * dim;
  c.page_stride = 8 * c.slot_stride;
  c.layer_stride = 10 * c.page_stride;
  c.cache_lengths = static_cast<const uint32_t*>(P(4096));
  c.page_table = static_cast<const uint32_t*>(P(8192));
  c.page_table_stride = 4;
  c.scale_mode = mode;
  c.scales = mode == PKV_SCALE_NONE ? nullptr : static_cast<float*>(P(12288));
  return c;
}

static int mla(const pkv_paged_cache* c, uint32_t T, uint32_t H, int32_t qdt, uint32_t layer = 1) {
  const int64_t qs = (int64_t)H * 64;
  return mla_rope_rmsnorm_quant(P(16384), qs, 64, P(20480), qs, 64, P(24576), 576,
                                static_cast<const uint32_t*>(P(28672)), 2, T, H, 64, 512,
                                static_cast<const float*>(P(32768)), 64, P(36864), 1e-6f, c,
                                layer, qdt, nullptr);
}

static int mla_inplace(const pkv_paged_cache* c, uint32_t T, uint32_t H, uint32_t layer = 1) {
  const int64_t qs = (int64_t)H * 64;
  return mla_rope_rmsnorm_inplace(P(16384), qs, 64, P(20480), qs, 64,
                                  static_cast<const uint32_t*>(P(28672)), 2, T, H, 64, 512,
                                  static_cast<const float*>(P(32768)), 64, P(36864), 1e-6f, c,
                                  layer, PKV_DTYPE_BF16, nullptr);
}

int main() {
  using namespace pkv;
  // --- MLA: per-token fp8, 40 heads, layer 1 of 2
  {
    pkv_paged_cache c = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TOKEN, 7);
    const int before = g_calls;
    EXPECT(mla(&c, 5, 40, PKV_DTYPE_BF16) == PKV_OK);
    EXPECT(g_calls == before + 1);
    EXPECT(g_mla_mode == MlaOut::Fp8PerToken);
    EXPECT(g_mla_hpw == 32);
    EXPECT(g_mla.chunks == 2);
    EXPECT(g_mla.cache.layer_base == static_cast<char*>(c.data) + c.layer_stride);
    EXPECT(g_mla.token_scales == c.scales + 7 * 16);
    EXPECT(!g_mla.q_out_f32);
    EXPECT(g_mla.total_tokens == 5 && g_mla.num_heads == 40 && g_mla.batch == 2);
    EXPECT(mla(&c, 5, 40, PKV_DTYPE_F32) == PKV_OK && g_mla.q_out_f32);
    EXPECT(mla(&c, 5, 16, PKV_DTYPE_BF16) == PKV_OK && g_mla.chunks == 1 && g_mla_hpw == 16);
    EXPECT(mla(&c, 5, 40, PKV_DTYPE_BF16, 0) == PKV_OK &&
           g_mla.cache.layer_base == c.data && g_mla.token_scales == c.scales);
  }
  // --- MLA: bf16 cache (2-byte elements), per-tensor fp8, refused calls, T = 0
  {
    pkv_paged_cache c = latent_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 7);
    EXPECT(mla(&c, 3, 8, PKV_DTYPE_BF16) == PKV_OK && g_mla_mode == MlaOut::Bf16);
    EXPECT(g_mla.cache.layer_base == static_cast<char*>(c.data) + 2 * c.layer_stride);
    pkv_paged_cache t = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    EXPECT(mla(&t, 3, 8, PKV_DTYPE_BF16) == PKV_OK && g_mla.tensor_scale == t.scales);
    const int before = g_calls;
    EXPECT(mla(&t, 0, 8, PKV_DTYPE_BF16) == PKV_OK);            // nothing to do
    EXPECT(mla(&t, 3, 8, PKV_DTYPE_FP8_E4M3FN) == PKV_ERR_DTYPE);
    EXPECT(mla(&t, 3, 8, PKV_DTYPE_BF16, 2) == PKV_ERR_RANGE);
    t.scales = nullptr;
    EXPECT(mla(&t, 3, 8, PKV_DTYPE_BF16) == PKV_ERR_NULL);
    t = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    t.slot_stride = 580;
    EXPECT(mla(&t, 3, 8, PKV_DTYPE_BF16) == PKV_ERR_ALIGN);
    EXPECT(g_calls == before);
  }
  // --- MLA in place: bf16 cache only, no latent buffer
  {
    pkv_paged_cache c = latent_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 7);
    EXPECT(mla_inplace(&c, 3, 40) == PKV_OK && g_mla_mode == MlaOut::Bf16InPlace);
    EXPECT(g_mla.latent == nullptr && g_mla.kv_row == 0 && g_mla.chunks == 2);
    EXPECT(g_mla.cache.layer_base == static_cast<char*>(c.data) + 2 * c.layer_stride);
    const int before = g_calls;
    pkv_paged_cache t = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    EXPECT(mla_inplace(&t, 3, 40) == PKV_ERR_DTYPE);
    EXPECT(mla_inplace(&c, 0, 40) == PKV_OK);
    EXPECT(mla_inplace(&c, 3, 40, 2) == PKV_ERR_RANGE);
    EXPECT(g_calls == before);
  }
  // --- Q/K RoPE: fp8 per-token K, mRoPE, K norm
  {
    pkv_paged_cache c = k_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TOKEN, 4, 128);
    const uint32_t sec[3] = {16, 24, 24};
    const int st = qk_rope_paged_ragged(P(16384), 40 * 128, 128, P(20480), 40 * 128, 128, 9, 40, 128,
                                        static_cast<const uint32_t*>(P(28672)), 2, &c, 2,
                                        static_cast<const float*>(P(32768)), 512,
                                        static_cast<const uint32_t*>(P(36864)), sec, 0, P(40960), 96,
                                        1e-6f, nullptr);
    EXPECT(st == PKV_OK);
    EXPECT(g_qk_mode == KMode::Fp8PerToken && g_qk_dim == 128 && !g_qk_inter);
    EXPECT(g_qk.chunks == 3);                                      // 40 heads, 16 per wave
    EXPECT(g_qk.mrope && g_qk.mrope_end0 == 16 && g_qk.mrope_end1 == 40);
    EXPECT(g_qk.k_norm_cols == 96);
    EXPECT(g_qk.k_scales == c.scales + 2 * 10 * 8 * 4);
    EXPECT(g_qk.cache.layer_base == static_cast<char*>(c.data) + 2 * c.layer_stride);
    const uint32_t bad[3] = {16, 24, 23};
    const int before = g_calls;
    EXPECT(qk_rope_paged_ragged(P(16384), 40 * 128, 128, P(20480), 40 * 128, 128, 9, 40, 128,
                                static_cast<const uint32_t*>(P(28672)), 2, &c, 2,
                                static_cast<const float*>(P(32768)), 512,
                                static_cast<const uint32_t*>(P(36864)), bad, 0, nullptr, 0, 1e-6f,
                                nullptr) == PKV_ERR_SHAPE);
    EXPECT(g_calls == before);
  }
  // --- Q/K RoPE with 96-wide heads: 16-lane groups, 16 heads per wave
  {
    pkv_paged_cache c = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 2, 96);
    EXPECT(qk_rope_paged_ragged(P(16384), 40 * 96, 96, P(20480), 40 * 96, 96, 9, 40, 96,
                                static_cast<const uint32_t*>(P(28672)), 2, &c, 1,
                                static_cast<const float*>(P(32768)), 512, nullptr, nullptr, 1,
                                nullptr, 0, 1e-6f, nullptr) == PKV_OK);
    EXPECT(g_qk_dim == 96 && g_qk_inter && g_qk.chunks == 3);
  }
  // --- K-cache norm: per-token statistic, bf16 two roundings
  {
    pkv_paged_cache c = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 8, 128);
    EXPECT(rms_norm_kv_cache_paged(&c, 1, P(40960), 100, 1e-6f, 0.5f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 0, 0, nullptr) ==
           PKV_OK);
    EXPECT(!g_norm.per_head && !g_norm_mbc && g_norm_mode == KMode::Bf16);
    EXPECT(g_norm.total_tokens == 7 && g_norm.gamma_len == 100 && g_norm.weight_offset == 0.5f);
    EXPECT(g_norm.head_dim == 128);
    pkv_paged_cache big = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 17, 128);
    EXPECT(rms_norm_kv_cache_paged(&big, 1, P(40960), 128, 1e-6f, 0.f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 0, 1, nullptr) ==
           PKV_ERR_UNSUPPORTED);
    EXPECT(rms_norm_kv_cache_paged(&big, 1, P(40960), 128, 1e-6f, 0.f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 1, 1, nullptr) ==
           PKV_OK && g_norm.per_head);
  }
  // --- gather: fp8 per-token cache -> bf16 rows with a padded stride
  {
    pkv_paged_cache c = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TOKEN, 7);
    EXPECT(mla_gather_latent_paged(P(16384), PKV_DTYPE_BF16, 584, nullptr, nullptr,
                                   static_cast<const uint32_t*>(P(28672)), 2, 33, &c, 1,
                                   nullptr) == PKV_OK);
    EXPECT(g_gather_kind == GatherKind::Fp8ToBf16 && g_gather_per_token);
    EXPECT(g_gather.out_row_bytes == 584 * 2 && g_gather.row_bytes == 576);
    EXPECT(g_gather.cache_scale == c.scales + 7 * 16);
    EXPECT(g_gather.total_rows == 33 && g_gather.batch == 2);
  }
  std::printf("host api: %d of %d checks passed\n", checks - failures, checks);
  return failures == 0 ? 0 : 1;
}
