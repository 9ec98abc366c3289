// Host-side unit test of the C ABI's argument handling (test infrastructure):
// pkv_api.cpp is linked against stand-in launchers that record the argument
// block instead of launching, and the whole binary is built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  It checks that valid calls reach a launcher
// with the right derived fields (layer base, scale blocks, chunk counts, flags),
// that refused calls reach none, and that zero-token calls launch nothing; then
// a seeded randomised sweep of 20 000 calls over all entry points.
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
bool g_qk_f16;
KMode g_qk_mode;
KvNormArgs g_norm;
bool g_norm_mbc;
KMode g_norm_mode;
GatherArgs g_gather;
GatherKind g_gather_kind;
bool g_gather_per_token;
PlanArgs g_plan;
}  // namespace

uint32_t mla_heads_per_wave(uint32_t heads, uint32_t rope_dim) {
  const uint32_t per_instr = 64 / (rope_dim / 8);
  return heads > 2 * per_instr ? 4 * per_instr : 2 * per_instr;
}
bool mla_rope_dim_supported(uint32_t r) { return r == 32 || r == 64 || r == 128; }
bool mla_nope_dim_supported(uint32_t d) { return d > 0 && d % 8 == 0 && d <= 512; }
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
hipError_t launch_qk_rope(const QkArgs& a, int head_dim, bool inter, bool f16, KMode km,
                          hipStream_t) {
  ++g_calls; g_qk = a; g_qk_dim = head_dim; g_qk_inter = inter; g_qk_f16 = f16; g_qk_mode = km;
  return hipSuccess;
}
hipError_t launch_kv_norm(const KvNormArgs& a, bool mbc, KMode km, hipStream_t) {
  ++g_calls; g_norm = a; g_norm_mbc = mbc; g_norm_mode = km;
  return hipSuccess;
}
hipError_t launch_gather(const GatherArgs& a, GatherKind kind, bool per_token, hipStream_t) {
  ++g_calls; g_gather = a; g_gather_kind = kind; g_gather_per_token = per_token;
  return hipSuccess;
}
hipError_t launch_plan(const PlanArgs& a, hipStream_t) {
  ++g_calls; g_plan = a;
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

// An MLA call whose q output has element type qdt (bf16 q, fp32 freqs, bf16 gamma).
static int mla(const pkv_paged_cache* c, uint32_t T, uint32_t H, int32_t qdt, uint32_t layer = 1) {
  const int64_t qs = (int64_t)H * 64;
  const pkv_elem_types types = {PKV_DTYPE_BF16, qdt, PKV_DTYPE_F32, PKV_DTYPE_BF16};
  return mla_rope_rmsnorm_quant(P(16384), qs, 64, P(20480), qs, 64, P(24576), 576,
                                static_cast<const uint32_t*>(P(28672)), 2, T, H, 64, 512,
                                P(32768), 64, P(36864), 1e-6f, c, layer, &types, nullptr);
}

// An MLA call of 5 tokens of 40 heads with the given element types and q
// output token stride (elements).
static int mla_types(const pkv_paged_cache* c, const pkv_elem_types* t,
                     int64_t qo_stride = 40 * 64) {
  return mla_rope_rmsnorm_quant(P(16384), qo_stride, 64, P(20480), 40 * 64, 64, P(24576), 576,
                                static_cast<const uint32_t*>(P(28672)), 2, 5, 40, 64, 512,
                                P(32768), 64, P(36864), 1e-6f, c, 1, t, nullptr);
}

// An MLA call with rope_dim R and kv_norm_dim Dn (q rows of H * R values).
static int mla_dims(const pkv_paged_cache* c, uint32_t T, uint32_t H, uint32_t R, uint32_t Dn) {
  const int64_t qs = (int64_t)H * R;
  return mla_rope_rmsnorm_quant(P(16384), qs, R, P(20480), qs, R, P(24576), Dn + R,
                                static_cast<const uint32_t*>(P(28672)), 2, T, H, R, Dn,
                                P(32768), 64, P(36864), 1e-6f, c, 1, nullptr, nullptr);
}

static int mla_inplace(const pkv_paged_cache* c, uint32_t T, uint32_t H, uint32_t layer = 1) {
  const int64_t qs = (int64_t)H * 64;
  return mla_rope_rmsnorm_inplace(P(16384), qs, 64, P(20480), qs, 64,
                                  static_cast<const uint32_t*>(P(28672)), 2, T, H, 64, 512,
                                  P(32768), 64, P(36864), 1e-6f, c, layer, nullptr, nullptr);
}

// Randomised sweep of the validation: descriptors and arguments drawn from
// mostly-valid values with one or more fields perturbed (zero, odd, huge,
// misaligned, NULL, out of range).  Every call must return a status code of
// the enum; a stand-in launcher may be reached only with PKV_OK and tokens
// (or rows) to process, and every reached launch must see a layer base inside
// the pool it was given.  AddressSanitizer / UBSan watch the whole sweep.
static uint64_t fz = 0x2545F4914F6CDD1Dull;
static uint32_t frand() {
  fz ^= fz << 13; fz ^= fz >> 7; fz ^= fz << 17;
  return (uint32_t)(fz >> 16);
}
static bool coin(uint32_t one_in) { return frand() % one_in == 0; }
static uint32_t pick_u32(const uint32_t* v, int n) { return v[frand() % (uint32_t)n]; }

static void perturb(pkv_paged_cache* c) {
  switch (frand() % 12) {
    case 0: c->data = coin(2) ? nullptr : static_cast<char*>(c->data) + 8; break;
    case 1: c->dtype = (int32_t)(frand() % 4); break;
    case 2: c->num_layers = frand() % 3; break;
    case 3: c->num_pages = coin(2) ? 0u : frand(); break;
    case 4: c->page_size = frand() % 3; break;
    case 5: c->num_heads = frand() % 40; break;
    case 6: c->head_dim = frand() % 1200; break;
    case 7: c->slot_stride += (int64_t)(frand() % 16) - 8; break;
    case 8: c->head_stride = coin(2) ? -16 : (int64_t)frand(); break;
    case 9: c->page_table = nullptr; break;
    case 10: c->scale_mode = (int32_t)(frand() % 4); break;
    case 11: c->scales = nullptr; break;
  }
}

static void fuzz(int iters) {
  using namespace pkv;
  const uint32_t dims[] = {64, 80, 96, 128, 256, 72, 512};
  int launched = 0, refused = 0;
  for (int it = 0; it < iters; ++it) {
    const int entry = (int)(frand() % 7);
    pkv_paged_cache c;
    if (entry <= 1 || entry >= 4) {
      c = latent_cache(coin(2) ? PKV_DTYPE_BF16 : PKV_DTYPE_FP8_E4M3FN,
                       (int32_t)(frand() % 3), 1 + frand() % 16);
      if (entry == 1 || c.dtype == PKV_DTYPE_BF16) c.scale_mode = PKV_SCALE_NONE;
    } else {
      const uint32_t d = pick_u32(dims, 7);
      c = k_cache(coin(3) ? PKV_DTYPE_FP8_E4M3FN : PKV_DTYPE_BF16, PKV_SCALE_NONE,
                  1 + frand() % 20, d);
      if (c.dtype == PKV_DTYPE_FP8_E4M3FN) c.scale_mode = coin(2) ? PKV_SCALE_PER_TENSOR
                                                                  : PKV_SCALE_PER_TOKEN;
      c.scales = static_cast<float*>(P(12288));
    }
    const int nbad = coin(3) ? 0 : 1 + (int)(frand() % 3);
    for (int k = 0; k < nbad; ++k) perturb(&c);
    const pkv_paged_cache* cp = coin(50) ? nullptr : &c;
    const uint32_t T = coin(4) ? 0u : 1 + frand() % 5000;
    const uint32_t B = coin(20) ? 0u : 1 + frand() % 600;
    const uint32_t layer = frand() % 4;
    void* q = coin(30) ? nullptr : (coin(20) ? P(16384 + 4) : P(16384));
    const uint32_t H = frand() % 200;
    // element types: mostly the defaults, sometimes any code in -1..4
    pkv_elem_types ty = {PKV_DTYPE_BF16, PKV_DTYPE_BF16, PKV_DTYPE_F32, PKV_DTYPE_BF16};
    int32_t* fields[4] = {&ty.q, &ty.q_out, &ty.freqs, &ty.gamma};
    for (int32_t* f : fields)
      if (coin(8)) *f = (int32_t)(frand() % 6) - 1;
    const pkv_elem_types* tp = coin(3) ? nullptr : &ty;
    const int before = g_calls;
    int st = -1;
    switch (entry) {
      case 0:
      case 1: {
        const int64_t ts = (int64_t)H * 64 + (coin(10) ? 4 : 0);
        if (entry == 0)
          st = mla_rope_rmsnorm_quant(P(20480), ts, 64, q, ts, 64, coin(20) ? nullptr : P(24576),
                                      coin(10) ? 580 : 576, static_cast<const uint32_t*>(P(28672)),
                                      B, T, H, coin(10) ? 32 : 64, coin(10) ? 256 : 512,
                                      P(32768), 1 + frand() % 9000,
                                      coin(30) ? nullptr : P(36864), 1e-6f, cp, layer, tp,
                                      nullptr);
        else
          st = mla_rope_rmsnorm_inplace(P(20480), ts, 64, q, ts, 64,
                                        static_cast<const uint32_t*>(P(28672)), B, T, H,
                                        coin(10) ? 32 : 64, 512,
                                        P(32768), 1 + frand() % 9000,
                                        coin(30) ? nullptr : P(36864), 1e-6f, cp, layer, tp,
                                        nullptr);
        break;
      }
      case 2: {
        const uint32_t D = cp ? cp->head_dim : 128;
        const uint32_t sec_ok[3] = {D / 4, D / 8, D / 2 - D / 4 - D / 8};
        const uint32_t sec_bad[3] = {1, 2, 3};
        const uint32_t* sec = coin(4) ? (coin(2) ? sec_ok : sec_bad) : nullptr;
        const uint32_t cols = coin(3) ? 0u : frand() % (D + 2);
        st = qk_rope_paged_ragged(P(20480), (int64_t)H * D, D, q, (int64_t)H * D, D, T, H, D,
                                  static_cast<const uint32_t*>(P(28672)), B, cp, layer,
                                  P(32768), 4096,
                                  coin(2) ? static_cast<const uint32_t*>(P(40960)) : nullptr, sec,
                                  (int)(frand() % 2), cols ? P(45056) : nullptr, cols, 1e-6f,
                                  tp, nullptr);
        break;
      }
      case 3: {
        const uint32_t D = cp ? cp->head_dim : 128;
        st = rms_norm_kv_cache_paged(cp, layer, coin(20) ? nullptr : P(45056),
                                     coin(10) ? 0u : 1 + frand() % (D + 1), 1e-6f, 0.25f, T,
                                     static_cast<const uint32_t*>(P(28672)), B,
                                     (int)(frand() % 2), (int)(frand() % 2), tp, nullptr);
        break;
      }
      case 5: {
        const int64_t ts = (int64_t)H * 64 + (coin(10) ? 4 : 0);
        const uint32_t* plan = coin(20) ? nullptr
                                        : static_cast<const uint32_t*>(P(coin(20) ? 40964 : 40960));
        st = mla_rope_rmsnorm_quant_planned(P(20480), ts, 64, q, ts, 64,
                                            coin(20) ? nullptr : P(24576), coin(10) ? 580 : 576,
                                            plan, T, H, coin(10) ? 32 : 64, coin(10) ? 256 : 512,
                                            P(32768), 1 + frand() % 9000,
                                            coin(30) ? nullptr : P(36864), 1e-6f, cp, layer, tp,
                                            nullptr);
        break;
      }
      case 6: {
        uint32_t* plan = coin(20) ? nullptr : static_cast<uint32_t*>(P(coin(20) ? 40964 : 40960));
        st = pkv_token_plan(plan, coin(20) ? nullptr : static_cast<const uint32_t*>(P(28672)), B,
                            T, cp, nullptr);
        break;
      }
      case 4: {
        const int32_t odt = coin(2) ? PKV_DTYPE_BF16 : PKV_DTYPE_FP8_E4M3FN;
        const uint32_t W = cp ? cp->head_dim : 576;
        st = mla_gather_latent_paged(P(49152), odt, (int64_t)W + (coin(10) ? 8 : 0),
                                     coin(5) ? nullptr : static_cast<float*>(P(53248)),
                                     coin(5) ? nullptr : static_cast<const float*>(P(57344)),
                                     static_cast<const uint32_t*>(P(28672)), B, T, cp, layer,
                                     nullptr);
        break;
      }
    }
    EXPECT(st >= PKV_OK && st <= PKV_ERR_LAUNCH);
    const bool reached = g_calls != before;
    if (reached) {
      ++launched;
      EXPECT(st == PKV_OK && T > 0 && cp != nullptr);
      const char* base = nullptr;
      switch (entry) {
        case 0: case 1: case 5: base = static_cast<const char*>(g_mla.cache.layer_base); break;
        case 2: base = static_cast<const char*>(g_qk.cache.layer_base); break;
        case 3: base = static_cast<const char*>(g_norm.cache.layer_base); break;
        case 4: base = static_cast<const char*>(g_gather.cache.layer_base); break;
      }
      if (entry == 6) {
        // the plan builder reads the lengths and page table, never the pool
        EXPECT(g_plan.total_tokens == T && g_plan.batch == B && B > 0);
        EXPECT(g_plan.page_table == cp->page_table && g_plan.page_size > 0);
        EXPECT(((uintptr_t)g_plan.plan & 15u) == 0);
        continue;
      }
      const int64_t eb = cp->dtype == PKV_DTYPE_BF16 ? 2 : 1;
      EXPECT(base == static_cast<const char*>(cp->data) + (int64_t)layer * cp->layer_stride * eb);
      EXPECT(layer < cp->num_layers);
      if (entry == 5) EXPECT(g_mla.plan != nullptr && g_mla.offsets == nullptr);
    } else {
      refused += st != PKV_OK;
    }
  }
  std::printf("host api sweep: %d calls, %d reached a launcher, %d refused\n", iters, launched,
              refused);
}

int main() {
  using namespace pkv;
  // --- token plan and the planned MLA step
  {
    pkv_paged_cache c = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    uint32_t* plan = static_cast<uint32_t*>(P(40960));
    const uint32_t* offs = static_cast<const uint32_t*>(P(28672));
    int before = g_calls;
    EXPECT(pkv_token_plan(plan, offs, 2, 9, &c, nullptr) == PKV_OK && g_calls == before + 1);
    EXPECT(g_plan.plan == plan && g_plan.offsets == offs && g_plan.batch == 2);
    EXPECT(g_plan.total_tokens == 9 && g_plan.cache_lengths == c.cache_lengths);
    EXPECT(g_plan.page_table == c.page_table && g_plan.pt_stride == 4);
    EXPECT(g_plan.num_pages == 7 && g_plan.page_size == 16);
    before = g_calls;
    EXPECT(pkv_token_plan(plan, offs, 2, 0, &c, nullptr) == PKV_OK);
    EXPECT(pkv_token_plan(plan + 1, offs, 2, 9, &c, nullptr) == PKV_ERR_ALIGN);
    EXPECT(pkv_token_plan(plan, offs, 0, 9, &c, nullptr) == PKV_ERR_SHAPE);
    EXPECT(g_calls == before);
    // the planned step: no lengths or page table needed, plan passed through
    c.cache_lengths = nullptr;
    c.page_table = nullptr;
    EXPECT(mla_rope_rmsnorm_quant_planned(P(16384), 40 * 64, 64, P(20480), 40 * 64, 64,
                                          P(24576), 576, plan, 5, 40, 64, 512,
                                          P(32768), 64, P(36864), 1e-6f, &c, 1, nullptr,
                                          nullptr) == PKV_OK);
    EXPECT(g_calls == before + 1 && g_mla.plan == plan && g_mla.offsets == nullptr);
    EXPECT(g_mla.batch == 0 && g_mla.total_tokens == 5 && g_mla.chunks == 2);
    EXPECT(g_mla_mode == MlaOut::Fp8PerTensor);
    EXPECT(g_mla.cache.layer_base == static_cast<char*>(c.data) + c.layer_stride);
    EXPECT(mla_rope_rmsnorm_quant_planned(P(16384), 40 * 64, 64, P(20480), 40 * 64, 64,
                                          P(24576), 576, plan + 2, 5, 40, 64, 512,
                                          P(32768), 64, P(36864), 1e-6f, &c, 1, nullptr,
                                          nullptr) == PKV_ERR_ALIGN);
    // the batch form never carries a plan
    pkv_paged_cache b = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    EXPECT(mla(&b, 5, 40, PKV_DTYPE_BF16) == PKV_OK && g_mla.plan == nullptr);
    // the planned K norm
    pkv_paged_cache k = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 8, 128);
    k.cache_lengths = nullptr;
    k.page_table = nullptr;
    before = g_calls;
    EXPECT(rms_norm_kv_cache_paged_planned(&k, 2, P(45056), 128, 1e-6f, 0.0f, 7, plan, 1, 1,
                                           nullptr, nullptr) == PKV_OK);
    EXPECT(g_calls == before + 1 && g_norm.plan == plan && g_norm.offsets == nullptr);
    EXPECT(g_norm.total_tokens == 7 && g_norm.batch == 0);
    EXPECT(g_norm.cache.layer_base == static_cast<char*>(k.data) + 2 * 2 * k.layer_stride);
    EXPECT(rms_norm_kv_cache_paged_planned(&k, 2, P(45056), 128, 1e-6f, 0.0f, 7, plan + 1, 1, 1,
                                           nullptr, nullptr) == PKV_ERR_ALIGN);
  }
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
    EXPECT(g_mla.qio == QIO::B_B && g_mla.freq_type == PKV_DTYPE_F32);
    EXPECT(g_mla.gamma_type == PKV_DTYPE_BF16);
    EXPECT(g_mla.total_tokens == 5 && g_mla.num_heads == 40 && g_mla.batch == 2);
    EXPECT(g_mla.rope_dim == 64 && g_mla.nope_chunks == 64 && g_mla.inv_dn == 1.0f / 512);
    EXPECT(mla(&c, 5, 40, PKV_DTYPE_F32) == PKV_OK && g_mla.qio == QIO::B_F);
    EXPECT(mla(&c, 5, 16, PKV_DTYPE_BF16) == PKV_OK && g_mla.chunks == 1 && g_mla_hpw == 16);
    EXPECT(mla(&c, 5, 40, PKV_DTYPE_BF16, 0) == PKV_OK &&
           g_mla.cache.layer_base == c.data && g_mla.token_scales == c.scales);
  }
  // --- MLA: other rope and non-rope widths (rows of Dn + R values)
  {
    struct { uint32_t R, Dn; int st; uint32_t hpw; } cases[] = {
        {32, 256, PKV_OK, 64}, {128, 512, PKV_OK, 16}, {64, 256, PKV_OK, 32},
        {32, 512, PKV_OK, 64}, {64, 16, PKV_OK, 32}, {128, 128, PKV_OK, 16},
        {48, 512, PKV_ERR_UNSUPPORTED, 0}, {16, 512, PKV_ERR_UNSUPPORTED, 0},
        {64, 520, PKV_ERR_UNSUPPORTED, 0}, {64, 100, PKV_ERR_UNSUPPORTED, 0},
        {256, 256, PKV_ERR_UNSUPPORTED, 0}};
    for (const auto& k : cases) {
      pkv_paged_cache c = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 3);
      const uint32_t W = k.Dn + k.R;
      c.head_dim = W;
      c.head_stride = c.slot_stride = W;
      c.page_stride = 16 * (int64_t)W;
      c.layer_stride = 3 * c.page_stride;
      const int before = g_calls;
      EXPECT(mla_dims(&c, 4, 40, k.R, k.Dn) == k.st);
      if (k.st != PKV_OK) {
        EXPECT(g_calls == before);
        continue;
      }
      EXPECT(g_calls == before + 1 && g_mla.rope_dim == k.R && g_mla.nope_chunks == k.Dn / 8);
      EXPECT(g_mla.inv_dn == (float)(1.0 / k.Dn) && (uint32_t)g_mla_hpw == k.hpw);
      EXPECT(g_mla.chunks == (40 + k.hpw - 1) / k.hpw);
    }
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
                                        P(32768), 512,
                                        static_cast<const uint32_t*>(P(36864)), sec, 0, P(40960), 96,
                                        1e-6f, nullptr, nullptr);
    EXPECT(st == PKV_OK);
    EXPECT(g_qk_mode == KMode::Fp8PerToken && g_qk_dim == 128 && !g_qk_inter && !g_qk_f16);
    EXPECT(g_qk.freq_type == PKV_DTYPE_F32);
    EXPECT(g_qk.chunks == 3);                                      // 40 heads, 16 per wave
    EXPECT(g_qk.mrope && g_qk.mrope_end0 == 16 && g_qk.mrope_end1 == 40);
    EXPECT(g_qk.k_norm_cols == 96 && g_qk.inv_norm_cols == (float)(1.0 / 96));
    EXPECT(g_qk.k_scales == c.scales + 2 * 10 * 8 * 4);
    EXPECT(g_qk.cache.layer_base == static_cast<char*>(c.data) + 2 * c.layer_stride);
    const uint32_t bad[3] = {16, 24, 23};
    const int before = g_calls;
    EXPECT(qk_rope_paged_ragged(P(16384), 40 * 128, 128, P(20480), 40 * 128, 128, 9, 40, 128,
                                static_cast<const uint32_t*>(P(28672)), 2, &c, 2,
                                P(32768), 512,
                                static_cast<const uint32_t*>(P(36864)), bad, 0, nullptr, 0, 1e-6f,
                                nullptr, nullptr) == PKV_ERR_SHAPE);
    EXPECT(g_calls == before);
  }
  // --- Q/K RoPE with 96-wide heads: 16-lane groups, 16 heads per wave
  {
    pkv_paged_cache c = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 2, 96);
    EXPECT(qk_rope_paged_ragged(P(16384), 40 * 96, 96, P(20480), 40 * 96, 96, 9, 40, 96,
                                static_cast<const uint32_t*>(P(28672)), 2, &c, 1,
                                P(32768), 512, nullptr, nullptr, 1,
                                nullptr, 0, 1e-6f, nullptr, nullptr) == PKV_OK);
    EXPECT(g_qk_dim == 96 && g_qk_inter && g_qk.chunks == 3);
  }
  // --- K-cache norm: per-token statistic, bf16 two roundings
  {
    pkv_paged_cache c = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 8, 128);
    EXPECT(rms_norm_kv_cache_paged(&c, 1, P(40960), 100, 1e-6f, 0.5f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 0, 0, nullptr,
                                   nullptr) == PKV_OK);
    EXPECT(!g_norm.per_head && !g_norm_mbc && g_norm_mode == KMode::Bf16);
    EXPECT(g_norm.total_tokens == 7 && g_norm.gamma_len == 100 && g_norm.weight_offset == 0.5f);
    EXPECT(g_norm.inv_cols == (float)(1.0 / 100) && g_norm.inv_token_cols == (float)(1.0 / 800));
    EXPECT(g_norm.head_dim == 128);
    // the per-token statistic over more heads than one register chunk holds
    pkv_paged_cache big = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 17, 128);
    EXPECT(rms_norm_kv_cache_paged(&big, 1, P(40960), 128, 1e-6f, 0.f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 0, 1, nullptr,
                                   nullptr) == PKV_OK && !g_norm.per_head &&
           g_norm.cache.num_heads == 17);
    EXPECT(rms_norm_kv_cache_paged(&big, 1, P(40960), 128, 1e-6f, 0.f, 7,
                                   static_cast<const uint32_t*>(P(28672)), 2, 1, 1, nullptr,
                                   nullptr) == PKV_OK && g_norm.per_head);
  }
  // --- element types: the six q / q-output pairs, freqs and gamma types, refusals
  {
    const int32_t BF = PKV_DTYPE_BF16, H = PKV_DTYPE_F16, F = PKV_DTYPE_F32;
    const int32_t E8 = PKV_DTYPE_FP8_E4M3FN;
    pkv_paged_cache c = latent_cache(PKV_DTYPE_FP8_E4M3FN, PKV_SCALE_PER_TENSOR, 7);
    struct { int32_t q, qo; QIO qio; } pairs[] = {{BF, BF, QIO::B_B}, {BF, H, QIO::B_H},
                                                  {BF, F, QIO::B_F},  {H, H, QIO::H_H},
                                                  {H, BF, QIO::H_B},  {H, F, QIO::H_F}};
    for (const auto& p : pairs) {
      const pkv_elem_types t = {p.q, p.qo, H, F};
      EXPECT(mla_types(&c, &t) == PKV_OK && g_mla.qio == p.qio);
      EXPECT(g_mla.freq_type == PKV_DTYPE_F16 && g_mla.gamma_type == PKV_DTYPE_F32);
    }
    const int before = g_calls;
    const pkv_elem_types refused[] = {{F, BF, F, BF}, {E8, BF, F, BF}, {BF, E8, F, BF},
                                      {BF, BF, E8, BF}, {BF, BF, F, E8}, {BF, BF, F, 7},
                                      {-1, BF, F, BF}};
    for (const auto& t : refused) EXPECT(mla_types(&c, &t) == PKV_ERR_DTYPE);
    // the q output's strides are 16-byte multiples of its own element size
    const pkv_elem_types f32_out = {BF, F, F, BF}, f16_out = {BF, H, F, BF};
    EXPECT(mla_types(&c, &f16_out, 40 * 64 + 4) == PKV_ERR_ALIGN);
    EXPECT(g_calls == before);
    EXPECT(mla_types(&c, &f32_out, 40 * 64 + 4) == PKV_OK);
    // Q/K RoPE: q and its output share a 16-bit type; the K-norm gamma is bf16
    pkv_paged_cache k = k_cache(PKV_DTYPE_BF16, PKV_SCALE_NONE, 2, 128);
    auto qk = [&](const pkv_elem_types* t, const void* gamma) {
      return qk_rope_paged_ragged(P(16384), 40 * 128, 128, P(20480), 40 * 128, 128, 9, 40, 128,
                                  static_cast<const uint32_t*>(P(28672)), 2, &k, 1, P(32768), 512,
                                  nullptr, nullptr, 0, gamma, gamma ? 128 : 0, 1e-6f, t, nullptr);
    };
    const pkv_elem_types hh = {H, H, BF, BF};
    EXPECT(qk(&hh, P(40960)) == PKV_OK && g_qk_f16 && g_qk.freq_type == PKV_DTYPE_BF16);
    EXPECT(qk(nullptr, nullptr) == PKV_OK && !g_qk_f16 && g_qk.freq_type == PKV_DTYPE_F32);
    const pkv_elem_types f32_gamma = {BF, BF, F, F};
    EXPECT(qk(&f32_gamma, nullptr) == PKV_OK);  // gamma type unused without a K norm
    const int before_qk = g_calls;
    EXPECT(qk(&f32_gamma, P(40960)) == PKV_ERR_DTYPE);
    const pkv_elem_types mixed = {H, BF, F, BF}, f32_q = {F, F, F, BF}, fp8_freqs = {BF, BF, E8, BF};
    EXPECT(qk(&mixed, nullptr) == PKV_ERR_DTYPE && qk(&f32_q, nullptr) == PKV_ERR_DTYPE);
    EXPECT(qk(&fp8_freqs, nullptr) == PKV_ERR_DTYPE && g_calls == before_qk);
    // K-cache norm: bf16, fp16 or fp32 gamma
    auto norm = [&](const pkv_elem_types* t) {
      return rms_norm_kv_cache_paged(&k, 1, P(40960), 100, 1e-6f, 0.f, 7,
                                     static_cast<const uint32_t*>(P(28672)), 2, 1, 1, t, nullptr);
    };
    const pkv_elem_types g16 = {BF, BF, F, H}, g32 = {BF, BF, F, F}, g8 = {BF, BF, F, E8};
    EXPECT(norm(&g16) == PKV_OK && g_norm.gamma_type == PKV_DTYPE_F16);
    EXPECT(norm(&g32) == PKV_OK && g_norm.gamma_type == PKV_DTYPE_F32);
    EXPECT(norm(nullptr) == PKV_OK && g_norm.gamma_type == PKV_DTYPE_BF16);
    const int before_norm = g_calls;
    EXPECT(norm(&g8) == PKV_ERR_DTYPE && g_calls == before_norm);
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
  fuzz(20000);
  std::printf("host api: %d of %d checks passed\n", checks - failures, checks);
  return failures == 0 ? 0 : 1;
}
