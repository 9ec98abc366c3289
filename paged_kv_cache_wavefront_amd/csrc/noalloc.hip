// noalloc.hip -- mla_rope_rmsnorm_quant_noalloc: the planned MLA step
// (token plan + fused RoPE / RMSNorm / quantised paged store) for callers that
// cannot allocate device memory -- code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc.  The token plan, which the planned
// entry points take as a caller-allocated workspace, lives here in a
// file-scope device array instead; the kernels are the ones the planned entry
// points use (token_plan.hip, mla_rope_rmsnorm_quant.hip), handed that
// array's device address like any workspace.
//
// The array: kScratchTokens plan entries of 16 bytes (4 MiB) on every device
// the library runs on, held until the process ends.  Its device address is
// resolved once per device, with that device current, by
// hipGetSymbolAddress, and only that address is used from host code (the
// array's name in host code is a host-side stand-in, not a device address).
// Every call on a device shares that device's array: calls that overlap on
// one device race (one call's plan build can overwrite the plan another call
// is reading).  Every entry a build writes is written (placed or zero), so
// nothing needs clearing between calls.
#include <mutex>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

constexpr uint32_t kScratchTokens = 1u << 18;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint32_t scratch[4 * kScratchTokens];

namespace {

std::mutex g_mutex;
uint32_t* g_scratch[kMaxDevices];   // the array's device address, per device
uint32_t g_built[kMaxDevices];      // tokens of the last plan built there

// The device a stream's work runs on (the current device for the null stream).
int stream_device(hipStream_t stream, int* device) {
  if (stream == nullptr) return hipGetDevice(device) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  hipDevice_t d;
  if (hipStreamGetDevice(stream, &d) != hipSuccess) return PKV_ERR_LAUNCH;
  *device = static_cast<int>(d);
  return PKV_OK;
}

// The scratch array's device address on `device`, resolved on first use with
// that device current (and the caller's current device restored).
int scratch_on(int device, uint32_t** out) {
  if (device < 0 || device >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[device] == nullptr) {
    int current = 0;
    if (hipGetDevice(&current) != hipSuccess) return PKV_ERR_LAUNCH;
    if (current != device && hipSetDevice(device) != hipSuccess) return PKV_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device && hipSetDevice(current) != hipSuccess) return PKV_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return PKV_ERR_LAUNCH;
    g_scratch[device] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch[device];
  return PKV_OK;
}

}  // namespace

extern "C" int mla_rope_rmsnorm_quant_noalloc(
    void* q_rope_out, int64_t qo_tok_stride, int64_t qo_head_stride, const void* q_rope,
    int64_t qi_tok_stride, int64_t qi_head_stride, const void* kv_latent, int64_t kv_row_stride,
    const uint32_t* input_row_offsets, uint32_t batch_size, uint32_t total_tokens,
    uint32_t num_heads, uint32_t rope_dim, uint32_t kv_norm_dim, const void* freqs_cis,
    uint32_t max_seq_len, const void* gamma, float epsilon, const pkv_paged_cache* kv_cache,
    uint32_t layer_idx, const pkv_elem_types* types, int build_plan, void* stream) {
  if (total_tokens > kScratchTokens) return PKV_ERR_UNSUPPORTED;
  // Host checks first, against a stand-in plan address (16-byte aligned,
  // never dereferenced): a refused call touches no device.
  uint32_t* const stand_in = reinterpret_cast<uint32_t*>(uintptr_t(256));
  pkv::MlaLaunch m;
  int st = pkv::mla_prepare_planned(q_rope_out, qo_tok_stride, qo_head_stride, q_rope,
                                    qi_tok_stride, qi_head_stride, kv_latent, kv_row_stride,
                                    stand_in, total_tokens, num_heads, rope_dim, kv_norm_dim,
                                    freqs_cis, max_seq_len, gamma, epsilon, kv_cache, layer_idx,
                                    types, &m);
  if (st != PKV_OK) return st;
  pkv::PlanArgs pa{};
  if (build_plan) {
    st = pkv::plan_prepare(stand_in, input_row_offsets, batch_size, total_tokens, kv_cache, &pa);
    if (st != PKV_OK) return st;
  }
  // The device the work runs on, and its array (a call with no tokens
  // resolves it too, so that a caller can do so before capturing a graph).
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int device = 0;
  uint32_t* plan = nullptr;
  if ((st = stream_device(s, &device)) != PKV_OK || (st = scratch_on(device, &plan)) != PKV_OK)
    return st;
  if (m.empty) return PKV_OK;
  if (build_plan) {
    pa.plan = plan;
    st = pkv::status_of(pkv::launch_plan(pa, s));
    if (st != PKV_OK) return st;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_built[device] = total_tokens;
  } else {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (total_tokens > g_built[device]) return PKV_ERR_SHAPE;  // no plan that long built here
  }
  m.args.plan = plan;
  return pkv::status_of(pkv::launch_mla(m.args, m.mode, m.heads_per_wave, s));
}
