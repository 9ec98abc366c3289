// token_plan.hip -- per-token placement of a ragged batch (page, offset,
// position), written once per batch layout.
//
// What it computes (page "mla_fused_rope_rmsnorm_quantization", Args:
// input_row_offsets and the KV collection's cache lengths and page table):
// for every new token t, the request b that owns it, its cache slot (= RoPE
// position) c[b] + t - o[b], and the physical page and offset of that slot.
// Every layer of a model step shares one batch layout, so a caller can build
// the plan once and hand it to mla_rope_rmsnorm_quant_planned for each layer:
// the fused step then reads one 16-byte entry per token instead of walking
// the two dependent steps of the address chain.
//
// Design: one wave64 per token, running the same address chain as the fused
// kernels (all offsets and prior lengths loaded at once, ballot, then the
// page-table entry); lane 0 writes the entry with one 16-byte store.  The
// plan is written with ordinary (cached) stores because every layer's kernel
// reads it back.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(256) void plan_kernel(const PlanArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t t = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  if (t >= a.total_tokens) return;
  const TokenSlot ts = find_slot(a.offsets, a.batch, a.cache_lengths, t, lane);
  PageSlot ps{};
  const bool placed =
      ts.ok && page_of(a.page_table, a.pt_stride, a.num_pages, a.page_size, ts, &ps);
  if (lane == 0) {
    const uint4 e = placed ? make_uint4(ps.page, ps.offset, ts.slot, 1u) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(a.plan + 4 * (uint64_t)t) = e;
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  const uint64_t blocks = ((uint64_t)a.total_tokens + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
