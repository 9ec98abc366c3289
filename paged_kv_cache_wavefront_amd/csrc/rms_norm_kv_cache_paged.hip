// rms_norm_kv_cache_paged.hip -- in-place RMSNorm of new K-cache rows, gfx950.
//
// What it computes (page "rms_norm_kv_cache_ragged_paged"): for each of the
// first total_seq_len new tokens, found through input_row_offsets and placed
// through the page table, and for each head, the first len(gamma) columns
// become x * r * (gamma + weight_offset), r = 1/sqrt(mean(x^2) + eps) over
// those columns; the other columns are not written.  multiply_before_cast
// selects one bf16 rounding after the gamma product, or a rounding of x * r
// before it and another after it.
//
// One wave64 per token; lane holds 8 consecutive columns (16 bytes) of one
// head, D/8 lanes per head, and the per-head sum of squares reduces with DPP
// inside the head's lanes.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16x2(v, 0.0f) << 16); }

template <int D, bool MBC>
__global__ __launch_bounds__(256) void kv_norm_kernel(const KvNormArgs a) {
  constexpr int LP = D / 8, HPI = kWave / LP;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t t =
      uniform(xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + (threadIdx.x / kWave));
  if (t >= a.total_tokens) return;
  const int m = lane % LP;
  const uint32_t hl = (uint32_t)(lane / LP);
  const uint32_t col0 = 8 * m;
  const uint32_t C = a.gamma_len;

  const CacheView& cv = a.cache;
  const TokenSlot ts = find_slot(a.offsets, a.batch, cv.cache_lengths, t, lane);
  PageSlot ps{};
  if (!(ts.ok && page_of(cv.page_table, cv.pt_stride, cv.num_pages, cv.page_size, ts, &ps))) {
    count_skip(cv.error_count, lane);
    return;
  }
  float g[8];
  if (col0 + 8 <= C) {
    unpack8(*reinterpret_cast<const uint4*>(a.gamma + col0), g);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      g[k] = (col0 + k < C) ? __uint_as_float((uint32_t)a.gamma[col0 + k] << 16) : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) g[k] += a.weight_offset;

  uint16_t* krow = static_cast<uint16_t*>(cv.layer_base) + (int64_t)ps.page * cv.page_stride +
                   (int64_t)ps.offset * cv.slot_stride + col0;
  const bool touches = col0 < C;
  for (uint32_t hbase = 0; hbase < cv.num_heads; hbase += HPI) {
    const uint32_t h = hbase + hl;
    const bool valid = h < cv.num_heads && touches;
    uint16_t* p = krow + (int64_t)h * cv.head_stride;
    uint4 raw = {};
    if (valid) raw = *reinterpret_cast<const uint4*>(p);
    float x[8];
    unpack8(raw, x);
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (col0 + k < C) ss = fmaf(x[k], x[k], ss);
    ss = group_sum<LP>(ss);
    const float r = 1.0f / sqrtf(ss / (float)C + a.epsilon);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (MBC) {
        x[k] = x[k] * r * g[k];
      } else {
        x[k] = round_bf16(x[k] * r) * g[k];
      }
    }
    if (valid) {
      if (col0 + 8 <= C) {
        *reinterpret_cast<uint4*>(p) = pack8_bf16(x);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (col0 + k < C) p[k] = (uint16_t)(pack_bf16x2(x[k], 0.0f) & 0xffffu);
      }
    }
  }
}

template <int D>
hipError_t launch_d(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  if (mbc)
    hipLaunchKernelGGL((kv_norm_kernel<D, true>), dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((kv_norm_kernel<D, false>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_norm(const KvNormArgs& a, bool multiply_before_cast, hipStream_t stream) {
  const uint64_t blocks = ((uint64_t)a.total_tokens + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const uint32_t nb = (uint32_t)blocks;
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, multiply_before_cast, nb, stream);
    case 128: return launch_d<128>(a, multiply_before_cast, nb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
