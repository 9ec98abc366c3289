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
// One wave64 per token; lane holds 8 consecutive columns (16 bytes of bf16,
// 8 bytes of fp8) of one head, D/8 lanes per head, and the per-head sum of
// squares (and, for a per-token fp8 cache, the max for the fresh scale)
// reduces with DPP inside the head's lanes.  An fp8 cache is read as
// code * scale; a per-tensor cache re-encodes the normalised columns with its
// scale, a per-token cache stores max|y| / 448 per head and re-encodes the
// whole head.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16x2(v, 0.0f) << 16); }

template <int D, bool MBC, KMode KM>
__global__ __launch_bounds__(256) void kv_norm_kernel(const KvNormArgs a) {
  constexpr int LP = D / 8, HPI = kWave / LP;
  constexpr int64_t EB = KM == KMode::Bf16 ? 2 : 1;
  // a per-token fp8 head shares one scale: the whole head is re-encoded
  constexpr bool kWholeHead = KM == KMode::Fp8PerToken;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t t =
      uniform(xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + (threadIdx.x / kWave));
  if (t >= a.total_tokens) return;
  const int m = lane % LP;
  const uint32_t hl = (uint32_t)(lane / LP);
  const uint32_t col0 = 8 * m;
  const uint32_t C = a.gamma_len;

  // gamma (+ weight_offset) of this lane's columns, loaded before the chain
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

  const CacheView& cv = a.cache;
  const TokenSlot ts = find_slot(a.offsets, a.batch, cv.cache_lengths, t, lane);
  PageSlot ps{};
  if (!(ts.ok && page_of(cv.page_table, cv.pt_stride, cv.num_pages, cv.page_size, ts, &ps))) {
    count_skip(cv.error_count, lane);
    return;
  }

  char* krow = static_cast<char*>(cv.layer_base) +
               EB * ((int64_t)ps.page * cv.page_stride + (int64_t)ps.offset * cv.slot_stride +
                     col0);
  const int64_t slot_head0 = ((int64_t)ps.page * cv.page_size + ps.offset) * cv.num_heads;
  const bool touches = kWholeHead || col0 < C;
  float tensor_scale = 1.0f, tensor_inv = 1.0f;
  if constexpr (KM == KMode::Fp8PerTensor) {
    tensor_scale = a.k_scales[0];
    tensor_inv = 1.0f / tensor_scale;
  }
  for (uint32_t hbase = 0; hbase < cv.num_heads; hbase += HPI) {
    const uint32_t h = hbase + hl;
    const bool valid = h < cv.num_heads && touches;
    char* p = krow + EB * (int64_t)h * cv.head_stride;
    float x[8];
    if constexpr (KM == KMode::Bf16) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (valid) raw = *reinterpret_cast<const uint4*>(p);
      unpack8(raw, x);
    } else {
      uint2 raw = make_uint2(0, 0);
      float ks = 0.0f;
      if (valid) {
        raw = *reinterpret_cast<const uint2*>(p);
        ks = KM == KMode::Fp8PerTensor ? tensor_scale : a.k_scales[slot_head0 + h];
      }
      unpack8_fp8(raw.x, raw.y, x);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] *= ks;
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (col0 + k < C) ss = fmaf(x[k], x[k], ss);
    ss = group_sum<LP>(ss);
    const float r = 1.0f / sqrtf(ss / (float)C + a.epsilon);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (col0 + k >= C) continue;
      if constexpr (MBC) {
        x[k] = x[k] * g[k] * r;
      } else {
        x[k] = round_bf16(x[k] * r) * g[k];
      }
    }
    if constexpr (KM == KMode::Bf16) {
      if (valid) {
        if (col0 + 8 <= C) {
          *reinterpret_cast<uint4*>(p) = pack8_bf16(x);
        } else {
          uint16_t* e = reinterpret_cast<uint16_t*>(p);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (col0 + k < C) e[k] = (uint16_t)(pack_bf16x2(x[k], 0.0f) & 0xffffu);
        }
      }
    } else {
      float inv = tensor_inv;
      if constexpr (KM == KMode::Fp8PerToken) {
        float am = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[k]));
        am = group_max<LP>(am);
        const float st = am / 448.0f;
        inv = st > 0.0f ? 1.0f / st : 0.0f;
        if (valid && m == 0) a.k_scales[slot_head0 + h] = st;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] *= inv;
      const uint2 codes = pack8_fp8(x);
      if (valid) {
        if (kWholeHead || col0 + 8 <= C) {
          *reinterpret_cast<uint2*>(p) = codes;
        } else {
          uint8_t* e = reinterpret_cast<uint8_t*>(p);
          const uint32_t w[2] = {codes.x, codes.y};
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (col0 + k < C) e[k] = (uint8_t)(w[k / 4] >> (8 * (k % 4)));
        }
      }
    }
  }
}

template <int D, KMode KM>
hipError_t launch_dk(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  if (mbc)
    hipLaunchKernelGGL((kv_norm_kernel<D, true, KM>), dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((kv_norm_kernel<D, false, KM>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const KvNormArgs& a, bool mbc, KMode km, uint32_t blocks, hipStream_t stream) {
  switch (km) {
    case KMode::Bf16: return launch_dk<D, KMode::Bf16>(a, mbc, blocks, stream);
    case KMode::Fp8PerTensor: return launch_dk<D, KMode::Fp8PerTensor>(a, true, blocks, stream);
    case KMode::Fp8PerToken: return launch_dk<D, KMode::Fp8PerToken>(a, true, blocks, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_norm(const KvNormArgs& a, bool multiply_before_cast, KMode kmode,
                          hipStream_t stream) {
  const uint64_t blocks = ((uint64_t)a.total_tokens + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const uint32_t nb = (uint32_t)blocks;
  switch (a.head_dim) {
    case 64: return launch_d<64>(a, multiply_before_cast, kmode, nb, stream);
    case 128: return launch_d<128>(a, multiply_before_cast, kmode, nb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
