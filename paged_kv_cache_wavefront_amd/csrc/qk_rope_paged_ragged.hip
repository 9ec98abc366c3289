// qk_rope_paged_ragged.hip -- paged-ragged fused Q/K RoPE for gfx950.
//
// What it computes (page "generic_fused_qk_rope_bshd_paged_ragged", summary,
// Parameters, Args): RoPE of every Q head into the output tensor and, in the
// same launch, RoPE in place of the new tokens' K rows in the paged cache of
// layer layer_idx (one launch, so the K rotation is ordered after whatever
// wrote K).  Position = position_ids[t] when given, else the token's slot.
// Optional per-head RMSNorm of K (first k_norm_cols columns, gamma) runs
// before the rotation, with a single bf16 rounding at the end.
//
// Lane geometry (one wave64 per token, D = head_dim):
// * interleaved: lane holds 8 consecutive values = 4 adjacent pairs, D/8 lanes
//   per head; one 16-byte load per head per lane, 64/(D/8) heads per wave
//   instruction (contiguous 1 KiB per instruction).
// * rotate-half: lane holds values 8m..8m+7 and D/2+8m..D/2+8m+7 = 8 pairs,
//   D/16 lanes per head, two 16-byte loads per head per lane.
// Pair i of a lane needs freqs columns 2i, 2i+1: 8 (interleaved) or 16
// consecutive floats per lane, loaded once per token.  The K norm sums over
// the lanes of one head with DPP inside a 16-lane row.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;

// gamma values for this lane's 8 columns base..base+7 (0 beyond cols).
__device__ __forceinline__ void load_gamma8(const uint16_t* __restrict__ g, uint32_t base,
                                            uint32_t cols, float (&out)[8]) {
  if (base + 8 <= cols) {
    unpack8(*reinterpret_cast<const uint4*>(g + base), out);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      out[k] = (base + k < cols) ? __uint_as_float((uint32_t)g[base + k] << 16) : 0.0f;
  }
}

template <int D, bool INTER>
struct Geometry {
  static constexpr int kLanesPerHead = INTER ? D / 8 : D / 16;
  static constexpr int kHeadsPerInstr = kWave / kLanesPerHead;
  static constexpr int kCs = INTER ? 8 : 16;  // cos/sin floats per lane
  static constexpr int kQBatch = 8;            // head-instructions in flight
};

// Rotate one lane's values in place.  Interleaved: pairs (a[2k], a[2k+1]),
// k < 4.  Rotate-half: pairs (a[k], b[k]), k < 8.  cs: cos/sin per pair.
template <bool INTER>
__device__ __forceinline__ void rotate(float (&a)[8], float (&b)[8], const float* cs) {
  if constexpr (INTER) {
#pragma unroll
    for (int k = 0; k < 4; ++k) rotate_pair(a[2 * k], a[2 * k + 1], cs[2 * k], cs[2 * k + 1]);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) rotate_pair(a[k], b[k], cs[2 * k], cs[2 * k + 1]);
  }
}

template <int D, bool INTER>
__global__ __launch_bounds__(256) void qk_rope_kernel(const QkArgs a) {
  using Geo = Geometry<D, INTER>;
  constexpr int LP = Geo::kLanesPerHead, HPI = Geo::kHeadsPerInstr, QB = Geo::kQBatch;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t t =
      uniform(xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + (threadIdx.x / kWave));
  if (t >= a.total_tokens) return;
  const int m = lane % LP;
  const uint32_t hl = (uint32_t)(lane / LP);
  const uint32_t col0 = 8 * m;                       // first column of this lane
  const uint32_t col1 = INTER ? 0u : D / 2 + 8 * m;  // rotate-half: second chunk

  const uint16_t* qsrc = a.q_in + (int64_t)t * a.qi_tok + col0;
  uint16_t* qdst = a.q_out + (int64_t)t * a.qo_tok + col0;
  uint4 qa[QB], qb[QB];
  auto load_q = [&](uint32_t hbase) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const uint32_t h = hbase + i * HPI + hl;
      if (h < a.num_q_heads) {
        const uint16_t* p = qsrc + (int64_t)h * a.qi_head;
        qa[i] = *reinterpret_cast<const uint4*>(p);
        if constexpr (!INTER) qb[i] = *reinterpret_cast<const uint4*>(p + D / 2);
      }
    }
  };
  load_q(0);

  const CacheView& cv = a.cache;
  const SlotAddr s = locate(a.offsets, a.batch, cv.cache_lengths, cv.page_table, cv.pt_stride,
                            cv.num_pages, cv.page_size, t, lane);
  uint32_t pos = s.slot;
  if (s.ok && a.position_ids != nullptr) pos = uniform(a.position_ids[t]);
  if (!s.ok || pos >= a.max_seq_len) {
    count_skip(cv.error_count, lane);
    return;
  }
  float cs[Geo::kCs];
  {
    const float4* fr =
        reinterpret_cast<const float4*>(a.freqs + (int64_t)pos * D + Geo::kCs * m);
#pragma unroll
    for (int i = 0; i < Geo::kCs / 4; ++i) {
      const float4 v = fr[i];
      cs[4 * i] = v.x; cs[4 * i + 1] = v.y; cs[4 * i + 2] = v.z; cs[4 * i + 3] = v.w;
    }
  }

  // ---- Q ----------------------------------------------------------------------
  auto rotate_store_q = [&](uint32_t hbase) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const uint32_t h = hbase + i * HPI + hl;
      if (h < a.num_q_heads) {
        float x[8], y[8];
        unpack8(qa[i], x);
        if constexpr (!INTER) unpack8(qb[i], y);
        rotate<INTER>(x, y, cs);
        uint16_t* p = qdst + (int64_t)h * a.qo_head;
        *reinterpret_cast<uint4*>(p) = pack8_bf16(x);
        if constexpr (!INTER) *reinterpret_cast<uint4*>(p + D / 2) = pack8_bf16(y);
      }
    }
  };
  rotate_store_q(0);
  for (uint32_t hbase = HPI * QB; hbase < a.num_q_heads; hbase += HPI * QB) {
    load_q(hbase);
    rotate_store_q(hbase);
  }

  // ---- K (in place), optional per-head RMSNorm first ------------------------
  const bool knorm = a.k_gamma != nullptr;
  const uint32_t C = a.k_norm_cols;
  float ga[8] = {}, gb[8] = {};
  if (knorm) {
    load_gamma8(a.k_gamma, col0, C, ga);
    if constexpr (!INTER) load_gamma8(a.k_gamma, col1, C, gb);
  }
  uint16_t* krow = static_cast<uint16_t*>(cv.layer_base) + (int64_t)s.page * cv.page_stride +
                   (int64_t)s.offset * cv.slot_stride + col0;
  for (uint32_t hbase = 0; hbase < cv.num_heads; hbase += HPI) {
    const uint32_t h = hbase + hl;
    const bool valid = h < cv.num_heads;
    uint16_t* p = krow + (int64_t)h * cv.head_stride;
    uint4 ka = {}, kb = {};
    if (valid) {
      ka = *reinterpret_cast<const uint4*>(p);
      if constexpr (!INTER) kb = *reinterpret_cast<const uint4*>(p + D / 2);
    }
    float x[8], y[8] = {};
    unpack8(ka, x);
    if constexpr (!INTER) unpack8(kb, y);
    if (knorm) {
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (col0 + k < C) ss = fmaf(x[k], x[k], ss);
        if (!INTER && col1 + k < C) ss = fmaf(y[k], y[k], ss);
      }
      ss = group_sum<LP>(ss);
      const float r = 1.0f / sqrtf(ss / (float)C + a.epsilon);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (col0 + k < C) x[k] = x[k] * r * ga[k];
        if (!INTER && col1 + k < C) y[k] = y[k] * r * gb[k];
      }
    }
    rotate<INTER>(x, y, cs);
    if (valid) {
      *reinterpret_cast<uint4*>(p) = pack8_bf16(x);
      if constexpr (!INTER) *reinterpret_cast<uint4*>(p + D / 2) = pack8_bf16(y);
    }
  }
}

template <int D, bool INTER>
hipError_t launch_one(const QkArgs& a, uint32_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((qk_rope_kernel<D, INTER>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_rope(const QkArgs& a, int head_dim, bool interleaved, hipStream_t stream) {
  const uint64_t blocks = ((uint64_t)a.total_tokens + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const uint32_t nb = (uint32_t)blocks;
  if (head_dim == 128)
    return interleaved ? launch_one<128, true>(a, nb, stream) : launch_one<128, false>(a, nb, stream);
  if (head_dim == 64)
    return interleaved ? launch_one<64, true>(a, nb, stream) : launch_one<64, false>(a, nb, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
