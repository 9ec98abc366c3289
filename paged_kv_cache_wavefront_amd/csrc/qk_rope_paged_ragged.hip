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
// Lane geometry (one wave64 per token, D = head_dim): each lane owns one
// 16-byte chunk (8 values) of a head, D/8 lanes per head, so every wave
// instruction moves 64 x 16 contiguous bytes.
// * interleaved: lane k holds values 8k..8k+7 = adjacent pairs 4k..4k+3.
// * rotate-half: lane k < D/16 holds values 8k.. of the first half; lane
//   k >= D/16 holds the second-half values of pairs 8(D/8-1-k)..; the partner
//   of lane k is lane D/8-1-k, reached by one DPP mirror per dword.
// Pair i needs freqs columns 2i, 2i+1: 8 or 16 consecutive floats per lane,
// loaded once per token.  Q is read with non-temporal loads.
//
// Optional K norm: r = 1/sqrt(mean(x^2) + eps) over the first C columns of a
// head (DPP sum over the head's lanes).  Normalised values enter the rotation
// as x * gamma (exact in fp32) and r is applied after it, so an fp32 rounding
// of x * r * gamma cannot be amplified by cancellation in the rotation; a
// pair with one normalised and one plain member takes r before the rotation.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;

// gamma for the 8 columns base..base+7; 1 where the column lies past cols or
// when there is no norm.
__device__ __forceinline__ void load_gamma8(const uint16_t* __restrict__ g, int base, int cols,
                                            bool use, float (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = 1.0f;
  if (!use || base >= cols) return;
  if (base + 8 <= cols) {
    unpack8(load16(g + base), out);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (base + j < cols) out[j] = __uint_as_float((uint32_t)g[base + j] << 16);
  }
}

template <int D, bool INTER>
struct Geometry {
  static constexpr int kLanesPerHead = D / 8;
  static constexpr int kHeadsPerInstr = kWave / kLanesPerHead;
  static constexpr int kCs = INTER ? 8 : 16;  // cos/sin floats per lane
  static constexpr int kQBatch = 8;            // head-instructions in flight
};

template <int D, bool INTER>
struct LaneRole {
  int k;            // lane within the head
  bool first;       // rotate-half: holds first-half values
  int chunk;        // 16-byte chunk of the head row it loads / stores
  int partner_chunk;
  int cs_base;      // first freqs column it needs
  __device__ __forceinline__ explicit LaneRole(int lane) {
    constexpr int LP = D / 8, HALF = LP / 2;
    k = lane % LP;
    if constexpr (INTER) {
      first = true;
      chunk = partner_chunk = k;
      cs_base = 8 * k;
    } else {
      first = k < HALF;
      const int pb = first ? k : LP - 1 - k;  // pair block: pairs 8pb..8pb+7
      chunk = first ? k : LP + HALF - 1 - k;
      partner_chunk = first ? LP + HALF - 1 - (LP - 1 - k) : LP - 1 - k;
      cs_base = 16 * pb;
    }
  }
};

// Rotate the lane's values.  own: this lane's 8 values; par: the partner's
// (rotate-half only).  pre_own / pre_par scale inputs, post scales outputs.
template <bool INTER>
__device__ __forceinline__ void rotate_lane(float (&own)[8], const float (&par)[8],
                                            const float* cs, bool first,
                                            const float (&pre_own)[8], const float (&pre_par)[8],
                                            const float (&post)[8]) {
  if constexpr (INTER) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = own[2 * q] * pre_own[2 * q], b = own[2 * q + 1] * pre_own[2 * q + 1];
      const float c = cs[2 * q], s = cs[2 * q + 1];
      own[2 * q] = sum_of_products(a, c, -b, s) * post[2 * q];
      own[2 * q + 1] = sum_of_products(b, c, a, s) * post[2 * q + 1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = par[j] * pre_par[j];
      own[j] = sum_of_products(own[j] * pre_own[j], cs[2 * j], first ? -p : p, cs[2 * j + 1]) *
               post[j];
    }
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
  const LaneRole<D, INTER> role(lane);
  const uint32_t hl = (uint32_t)(lane / LP);
  const int col = 8 * role.chunk;          // first column this lane owns
  const int pcol = 8 * role.partner_chunk;  // first column of the partner's values

  const uint16_t* qsrc = a.q_in + (int64_t)t * a.qi_tok + col;
  uint16_t* qdst = a.q_out + (int64_t)t * a.qo_tok + col;
  uint4 qv[QB];
  auto load_q = [&](uint32_t hbase) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const uint32_t h = hbase + i * HPI + hl;
      qv[i] = make_uint4(0, 0, 0, 0);
      if (h < a.num_q_heads) qv[i] = load16_stream(qsrc + (int64_t)h * a.qi_head);
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
    const float4* fr = reinterpret_cast<const float4*>(a.freqs + (int64_t)pos * D + role.cs_base);
#pragma unroll
    for (int i = 0; i < Geo::kCs / 4; ++i) {
      const float4 v = fr[i];
      cs[4 * i] = v.x; cs[4 * i + 1] = v.y; cs[4 * i + 2] = v.z; cs[4 * i + 3] = v.w;
    }
  }
  float ones[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = 1.0f;

  // ---- Q ----------------------------------------------------------------------
  auto rotate_store_q = [&](uint32_t hbase) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      float own[8], par[8] = {};
      unpack8(qv[i], own);
      if constexpr (!INTER) unpack8(mirror16<LP>(qv[i]), par);
      rotate_lane<INTER>(own, par, cs, role.first, ones, ones, ones);
      const uint32_t h = hbase + i * HPI + hl;
      if (h < a.num_q_heads) store16(qdst + (int64_t)h * a.qo_head, pack8_bf16(own));
    }
  };
  rotate_store_q(0);
  for (uint32_t hbase = HPI * QB; hbase < a.num_q_heads; hbase += HPI * QB) {
    load_q(hbase);
    rotate_store_q(hbase);
  }

  // ---- K (in place), optional per-head RMSNorm first ------------------------
  const bool knorm = a.k_gamma != nullptr;
  const int C = (int)a.k_norm_cols;
  float g[8], gp[8];  // gamma of this lane's columns and of the partner's
  load_gamma8(a.k_gamma, col, C, knorm, g);
  load_gamma8(a.k_gamma, pcol, C, knorm && !INTER, gp);
  uint16_t* krow = static_cast<uint16_t*>(cv.layer_base) + (int64_t)s.page * cv.page_stride +
                   (int64_t)s.offset * cv.slot_stride + col;
  for (uint32_t hbase = 0; hbase < cv.num_heads; hbase += HPI) {
    const uint32_t h = hbase + hl;
    const bool valid = h < cv.num_heads;
    uint16_t* p = krow + (int64_t)h * cv.head_stride;
    uint4 kv = make_uint4(0, 0, 0, 0);
    if (valid) kv = load16(p);
    float own[8], par[8] = {};
    unpack8(kv, own);
    if constexpr (!INTER) unpack8(mirror16<LP>(kv), par);
    float pre_own[8], pre_par[8], post[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pre_own[j] = pre_par[j] = post[j] = 1.0f;
    if (knorm) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (col + j < C) ss = fmaf(own[j], own[j], ss);
      ss = group_sum<LP>(ss);
      const float r = 1.0f / sqrtf(ss / (float)C + a.epsilon);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        own[j] *= g[j];  // exact (bf16 x bf16); g = 1 past C
        par[j] *= gp[j];
        // is this value / its pair partner inside the normalised span?
        bool in_me, in_other;
        if constexpr (INTER) {
          in_me = col + j < C;
          in_other = col + (j ^ 1) < C;
        } else {
          in_me = col + j < C;
          in_other = pcol + j < C;
        }
        pre_own[j] = (in_me && !in_other) ? r : 1.0f;
        pre_par[j] = (in_other && !in_me) ? r : 1.0f;
        post[j] = (in_me && in_other) ? r : 1.0f;
      }
    }
    rotate_lane<INTER>(own, par, cs, role.first, pre_own, pre_par, post);
    if (valid) store16(p, pack8_bf16(own));
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
