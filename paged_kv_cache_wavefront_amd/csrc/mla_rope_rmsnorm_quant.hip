// mla_rope_rmsnorm_quant.hip -- fused MLA pre-attention kernel for gfx950.
//
// What it computes (page "mla_fused_rope_rmsnorm_quantization", summary and
// Args; "mla_graph" module page, entry fused_rope_rmsnorm_quantization_kernel):
// for each new token, RoPE on every head of q_rope into q_rope_output, RMSNorm
// with gamma on the kv_norm_dim non-rope values of the latent row, RoPE on the
// row's rope tail, quantisation of the whole row, and its store into the paged
// cache of layer layer_idx at the token's slot.
//
// Design (bandwidth bound; no dense contraction, so no MFMA):
// * One wave64 per (token, chunk of heads).  Lane l handles head
//   16*g + l/4 of each 16-head group g, and within it the 8 rotate-half pairs
//   (8m + k, 32 + 8m + k), m = l % 4: two 16-byte loads per head per lane,
//   one per half, so no cross-lane exchange is needed for the pairing and each
//   wave instruction reads 16 heads x 64 contiguous bytes.
// * All q loads of the wave are issued before the address chain (offsets ->
//   cache length -> page table -> freqs row), so the chain's latency hides
//   behind the bulk traffic.
// * The 16 cos/sin floats a lane needs sit contiguously in the freqs row and
//   are identical for the 16 heads the wave touches: one 64-byte vector load
//   per lane per token, kept in registers (no LDS round trip).
// * The head-chunk-0 wave also owns the latent row: lane l holds non-rope
//   values 8l..8l+7 (one 16-byte load), lanes 0..3 hold the rope tail with
//   the same pairing and cos/sin as q.  The sum of squares (and the per-token
//   amax) reduce across the wave with DPP inside rows and readlane across
//   rows.  The row is converted to fp8 in registers (clamp to +-448, then
//   hardware round-to-nearest-even) and written with 8-byte stores.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRope = 64;               // rope_dim
constexpr int kNope = 512;              // kv_norm_dim = 64 lanes x 8
constexpr int kHalf = kRope / 2;
constexpr int kWavesPerBlock = 4;

// Rotate the 8 rotate-half pairs (lo[k], hi[k]) of one lane.  cs holds
// cos, sin of pair k at 2k, 2k+1.
__device__ __forceinline__ void rotate_pairs(float (&lo)[8], float (&hi)[8],
                                             const float (&cs)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) rotate_pair(lo[k], hi[k], cs[2 * k], cs[2 * k + 1]);
}

template <int G, MlaOut MODE>
__global__ __launch_bounds__(256) void mla_kernel(const MlaArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave =
      xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + (threadIdx.x / kWave);
  const uint32_t t = uniform(wave / a.chunks);
  const uint32_t chunk = uniform(wave - t * a.chunks);
  if (t >= a.total_tokens) return;

  // ---- issue the bulk loads (addresses depend on t only) --------------------
  const int m = lane & 3;
  const uint32_t h_lane = chunk * (16 * G) + (uint32_t)(lane >> 2);
  const uint16_t* qsrc = a.q_in + (int64_t)t * a.qi_tok + 8 * m;
  uint4 qlo[G], qhi[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t h = h_lane + 16 * g;
    if (h < a.num_heads) {
      const uint16_t* p = qsrc + (int64_t)h * a.qi_head;
      qlo[g] = *reinterpret_cast<const uint4*>(p);
      qhi[g] = *reinterpret_cast<const uint4*>(p + kHalf);
    }
  }
  const bool latent_wave = chunk == 0;
  uint4 xn = {}, gm = {}, tlo = {}, thi = {};
  if (latent_wave) {
    const uint16_t* row = a.latent + (int64_t)t * a.kv_row;
    xn = *reinterpret_cast<const uint4*>(row + 8 * lane);
    gm = *reinterpret_cast<const uint4*>(a.gamma + 8 * lane);
    if (lane < 4) {
      tlo = *reinterpret_cast<const uint4*>(row + kNope + 8 * lane);
      thi = *reinterpret_cast<const uint4*>(row + kNope + kHalf + 8 * lane);
    }
  }

  // ---- address chain: request, slot (= position), page, offset -------------
  const CacheView& cv = a.cache;
  const SlotAddr s = locate(a.offsets, a.batch, cv.cache_lengths, cv.page_table, cv.pt_stride,
                            cv.num_pages, cv.page_size, t, lane);
  if (!s.ok || s.slot >= a.max_seq_len) {
    if (latent_wave) count_skip(cv.error_count, lane);
    return;
  }
  float cs[16];
  {
    const float4* fr =
        reinterpret_cast<const float4*>(a.freqs + (int64_t)s.slot * kRope + 16 * m);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = fr[i];
      cs[4 * i] = v.x; cs[4 * i + 1] = v.y; cs[4 * i + 2] = v.z; cs[4 * i + 3] = v.w;
    }
  }

  // ---- q: rotate and store ---------------------------------------------------
  uint16_t* qdst = a.q_out + (int64_t)t * a.qo_tok + 8 * m;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t h = h_lane + 16 * g;
    if (h < a.num_heads) {
      float lo[8], hi[8];
      unpack8(qlo[g], lo);
      unpack8(qhi[g], hi);
      rotate_pairs(lo, hi, cs);
      uint16_t* p = qdst + (int64_t)h * a.qo_head;
      *reinterpret_cast<uint4*>(p) = pack8_bf16(lo);
      *reinterpret_cast<uint4*>(p + kHalf) = pack8_bf16(hi);
    }
  }
  if (!latent_wave) return;

  // ---- latent row: RMSNorm (non-rope part), RoPE (tail) ---------------------
  float y[8], g8[8];
  unpack8(xn, y);
  unpack8(gm, g8);
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(y[k], y[k], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / kNope) + a.epsilon);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = y[k] * r * g8[k];
  float tl[8], th[8];
  unpack8(tlo, tl);
  unpack8(thi, th);
  rotate_pairs(tl, th, cs);  // meaningful on lanes 0..3 only

  const int64_t row_elems = (int64_t)s.page * cv.page_stride + (int64_t)s.offset * cv.slot_stride;
  if constexpr (MODE == MlaOut::Bf16) {
    uint16_t* row = static_cast<uint16_t*>(cv.layer_base) + row_elems;
    *reinterpret_cast<uint4*>(row + 8 * lane) = pack8_bf16(y);
    if (lane < 4) {
      *reinterpret_cast<uint4*>(row + kNope + 8 * lane) = pack8_bf16(tl);
      *reinterpret_cast<uint4*>(row + kNope + kHalf + 8 * lane) = pack8_bf16(th);
    }
    return;
  } else {
    float inv;
    if constexpr (MODE == MlaOut::Fp8PerTensor) {
      inv = 1.0f / *a.tensor_scale;
    } else {
      float am = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(y[k]));
      if (lane < 4) {
#pragma unroll
        for (int k = 0; k < 8; ++k) am = fmaxf(am, fmaxf(fabsf(tl[k]), fabsf(th[k])));
      }
      am = wave_max(am);
      const float st = am / 448.0f;
      inv = st > 0.0f ? 1.0f / st : 0.0f;
      if (lane == 0)
        a.token_scales[((int64_t)s.page * cv.page_size + s.offset) * cv.num_heads] = st;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      y[k] *= inv;
      tl[k] *= inv;
      th[k] *= inv;
    }
    uint8_t* row = static_cast<uint8_t*>(cv.layer_base) + row_elems;
    *reinterpret_cast<uint2*>(row + 8 * lane) = pack8_fp8(y);
    if (lane < 4) {
      *reinterpret_cast<uint2*>(row + kNope + 8 * lane) = pack8_fp8(tl);
      *reinterpret_cast<uint2*>(row + kNope + kHalf + 8 * lane) = pack8_fp8(th);
    }
  }
}

template <int G>
hipError_t launch_g(const MlaArgs& a, MlaOut mode, uint32_t blocks, hipStream_t stream) {
  switch (mode) {
    case MlaOut::Fp8PerTensor:
      hipLaunchKernelGGL((mla_kernel<G, MlaOut::Fp8PerTensor>), dim3(blocks), dim3(256), 0,
                         stream, a);
      break;
    case MlaOut::Fp8PerToken:
      hipLaunchKernelGGL((mla_kernel<G, MlaOut::Fp8PerToken>), dim3(blocks), dim3(256), 0,
                         stream, a);
      break;
    case MlaOut::Bf16:
      hipLaunchKernelGGL((mla_kernel<G, MlaOut::Bf16>), dim3(blocks), dim3(256), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaArgs& a, MlaOut mode, int heads_per_wave, hipStream_t stream) {
  const uint64_t waves = (uint64_t)a.total_tokens * a.chunks;
  const uint64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  switch (heads_per_wave) {
    case 16: return launch_g<1>(a, mode, (uint32_t)blocks, stream);
    case 32: return launch_g<2>(a, mode, (uint32_t)blocks, stream);
    case 64: return launch_g<4>(a, mode, (uint32_t)blocks, stream);
    case 128: return launch_g<8>(a, mode, (uint32_t)blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
