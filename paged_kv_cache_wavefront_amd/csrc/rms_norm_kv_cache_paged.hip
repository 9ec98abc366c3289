// rms_norm_kv_cache_paged.hip -- in-place RMSNorm of new K-cache rows, gfx950.
//
// What it computes (page "rms_norm_kv_cache_ragged_paged"): for each of the
// first total_seq_len new tokens, found through input_row_offsets and placed
// through the page table, and for each head, the first len(gamma) columns
// become x * r * (gamma + weight_offset), r = 1/sqrt(mean(x^2) + eps) over
// those columns (gamma bf16, fp16 or fp32); the other columns are not
// written.  multiply_before_cast selects one bf16 rounding after the gamma
// product, or a rounding of x * r before it and another after it.
//
// Per-token statistic (per_head_norm = 0, a reading: the page lists the flag
// without describing it): one r over the first len(gamma) columns of every
// head of the token, from a wave-wide sum.  Both forms load a chunk of up to
// 4 head groups first (phase 1, sums), then normalise and store it (phase 2).
// A token whose heads fill more than one chunk first sums the statistic over
// all of them (ordinary loads, so that the lines stay in L2 for phase 1 of
// each chunk, which then only reloads and normalises).
//
// Planned form: with a token plan (token_plan.hip) the token's (page,
// offset) is one checked plan entry instead of the address chain, which in
// this in-place kernel lies wholly in front of the row loads.
//
// One wave64 per token; lane holds 8 consecutive columns (16 bytes of bf16,
// 8 bytes of fp8) of one head, a head occupies LP lanes (D/8 rounded up to a
// power of two: the lanes past the head's D/8 chunks idle for D = 80, 96),
// and the per-head sum of squares (and, for a per-token fp8 cache, the max
// for the fresh scale) reduces with DPP inside the head's lanes.  An fp8 cache is read as
// code * scale; a per-tensor cache re-encodes the normalised columns with its
// scale, a per-token cache stores max|y| / 448 per head and re-encodes the
// whole head.  K rows are read and written with non-temporal accesses (they
// are touched once; plain loads measured slower here, before the
// non-temporal stores of the same lines).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxIter = 4;  // head groups held in registers at once

__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16x2(v, 0.0f) << 16); }

// PLANNED: each token's (page, offset) comes from a token plan entry, one
// scalar 16-byte load, instead of the two-step address chain.  GT: gamma of
// the type in a.gamma_type; otherwise bf16, with no type branch.
template <int D, bool MBC, KMode KM, bool PER_HEAD, bool PLANNED, bool GT>
__global__ __launch_bounds__(256) void kv_norm_kernel(const KvNormArgs a) {
  constexpr int NC = D / 8, LP = pow2_at_least(NC), HPI = kWave / LP;
  constexpr int64_t EB = KM == KMode::Bf16 ? 2 : 1;
  // a per-token fp8 head shares one scale: the whole head is re-encoded
  constexpr bool kWholeHead = KM == KMode::Fp8PerToken;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t t =
      uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
  if (t >= a.total_tokens) return;
  const int m = lane % LP;
  const bool active = m < NC;  // always true unless D/8 is not a power of two
  const uint32_t hl = (uint32_t)(lane / LP);
  const uint32_t col0 = active ? 8 * m : 0;
  const uint32_t C = a.gamma_len;

  // gamma of this lane's columns (bf16, fp16 or fp32, widened exactly): a
  // whole chunk is loaded here, before the chain, and widened only before its
  // first use, so that its wait holds up neither the chain's nor the rows' loads
  const int gamma_type = GT ? a.gamma_type : (int)kBf16;
  const bool gamma_chunk = col0 + 8 <= C;
  uint4 g_lo = make_uint4(0, 0, 0, 0), g_hi = make_uint4(0, 0, 0, 0);
  if (gamma_chunk) {
    const uint4* gp = reinterpret_cast<const uint4*>(static_cast<const char*>(a.gamma) +
                                                     (gamma_type == kF32 ? 4 : 2) * col0);
    g_lo = load16(gp);
    if (gamma_type == kF32) g_hi = load16(gp + 1);
  }

  const CacheView& cv = a.cache;
  PageSlot ps{};
  bool placed;
  if constexpr (PLANNED) {
    const uint4 e = *reinterpret_cast<const uint4*>(a.plan + 4 * (uint64_t)t);
    ps.page = uniform(e.x);
    ps.offset = uniform(e.y);
    placed = e.w != 0 && ps.page < cv.num_pages && ps.offset < cv.page_size;
  } else {
    const TokenSlot ts = find_slot(a.offsets, a.batch, cv.cache_lengths, t, lane);
    placed = ts.ok && page_of(cv.page_table, cv.pt_stride, cv.num_pages, cv.page_size, ts, &ps);
  }
  if (!placed) {
    count_skip(cv.error_count, lane);
    return;
  }

  char* krow = static_cast<char*>(cv.layer_base) +
               EB * ((int64_t)ps.page * cv.page_stride + (int64_t)ps.offset * cv.slot_stride +
                     col0);
  const int64_t slot_head0 = ((int64_t)ps.page * cv.page_size + ps.offset) * cv.num_heads;
  const bool touches = active && (kWholeHead || col0 < C);
  float tensor_scale = 1.0f, tensor_inv = 1.0f;
  if constexpr (KM == KMode::Fp8PerTensor) {
    tensor_scale = a.k_scales[0];
    tensor_inv = rcp_hw(tensor_scale);
  }
  // head groups of HPI heads, kMaxIter groups at a time
  const uint32_t nit = (cv.num_heads + HPI - 1) / HPI;
  // per-token statistic over more than one chunk: summed in a pass of its own
  const bool presum = !PER_HEAD && nit > (uint32_t)kMaxIter;
  float r_presum = 0.0f;
  if (!PER_HEAD && presum) {
    float ss_all = 0.0f;
    for (uint32_t it = 0; it < nit; ++it) {
      const uint32_t h = it * HPI + hl;
      const bool valid = h < cv.num_heads && touches;
      const char* p = krow + EB * (int64_t)h * cv.head_stride;
      float y[8];
      if constexpr (KM == KMode::Bf16) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (valid) raw = load16(p);
        unpack8(raw, y);
      } else {
        uint2 raw = make_uint2(0, 0);
        float ks = 0.0f;
        if (valid) {
          raw = *reinterpret_cast<const uint2*>(p);
          ks = KM == KMode::Fp8PerTensor ? tensor_scale : a.k_scales[slot_head0 + h];
        }
        unpack8_fp8(raw.x, raw.y, y);
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] *= ks;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (col0 + k < C) ss_all = fmaf(y[k], y[k], ss_all);
    }
    r_presum = rsqrt_hw(wave_sum(ss_all) * a.inv_token_cols + a.epsilon);
  }
  for (uint32_t base = 0; base < nit; base += kMaxIter) {
    // phase 1: load the chunk's heads this lane serves, then the sums of
    // squares.  Every load is issued before any value is used: the chunk's
    // head groups end at a uniform break, which no load may be moved across,
    // so a use between two loads would make each wait for the one before.
    // A lane outside the rows skips its load and takes zeros only in the
    // second loop (a zero written before the load would make the load wait
    // for everything still in flight).
    uint4 raw16[kMaxIter];  // bf16 rows
    uint2 raw8[kMaxIter];   // fp8 codes
    float ks[kMaxIter];     // their scales
    bool valid[kMaxIter];
#pragma unroll
    for (int it = 0; it < kMaxIter; ++it) {
      if (base + it >= nit) break;
      const uint32_t h = (base + it) * HPI + hl;
      valid[it] = h < cv.num_heads && touches;
      const char* p = krow + EB * (int64_t)h * cv.head_stride;
      if (valid[it]) {
        if constexpr (KM == KMode::Bf16) {
          raw16[it] = load16_stream(p);
        } else {
          raw8[it] = load8_stream(p);
          ks[it] = KM == KMode::Fp8PerTensor ? tensor_scale : a.k_scales[slot_head0 + h];
        }
      }
    }
    // the values of head group it, widened from the packed loads (twice:
    // for the sums and again for the stores, which keeps the chunk packed in
    // registers between the two phases)
    auto widen = [&](int it, float (&y)[8]) {
      if constexpr (KM == KMode::Bf16) {
        unpack8(raw16[it], y);
      } else {
        unpack8_fp8(raw8[it].x, raw8[it].y, y);
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] *= ks[it];
      }
    };
    float rh[kMaxIter];
    float ss_token = 0.0f;
#pragma unroll
    for (int it = 0; it < kMaxIter; ++it) {
      if (base + it >= nit) break;
      if (!valid[it]) {
        raw16[it] = make_uint4(0, 0, 0, 0);
        raw8[it] = make_uint2(0, 0);
        ks[it] = 0.0f;
      }
      float y[8];
      widen(it, y);
      float ss = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (col0 + k < C) ss = fmaf(y[k], y[k], ss);
      if constexpr (PER_HEAD) {
        ss = group_sum<LP>(ss);
        rh[it] = rsqrt_hw(ss * a.inv_cols + a.epsilon);
      } else {
        ss_token += ss;
      }
    }
    float r_token = r_presum;
    if constexpr (!PER_HEAD) {
      if (!presum)
        r_token = rsqrt_hw(wave_sum(ss_token) * a.inv_token_cols + a.epsilon);
    }

    // gamma + weight_offset, widened only now that phase 1 has issued its
    // loads: the chunk loaded above (the empty asm keeps the widening, and
    // with it the wait for gamma, from being hoisted in front of them), or a
    // partial chunk (the columns past gamma_len take 0) element by element
    float g[8];
    if (gamma_chunk) {
      pin_vgprs(g_lo);
      if (gamma_type == kF32) {
        pin_vgprs(g_hi);
        const uint32_t w[8] = {g_lo.x, g_lo.y, g_lo.z, g_lo.w, g_hi.x, g_hi.y, g_hi.z, g_hi.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) g[k] = __uint_as_float(w[k]);
      } else {
        unpack8_16(g_lo, gamma_type == kF16, g);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        g[k] = (col0 + k < C) ? load_elem(a.gamma, col0 + k, gamma_type) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] += a.weight_offset;

    // phase 2: normalise, re-encode, store
#pragma unroll
    for (int it = 0; it < kMaxIter; ++it) {
      if (base + it >= nit) break;
      const uint32_t h = (base + it) * HPI + hl;
      const bool lane_valid = valid[it];
      char* p = krow + EB * (int64_t)h * cv.head_stride;
      const float r = PER_HEAD ? rh[it] : r_token;
      float v[8];
      widen(it, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (col0 + k >= C) continue;
        if constexpr (MBC) {
          v[k] = v[k] * g[k] * r;
        } else {
          v[k] = round_bf16(v[k] * r) * g[k];
        }
      }
      if constexpr (KM == KMode::Bf16) {
        if (lane_valid) {
          if (col0 + 8 <= C) {
            store16_stream(p, pack8_bf16(v));
          } else {
            uint16_t* e = reinterpret_cast<uint16_t*>(p);
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (col0 + k < C) e[k] = (uint16_t)(pack_bf16x2(v[k], 0.0f) & 0xffffu);
          }
        }
      } else {
        float inv = tensor_inv;
        if constexpr (KM == KMode::Fp8PerToken) {
          float am = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(v[k]));
          am = group_max_abs<LP>(am);
          const float st = am / 448.0f;
          inv = st > 0.0f ? rcp_hw(st) : 0.0f;
          if (lane_valid && m == 0) a.k_scales[slot_head0 + h] = st;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] *= inv;
        const uint2 codes = pack8_fp8(v);
        if (lane_valid) {
          if (kWholeHead || col0 + 8 <= C) {
            store8_stream(p, codes);
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
  }  // chunk
}

template <int D, KMode KM, bool PER_HEAD, bool PLANNED, bool GT>
hipError_t launch_dkhpg(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  if (mbc)
    hipLaunchKernelGGL((kv_norm_kernel<D, true, KM, PER_HEAD, PLANNED, GT>), dim3(blocks),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((kv_norm_kernel<D, false, KM, PER_HEAD, PLANNED, GT>), dim3(blocks),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

// A bf16 gamma takes the kernels without the type branch (measured 17.9
// against 18.4 us on the Llama-shaped batch).
template <int D, KMode KM, bool PER_HEAD, bool PLANNED>
hipError_t launch_dkhp(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  return a.gamma_type == kBf16 ? launch_dkhpg<D, KM, PER_HEAD, PLANNED, false>(a, mbc, blocks, stream)
                               : launch_dkhpg<D, KM, PER_HEAD, PLANNED, true>(a, mbc, blocks, stream);
}

template <int D, KMode KM, bool PER_HEAD>
hipError_t launch_dkh(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  return a.plan != nullptr ? launch_dkhp<D, KM, PER_HEAD, true>(a, mbc, blocks, stream)
                           : launch_dkhp<D, KM, PER_HEAD, false>(a, mbc, blocks, stream);
}

template <int D, KMode KM>
hipError_t launch_dk(const KvNormArgs& a, bool mbc, uint32_t blocks, hipStream_t stream) {
  return a.per_head ? launch_dkh<D, KM, true>(a, mbc, blocks, stream)
                    : launch_dkh<D, KM, false>(a, mbc, blocks, stream);
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
    case 80: return launch_d<80>(a, multiply_before_cast, kmode, nb, stream);
    case 96: return launch_d<96>(a, multiply_before_cast, kmode, nb, stream);
    case 128: return launch_d<128>(a, multiply_before_cast, kmode, nb, stream);
    case 256: return launch_d<256>(a, multiply_before_cast, kmode, nb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
