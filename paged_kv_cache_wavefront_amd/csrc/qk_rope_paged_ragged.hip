// qk_rope_paged_ragged.hip -- paged-ragged fused Q/K RoPE for gfx950.
//
// What it computes (page "generic_fused_qk_rope_bshd_paged_ragged", summary,
// Parameters, Args): RoPE of every Q head into the output tensor and, in the
// same launch, RoPE in place of the new tokens' K rows in the paged cache of
// layer layer_idx (one launch, so the K rotation is ordered after whatever
// wrote K).  Position = position_ids[t] when given, else the token's slot.
// Optional per-head RMSNorm of K (first k_norm_cols columns, gamma) runs
// before the rotation, with a single rounding at the end (bf16, or fp8 for
// an fp8 K cache).
//
// Waves: one wave64 per (token, chunk of kQInstrPerWave x 64/LP Q heads);
// the chunk-0 wave of a token also rotates the token's K heads.  Lane
// geometry (D = head_dim): each lane owns one 16-byte chunk (8 values) of a
// head; a head occupies a group of LP lanes, LP = D/8 rounded up to a power
// of two, so for D = 64, 128, 256 every Q instruction moves 64 x 16
// contiguous bytes, and for D = 80, 96 (10 or 12 chunks in a 16-lane group)
// the idle lanes of each group neither load nor store.  An fp8 K head is read
// as 8 codes per lane (8 bytes), decoded in registers, rotated, scaled (the
// head's scale applies to both members of every pair, so it commutes with the
// rotation), and re-encoded with the tensor scale or with a fresh per-(slot,
// head) scale max|y| / 448 from a DPP max over the head's lanes.
// * interleaved: lane k holds values 8k..8k+7 = adjacent pairs 4k..4k+3.
// * rotate-half (H = D/16 chunks per half): lane k < H holds values 8k.. of
//   the first half; lane LP-1-k holds the second-half values of the same
//   pairs 8k..8k+7, so the partner of lane k is lane LP-1-k, reached by one
//   DPP mirror per dword (a ds_swizzle for D = 256, whose heads span 32
//   lanes).
// Pair i needs freqs columns 2i, 2i+1: 8 or 16 consecutive values per lane
// (fp32, or bf16 / fp16 widened exactly), loaded once per token.  Q (bf16 or
// fp16, a template parameter; the output takes q's type) is read, and Q and K
// are written, with non-temporal accesses.
//
// Multimodal RoPE: three position rows; pair i uses the row of its section
// (temporal / height / width pair ranges), cos/sin fetched per pair.
//
// Optional K norm: r = 1/sqrt(mean(x^2) + eps) over the first C columns of a
// head (DPP sum over the head's lanes).  Normalised values enter the rotation
// as x * gamma (exact in fp32) and r is applied after it, so an fp32 rounding
// of x * r * gamma cannot be amplified by cancellation in the rotation; a
// pair with one normalised and one plain member takes r before the rotation.
// An fp8 head enters the rotation as its codes (times gamma), and its scale
// joins r after the rotation for the same reason.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;
// 16-byte Q loads per lane per wave.  Measured with rotating buffers on the
// Llama-shaped batch (19141 tokens, 32 Q heads of 128, fused K norm): 2 per
// wave 67.5 us, 4 per wave 64.4 us, 8 per wave 67.4 us; handing the K heads
// to all of a token's waves instead of the first one alone: 65.3 us.
constexpr int kQInstrPerWave = 4;

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

// A head of D values is D/8 chunks of 8; it occupies a group of LP lanes,
// LP = D/8 rounded up to a power of two so that the DPP / swizzle mirror and
// the group reductions work inside the group (D = 80 and 96 leave 6 and 4
// lanes of each 16-lane group idle).
template <int D, bool INTER>
struct Geometry {
  static constexpr int kChunks = D / 8;
  static constexpr int kLanesPerHead = pow2_at_least(kChunks);
  static constexpr bool kPadded = kLanesPerHead != kChunks;
  static constexpr int kHeadsPerInstr = kWave / kLanesPerHead;
  static constexpr int kCs = INTER ? 8 : 16;  // cos/sin floats per lane
};

// Rotate-half: the first HALF lanes of a group hold the first-half chunks in
// order, the last HALF lanes hold the second-half chunks mirrored, so the
// partner of lane k is lane LP-1-k; lanes in between (padded groups) idle.
// Interleaved: lane k holds chunk k; lanes past the last chunk idle.
template <int D, bool INTER>
struct LaneRole {
  int k;            // lane within the head group
  bool active;      // holds a chunk of the head
  bool first;       // rotate-half: holds first-half values
  int chunk;        // 16-byte chunk of the head row it loads / stores
  int partner_chunk;
  int cs_base;      // first freqs column it needs
  __device__ __forceinline__ explicit LaneRole(int lane) {
    constexpr int LP = Geometry<D, INTER>::kLanesPerHead;
    constexpr int NC = Geometry<D, INTER>::kChunks, HALF = NC / 2;
    k = lane % LP;
    if constexpr (INTER) {
      active = k < NC;
      first = true;
      chunk = partner_chunk = active ? k : 0;
      cs_base = 8 * chunk;
    } else {
      first = k < HALF;
      active = first || k >= LP - HALF;
      const int pb = first ? k : (active ? LP - 1 - k : 0);  // pairs 8pb..8pb+7
      chunk = first ? k : HALF + pb;
      partner_chunk = first ? HALF + k : pb;
      cs_base = 16 * pb;
    }
  }
};

// Plain rotation of one lane's values (Q, and K without a norm).  cs holds
// (cos, sin) per pair; for rotate-half the sines are pre-negated on
// first-half lanes, so every output is own*cos + other*sin.
template <bool INTER>
__device__ __forceinline__ void rotate_plain(float (&own)[8], const float (&par)[8],
                                             const float* cs) {
  if constexpr (INTER) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = own[2 * q], b = own[2 * q + 1], c = cs[2 * q], s = cs[2 * q + 1];
      own[2 * q] = sum_of_products(a, c, -b, s);
      own[2 * q + 1] = sum_of_products(b, c, a, s);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) own[j] = sum_of_products(own[j], cs[2 * j], par[j], cs[2 * j + 1]);
  }
}

// Rotation with per-value scalings (K with a norm): inputs scaled by pre_own /
// pre_par before, outputs by post after.
template <bool INTER>
__device__ __forceinline__ void rotate_scaled(float (&own)[8], const float (&par)[8],
                                              const float* cs, const float (&pre_own)[8],
                                              const float (&pre_par)[8], const float (&post)[8]) {
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
    for (int j = 0; j < 8; ++j)
      own[j] = sum_of_products(own[j] * pre_own[j], cs[2 * j], par[j] * pre_par[j],
                               cs[2 * j + 1]) * post[j];
  }
}

// Q of one wave: NI instructions of HPI heads.  Base and step are wave-uniform
// byte addresses; lane_off is the lane's byte offset.  GUARD masks heads past
// num_heads.  QF16: q and its output are fp16, else bf16.
// 16 bytes of zeros: what a lane that holds no Q value loads instead.
__device__ uint4 kZero16 = {0u, 0u, 0u, 0u};

// Q loads of one item: NI instructions of HPI heads each, issued before the
// address chain resolves (their addresses need only the token).  A lane of
// a head past num_heads, or a padding lane, loads kZero16 instead: every
// path issues the same loads, so the chain's waits can leave them in flight.
template <int D, bool INTER, int NI>
__device__ __forceinline__ void q_load(uint4 (&v)[NI], const char* src, int64_t in_step,
                                       uint32_t in_off, uint32_t h_lane, uint32_t num_heads,
                                       bool active) {
  using Geo = Geometry<D, INTER>;
  constexpr int HPI = Geo::kHeadsPerInstr;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bool ok = h_lane + HPI * i < num_heads && (!Geo::kPadded || active);
    v[i] = load16_stream(ok ? src + i * in_step + in_off
                            : reinterpret_cast<const char*>(&kZero16));
  }
}

// Rotate the loaded Q values and store them (GUARD: heads past num_heads
// are not stored).
template <int D, bool INTER, int NI, bool GUARD, bool QF16>
__device__ __forceinline__ void q_rope(const uint4 (&v)[NI], char* dst, int64_t out_step,
                                       uint32_t out_off, uint32_t h_lane, uint32_t num_heads,
                                       bool active, const float* cs) {
  using Geo = Geometry<D, INTER>;
  constexpr int HPI = Geo::kHeadsPerInstr, LP = Geo::kLanesPerHead;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float own[8], par[8] = {};
    unpack8_16(v[i], QF16, own);
    if constexpr (!INTER) unpack8_16(mirror16<LP>(v[i]), QF16, par);
    rotate_plain<INTER>(own, par, cs);
    if (GUARD && h_lane + HPI * i >= num_heads) continue;
    if (Geo::kPadded && !active) continue;
    store16_stream(dst + i * out_step + out_off, QF16 ? pack8_f16(own) : pack8_bf16(own));
  }
}

// One wave per (token, chunk of Q heads); chunk 0 also rotates (and
// optionally normalises) the token's K heads.
template <int D, bool INTER, int NI, KMode KM, bool QF16>
__global__ __launch_bounds__(256) void qk_rope_kernel(const QkArgs a) {
  using Geo = Geometry<D, INTER>;
  constexpr int LP = Geo::kLanesPerHead, HPI = Geo::kHeadsPerInstr;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
  const uint32_t t = uniform(udiv_uniform(wave, a.chunks));
  const uint32_t chunk = wave - t * a.chunks;
  if (t >= a.total_tokens) return;
  const LaneRole<D, INTER> role(lane);
  const uint32_t hl = (uint32_t)(lane / LP);
  const int col = 8 * role.chunk;          // first column this lane owns
  const int pcol = 8 * role.partner_chunk;  // first column of the partner's values

  // ---- loads that need only t: the request lookup's first step, then Q ------
  // (in that order: the load counter is in order, so the lookup can be
  // resolved while the Q loads are still in flight)
  const CacheView& cv = a.cache;
  SlotLoads sl;
  slot_issue(a.offsets, a.batch, cv.cache_lengths, lane, sl);
  const uint32_t h0 = chunk * (HPI * NI);
  const uint32_t h_lane = h0 + hl;
  const bool all_heads = h0 + HPI * NI <= a.num_q_heads;
  const char* qsrc = reinterpret_cast<const char*>(a.q_in + (int64_t)t * a.qi_tok +
                                                    (int64_t)h0 * a.qi_head);
  char* qdst = reinterpret_cast<char*>(a.q_out + (int64_t)t * a.qo_tok + (int64_t)h0 * a.qo_head);
  const uint32_t qi_off = 2 * (hl * (uint32_t)a.qi_head + (uint32_t)col);
  const uint32_t qo_off = 2 * (hl * (uint32_t)a.qo_head + (uint32_t)col);
  const int64_t qi_step = 2 * HPI * a.qi_head, qo_step = 2 * HPI * a.qo_head;
  uint4 qv[NI];
  q_load<D, INTER, NI>(qv, qsrc, qi_step, qi_off, h_lane, a.num_q_heads, role.active);

  // ---- address chain: step 1 = {position id(s), offsets, prior lengths};
  //      step 2 = {freqs row(s), page-table entry} ----------------------------------
  uint32_t pid[3] = {0, 0, 0};
  if (a.position_ids != nullptr) {
    pid[0] = uniform(a.position_ids[t]);
    if (a.mrope) {
      pid[1] = uniform(a.position_ids[(uint64_t)a.total_tokens + t]);
      pid[2] = uniform(a.position_ids[2 * (uint64_t)a.total_tokens + t]);
    }
  }
  const TokenSlot ts = slot_resolve(sl, a.offsets, a.batch, cv.cache_lengths, t, lane);
  const uint32_t pos = a.position_ids != nullptr ? pid[0] : ts.slot;
  bool pos_ok = ts.ok && pos < a.max_seq_len;
  if (a.mrope) pos_ok = pos_ok && pid[1] < a.max_seq_len && pid[2] < a.max_seq_len;
  float cs[Geo::kCs];
  const bool f32 = a.freq_type == kF32, f16 = a.freq_type == kF16;
  const int64_t feb = f32 ? 4 : 2;  // freqs element bytes
  const char* freqs = static_cast<const char*>(a.freqs);
  if (pos_ok && !a.mrope) {
    load_typed<Geo::kCs>(freqs + feb * ((int64_t)pos * D + role.cs_base), a.freq_type, cs);
  } else if (pos_ok) {
    // multimodal RoPE: pair i takes cos/sin from the row of its section
#pragma unroll
    for (int j = 0; j < Geo::kCs / 2; ++j) {
      const uint32_t i = (uint32_t)role.cs_base / 2 + j;
      const uint32_t p = i < a.mrope_end0 ? pid[0] : (i < a.mrope_end1 ? pid[1] : pid[2]);
      const char* e = freqs + feb * ((int64_t)p * D + 2 * i);
      if (f32) {
        const float2 v = *reinterpret_cast<const float2*>(e);
        cs[2 * j] = v.x;
        cs[2 * j + 1] = v.y;
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(e);
        cs[2 * j] = half_of(w, 0, f16);
        cs[2 * j + 1] = half_of(w, 1, f16);
      }
    }
  }
  PageSlot ps{};
  if (!(pos_ok && page_of(cv.page_table, cv.pt_stride, cv.num_pages, cv.page_size, ts, &ps))) {
    if (chunk == 0) count_skip(cv.error_count, lane);
    return;
  }
  if constexpr (!INTER) {
    if (role.first) {
#pragma unroll
      for (int j = 0; j < 8; ++j) cs[2 * j + 1] = -cs[2 * j + 1];
    }
  }

  // ---- Q ------------------------------------------------------------------------
  if (all_heads)
    q_rope<D, INTER, NI, false, QF16>(qv, qdst, qo_step, qo_off, h_lane, a.num_q_heads,
                                      role.active, cs);
  else if (h0 < a.num_q_heads)
    q_rope<D, INTER, NI, true, QF16>(qv, qdst, qo_step, qo_off, h_lane, a.num_q_heads,
                                     role.active, cs);
  if (chunk != 0) return;

  // ---- K (in place), optional per-head RMSNorm first ------------------------
  // bf16: 16 bytes per lane; fp8: 8 bytes per lane, decoded to the codes'
  // exact values.  Both members of a rotation pair belong to one head and so
  // share its scale (and its r), so the rotation runs on code x gamma (exact
  // in fp32: 4- and 8-bit significands) and scale x r is applied once after
  // it; a per-tensor cache re-encodes with its scale, a per-token cache
  // stores a fresh max|y| / 448 per head.
  constexpr int64_t EB = KM == KMode::Bf16 ? 2 : 1;
  const bool knorm = a.k_gamma != nullptr;
  const int C = (int)a.k_norm_cols;
  float g[8], gp[8];  // gamma of this lane's columns and of the partner's
  load_gamma8(a.k_gamma, col, C, knorm, g);
  load_gamma8(a.k_gamma, pcol, C, knorm && !INTER, gp);
  char* krow = static_cast<char*>(cv.layer_base) +
               EB * ((int64_t)ps.page * cv.page_stride + (int64_t)ps.offset * cv.slot_stride);
  const uint32_t k_off = (uint32_t)EB * (hl * (uint32_t)cv.head_stride + (uint32_t)col);
  const int64_t slot_head0 = ((int64_t)ps.page * cv.page_size + ps.offset) * cv.num_heads;
  float tensor_inv = 1.0f;
  if constexpr (KM == KMode::Fp8PerTensor) tensor_inv = rcp_hw(a.k_scales[0]);
  for (uint32_t hbase = 0; hbase < cv.num_heads; hbase += HPI) {
    const uint32_t h = hbase + hl;
    const bool valid = h < cv.num_heads && (!Geo::kPadded || role.active);
    char* p = krow + EB * (int64_t)hbase * cv.head_stride + k_off;
    float own[8], par[8] = {};
    float ks = 1.0f;  // the head's dequantisation scale (fp8)
    if constexpr (KM == KMode::Bf16) {
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (valid) kv = load16(p);
      unpack8(kv, own);
      if constexpr (!INTER) unpack8(mirror16<LP>(kv), par);
    } else {
      uint2 kv = make_uint2(0, 0);
      ks = 0.0f;
      if (valid) {
        kv = *reinterpret_cast<const uint2*>(p);
        ks = KM == KMode::Fp8PerTensor ? a.k_scales[0] : a.k_scales[slot_head0 + h];
      }
      unpack8_fp8(kv.x, kv.y, own);
      if constexpr (!INTER) unpack8_fp8(mirror_u32<LP>(kv.x), mirror_u32<LP>(kv.y), par);
    }
    if (!knorm) {
      rotate_plain<INTER>(own, par, cs);
      if constexpr (KM != KMode::Bf16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) own[j] *= ks;
      }
    } else {
      // statistic of the head's values x = code x scale (bf16: scale 1):
      // mean(x^2) = scale^2 mean(code^2)
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (col + j < C) ss = fmaf(own[j], own[j], ss);
      ss = group_sum<LP>(ss);
      if constexpr (KM != KMode::Bf16) ss = (ss * ks) * ks;
      const float r = rsqrt_hw(ss * a.inv_norm_cols + a.epsilon);
      const float kr = ks * r;
      float pre_own[8], pre_par[8], post[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        own[j] *= g[j];  // exact: bf16 x bf16 or code x bf16; g = 1 past C
        par[j] *= gp[j];
        // is this value / its pair partner inside the normalised span?  A
        // pair with both members inside takes scale x r after the rotation,
        // a pair with one member inside takes r on that member before it.
        const bool in_me = col + j < C;
        const bool in_other = INTER ? (col + (j ^ 1) < C) : (pcol + j < C);
        pre_own[j] = (in_me && !in_other) ? r : 1.0f;
        pre_par[j] = (in_other && !in_me) ? r : 1.0f;
        post[j] = (in_me && in_other) ? kr : ks;
      }
      rotate_scaled<INTER>(own, par, cs, pre_own, pre_par, post);
    }
    if constexpr (KM == KMode::Bf16) {
      if (valid) store16_stream(p, pack8_bf16(own));
    } else {
      float inv = tensor_inv;
      if constexpr (KM == KMode::Fp8PerToken) {
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(own[j]));
        am = group_max_abs<LP>(am);
        const float st = am / 448.0f;
        inv = st > 0.0f ? rcp_hw(st) : 0.0f;
        if (valid && role.k == 0) a.k_scales[slot_head0 + h] = st;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) own[j] *= inv;
      if (valid) store8_stream(p, pack8_fp8(own));
    }
  }
}

template <int D, bool INTER, KMode KM>
hipError_t launch_one(const QkArgs& a, bool q_f16, uint32_t blocks, hipStream_t stream) {
  if (q_f16)
    hipLaunchKernelGGL((qk_rope_kernel<D, INTER, kQInstrPerWave, KM, true>), dim3(blocks),
                       dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((qk_rope_kernel<D, INTER, kQInstrPerWave, KM, false>), dim3(blocks),
                       dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool INTER>
hipError_t launch_k(const QkArgs& a, bool q_f16, KMode km, uint32_t blocks, hipStream_t stream) {
  switch (km) {
    case KMode::Bf16: return launch_one<D, INTER, KMode::Bf16>(a, q_f16, blocks, stream);
    case KMode::Fp8PerTensor:
      return launch_one<D, INTER, KMode::Fp8PerTensor>(a, q_f16, blocks, stream);
    case KMode::Fp8PerToken:
      return launch_one<D, INTER, KMode::Fp8PerToken>(a, q_f16, blocks, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const QkArgs& a, bool interleaved, bool q_f16, KMode km, uint32_t blocks,
                    hipStream_t stream) {
  return interleaved ? launch_k<D, true>(a, q_f16, km, blocks, stream)
                     : launch_k<D, false>(a, q_f16, km, blocks, stream);
}

}  // namespace

// Q heads per wave: kQInstrPerWave instructions of 64 / LP heads (LP = lanes
// per head group), i.e. 4 KiB of Q per wave for head_dim 64, 128 and 256 (32,
// 16 and 8 heads), 16 heads of 80 or 96.
uint32_t qk_heads_per_wave(int head_dim) {
  return (uint32_t)kQInstrPerWave * (uint32_t)(kWave / pow2_at_least(head_dim / 8));
}

hipError_t launch_qk_rope(const QkArgs& a, int head_dim, bool interleaved, bool q_f16,
                          KMode kmode, hipStream_t stream) {
  const uint64_t waves = (uint64_t)a.total_tokens * a.chunks;
  const uint64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  // the kernel numbers waves (block * waves per block + wave) in 32 bits
  if (blocks * kWavesPerBlock > 0xffffffffull) return hipErrorInvalidValue;
  const uint32_t nb = (uint32_t)blocks;
  switch (head_dim) {
    case 64: return launch_d<64>(a, interleaved, q_f16, kmode, nb, stream);
    case 80: return launch_d<80>(a, interleaved, q_f16, kmode, nb, stream);
    case 96: return launch_d<96>(a, interleaved, q_f16, kmode, nb, stream);
    case 128: return launch_d<128>(a, interleaved, q_f16, kmode, nb, stream);
    case 256: return launch_d<256>(a, interleaved, q_f16, kmode, nb, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
