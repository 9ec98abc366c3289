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
// * One wave64 per (token, chunk of heads) work item.  Each wave instruction
//   moves 1 KiB of contiguous q: a head's rope slice of R values is R/8
//   16-byte chunks held by a group of LP = R/8 lanes (LP = 4, 8, 16 for
//   rope_dim 32, 64, 128), 64/LP heads per instruction.  Within a group,
//   lane k < LP/2 holds values 8k..8k+7 (first half) and lane LP-1-k holds
//   the second-half values of the same pairs, so the rotate-half partner of
//   lane k is lane LP-1-k and arrives with one DPP mirror per dword (quad,
//   half-row or row mirror): no LDS round trip, and every load and store
//   covers full 128-byte lines.
// * q and latent are read and q_rope_output written with non-temporal
//   accesses (streamed once).  The address chain takes two dependent steps
//   ({offsets, cache lengths}, then {freqs row, page-table entry}) and hides
//   behind the bulk traffic: with 32 heads per wave the chunk-0 wave issues
//   its latent row and the chain's first step ahead of its q loads and
//   resolves the chain while q is in flight; with at most 16 heads per wave,
//   or a plan entry, the q loads are issued first (chain_first below).
// * The 16 cos/sin values a lane needs sit contiguously in the freqs row and
//   are the same for every head: one 64-byte load per lane per token (32
//   bytes for a 16-bit table), kept in registers.
// * The head-chunk-0 wave of a token also owns its latent row: lane l holds
//   non-rope values 8l..8l+7 (lanes below kv_norm_dim / 8) and rope-tail
//   value l (and l + 64 for rope_dim 128): one tail value per lane instead
//   of eight on a few lanes, since every lane of a wave pays for every
//   instruction.  A tail pair's partner comes from lane l +- R/2 (a
//   cross-lane permute; in the same lane for rope_dim 128), and its cos/sin
//   with one 8-byte load from the freqs row.  The sum of squares (and the
//   per-token amax) reduce across the wave with DPP inside rows and readlane
//   across rows; the sum of squares is reduced while the second step of the
//   address chain is in flight.  The non-rope value is formed as
//   (x * gamma) * (r / scale): x * gamma is exact in fp32 for a bf16 or fp16
//   gamma (8 + 8 or 8 + 11 significant bits).  The row is converted to fp8 in registers (clamp to
//   +-448, then hardware round-to-nearest-even) and written with 8-byte
//   non-temporal stores.
// * Element types ("mla_fused_rope_rmsnorm_quantization", Parameters: dtype,
//   out_rope_dtype, freq_dtype, gamma_dtype): q in bf16 or fp16 and
//   q_rope_output in bf16, fp16 or fp32 are a template pair (QIO); freqs_cis
//   and gamma in fp32, bf16 or fp16 widen exactly to fp32 behind uniform
//   branches that only the GT instances carry, so that the default fp32 freqs
//   and bf16 gamma run without them.
// * Planned form: with a token plan (token_plan.hip) each wave reads its
//   token's (page, offset, position, placed) entry with one scalar 16-byte
//   load instead of the two-step chain; the entry is checked against the
//   pool and the freqs table like the chain's results.
// * In-place form ("mla_graph" module page: fused_rope_rmsnorm_kernel, and the
//   first two steps of the fp8 prefill and decode branches, which apply RoPE
//   and RMSNorm to the key cache in place): the latent row is not in a buffer
//   but already sits in a bf16 cache at the token's slot; the chunk-0 wave
//   reads it from there once the page lookup has resolved, issued before the
//   q rotation so that its latency overlaps the q stores, and writes the
//   normalised, rotated row back over it.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxNope = 512;  // kv_norm_dim: at most one 16-byte chunk per lane

// Lane roles inside the LP-lane group of one head (rotate-half, rope_dim R).
template <int R>
struct HeadLane {
  static constexpr int LP = R / 8;  // lanes per head
  int k;          // lane within the group
  bool first;     // holds first-half values
  int pair_block; // holds pairs 8*pair_block .. 8*pair_block+7
  int chunk;      // 16-byte chunk of the head's rope slice it loads/stores
  __device__ __forceinline__ explicit HeadLane(int lane) {
    k = lane % LP;
    first = k < LP / 2;
    pair_block = first ? k : LP - 1 - k;
    chunk = first ? k : LP / 2 + pair_block;
  }
};

// The latent row's rope tail, one value per lane (two for rope_dim 128): lane
// l holds tail value l (rope_dim 32: lanes 0..31 only) and, for rope_dim 128,
// value l + 64 in the upper half of its word.  Value i belongs to pair
// i mod R/2; for rope_dim 32 and 64 the pair's other member sits in lane
// l ^ R/2, for 128 in the same lane.
template <int R>
struct TailLane {
  bool active;  // holds tail values
  int pair;     // rotation pair of its (first) value
  bool first;   // its (first) value is the pair's first member
  __device__ __forceinline__ explicit TailLane(int lane) {
    active = R == 128 || lane < R;
    pair = R == 128 ? lane : lane % (R / 2);
    first = R == 128 || lane % R < R / 2;
  }
};

__device__ __forceinline__ uint32_t load2_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(p);
}

// The lane's tail values as loaded: value l in lo, and for rope_dim 128 value
// l + 64 in hi (joined into one word only where they are used).
template <int R>
__device__ __forceinline__ void load_tail(const uint16_t* tail_row, int lane, uint32_t& lo,
                                          uint32_t& hi) {
  if constexpr (R == 128) {
    lo = load2_stream(tail_row + lane);
    hi = load2_stream(tail_row + 64 + lane);
  } else {
    lo = lane < R ? load2_stream(tail_row + lane) : 0u;
  }
}

// Rotated tail values of this lane (tv[1] only for rope_dim 128); tcs is the
// (cos, sin) of the lane's pair.
template <int R>
__device__ __forceinline__ void rotate_tail(uint32_t raw, const float2& tcs,
                                            const TailLane<R>& tl, float (&tv)[2]) {
  const float own = bf16_lo(raw);
  if constexpr (R == 128) {
    const float hi = bf16_hi(raw);
    tv[0] = sum_of_products(own, tcs.x, hi, -tcs.y);
    tv[1] = sum_of_products(hi, tcs.x, own, tcs.y);
  } else {
    const float par = R == 64 ? __uint_as_float(swap_halves_u32(__float_as_uint(own), tl.first))
                              : swizzle<kSwizzleXor16>(own);
    tv[0] = sum_of_products(own, tcs.x, par, tl.first ? -tcs.y : tcs.y);
    tv[1] = 0.0f;
  }
}

// q input / output element types of a QIO pair.
template <QIO X>
struct QTypes {
  static constexpr bool kInF16 = X == QIO::H_H || X == QIO::H_B || X == QIO::H_F;
  static constexpr int kOut = (X == QIO::B_F || X == QIO::H_F) ? kF32
                              : (X == QIO::B_H || X == QIO::H_H) ? kF16 : kBf16;
  static constexpr int64_t kOutBytes = kOut == kF32 ? 4 : 2;
};

// One rotated value: x c + p s for the value x of this lane and the value p
// of the mirrored lane of its LP-lane group (the pair partner); first-half
// lanes pass the sine negated (out = x cos - p sin), second-half lanes as is
// (out = x cos + p sin).  Kahan's algorithm with the rounding error of x c
// recovered (the same bound as recovering that of p s): p is needed once, in
// the fused multiply-add, so it arrives by one DPP mirror of the unpacked
// value and the partner needs no unpacking of its own.  An infinite x c has
// no error to recover: its error term is clamped as in sum_of_products.
template <int LP>
__device__ __forceinline__ float rotate_with_mirror(float x, float c, float s) {
  const float xc = x * c;
  const float xc_err = fminf(fmaf(x, c, -xc), 3.402823466e38f);  // x*c - xc, exact
  const float p = __uint_as_float(mirror_u32<LP>(__float_as_uint(x)));
  return fmaf(p, s, xc) + xc_err;
}

// 16 bytes of zeros: what a lane of a head past num_heads loads instead of q
// (with no heads at all, q may be a null pointer).
__device__ uint4 kZero16 = {0u, 0u, 0u, 0u};

// q loads / stores of one item: NI instructions of 64/LP heads each.  The
// token and chunk parts of the address are wave-uniform (scalar registers);
// each lane adds a 32-bit offset.  A lane of a head past num_heads (last
// chunk of a token) loads kZero16 instead, and its result is not stored
// (GUARD on the stores).  So the loads take one straight path, the same NI
// loads for every item, with no zero written ahead of a load (such a write
// waits for the loads in flight, and paths with different load counts make
// later waits conservative).  (base and step in bytes, wave-uniform;
// lane_off in bytes, per lane.)
template <int NI, int HPI>
__device__ __forceinline__ void load_q(uint4 (&q)[NI], const char* base, int64_t step,
                                       uint32_t lane_off, uint32_t h_lane, uint32_t num_heads) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bool ok = h_lane + HPI * i < num_heads;
    q[i] = load16_stream(ok ? base + i * step + lane_off
                            : reinterpret_cast<const char*>(&kZero16));
  }
}

// Rotate and store: bf16 or fp16 output (16 bytes per lane) or fp32 output
// (32 bytes per lane: two 16-byte stores).
template <int NI, int HPI, int LP, bool GUARD, QIO X>
__device__ __forceinline__ void rotate_store_q(const uint4 (&q)[NI], const float (&cs)[16],
                                               char* base, int64_t step, uint32_t lane_off,
                                               uint32_t h_lane, uint32_t num_heads) {
  using QT = QTypes<X>;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float in[8], own[8];
    unpack8_16(q[i], QT::kInF16, in);
#pragma unroll
    for (int j = 0; j < 8; ++j) own[j] = rotate_with_mirror<LP>(in[j], cs[2 * j], cs[2 * j + 1]);
    if (GUARD && h_lane + HPI * i >= num_heads) continue;
    char* p = base + i * step + lane_off;
    if constexpr (QT::kOut == kF16) {
      store16_stream(p, pack8_f16(own));
    } else if constexpr (QT::kOut == kF32) {
      store16_stream(p, make_uint4(__float_as_uint(own[0]), __float_as_uint(own[1]),
                            __float_as_uint(own[2]), __float_as_uint(own[3])));
      store16_stream(p + 16, make_uint4(__float_as_uint(own[4]), __float_as_uint(own[5]),
                                 __float_as_uint(own[6]), __float_as_uint(own[7])));
    } else {
      store16_stream(p, pack8_bf16(own));
    }
  }
}

// The 8 gamma values of a lane (values 8l..8l+7), raw: two 16-byte chunks of
// fp32, or one of a 16-bit type (loaded twice: the loads do not depend on
// the type, so that no wait for them sits under a branch).
struct Gamma8 {
  uint4 lo, hi;
};

__device__ __forceinline__ Gamma8 load_gamma8(const void* gamma, int type, int lane) {
  const bool f32 = type == kF32;
  const uint4* p = static_cast<const uint4*>(gamma) + (f32 ? 2 * lane : lane);
  return Gamma8{load16(p), load16(p + (f32 ? 1 : 0))};
}

// RMSNorm statistic of the latent row's non-rope part (lane l holds values
// 8l..8l+7; lanes past kv_norm_dim / 8 hold zeros): returns
// r = 1/sqrt(mean(x^2) + eps), wave-uniform, and leaves x * gamma in xg
// (exact in fp32 for a bf16 or fp16 gamma: 8 + 8 or 8 + 11 significant bits;
// one rounding for an fp32 gamma).
__device__ __forceinline__ float latent_rms(const uint4& xn, const Gamma8& gm, int gamma_type,
                                            float (&xg)[8], float inv_dn, float epsilon) {
  float g8[8];
  unpack8(xn, xg);
  if (gamma_type == kF32) {
    const uint32_t w[8] = {gm.lo.x, gm.lo.y, gm.lo.z, gm.lo.w, gm.hi.x, gm.hi.y, gm.hi.z, gm.hi.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) g8[k] = __uint_as_float(w[k]);
  } else {
    unpack8_16(gm.lo, gamma_type == kF16, g8);
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ss = fmaf(xg[k], xg[k], ss);
    xg[k] *= g8[k];
  }
  ss = wave_sum(ss);
  return rsqrt_hw(ss * inv_dn + epsilon);
}

// Issue order of an item's loads.  The load counter is in order, so a wave
// can wait for its first loads alone while later ones are still in flight.
// With 32 heads per wave and the address chain in the kernel (unplanned),
// the token's chunk-0 wave issues its latent row and the chain's first step
// before its q loads, and resolves the chain while q is still arriving
// (128-head decode batch 3.66 -> 3.50 us, 17108-token prefill 94.6 -> 94.1
// us).  With at most 16 heads per wave, and with a plan entry, the q loads go
// first and the chain is issued after them, which measured faster there
// (16-head mixed batch 11.08 against 11.3 -- 11.8 us, planned decode 3.59
// against 3.65 us).
template <int NI, bool PLANNED>
constexpr bool chain_first() {
  return NI == 4 && !PLANNED;
}

// The loads of one work item that need only the item's index: its q chunks,
// for a token's chunk-0 wave its latent row (buffer form), and its plan entry
// (planned form) or, chain first, the address chain's first step.
template <int NI>
struct ItemLoads {
  uint4 q[NI];
  uint4 xn;
  uint32_t tail, tail_hi;  // the rope tail as load_tail leaves it
  uint4 pe;
  SlotLoads sl;
};

template <int R, int NI, MlaOut MODE, bool PLANNED>
__device__ __forceinline__ void issue_item(const MlaArgs& a, uint32_t t, uint32_t chunk,
                                           int lane, ItemLoads<NI>& L) {
  using HL = HeadLane<R>;
  constexpr int LP = HL::LP, HPI = kWave / LP;
  const HL hl(lane);
  const auto issue_q = [&] {
    const uint32_t h0 = chunk * (HPI * NI);  // first head of this item
    const uint32_t h_lane = h0 + (uint32_t)(lane / LP);
    const char* qsrc = reinterpret_cast<const char*>(a.q_in + (int64_t)t * a.qi_tok +
                                                      (int64_t)h0 * a.qi_head);
    const uint32_t qi_lane = 2 * ((uint32_t)(lane / LP) * (uint32_t)a.qi_head + 8 * hl.chunk);
    load_q<NI, HPI>(L.q, qsrc, 2 * HPI * a.qi_head, qi_lane, h_lane, a.num_heads);
  };
  const auto issue_latent = [&] {
    L.xn = make_uint4(0, 0, 0, 0);
    L.tail = L.tail_hi = 0;
    if constexpr (MODE != MlaOut::Bf16InPlace) {
      if (chunk == 0) {
        const uint16_t* row = a.latent + (int64_t)t * a.kv_row;
        if ((uint32_t)lane < a.nope_chunks) L.xn = load16_stream(row + 8 * lane);
        load_tail<R>(row + 8 * a.nope_chunks, lane, L.tail, L.tail_hi);
      }
    }
  };
  if constexpr (chain_first<NI, PLANNED>()) {
    issue_latent();
    slot_issue(a.offsets, a.batch, a.cache.cache_lengths, lane, L.sl);
    issue_q();
  } else {
    issue_q();
    issue_latent();
    if constexpr (PLANNED) L.pe = *reinterpret_cast<const uint4*>(a.plan + 4 * (uint64_t)t);
  }
}

// Everything after the bulk loads: the address chain (or the plan entry),
// the q rotation and stores, and for the chunk-0 wave the latent row's
// normalisation, tail rotation, quantisation and paged store.
// GT: freqs and gamma of the types in a.freq_type / a.gamma_type; otherwise
// the default fp32 freqs and bf16 gamma, with no type branches.
template <int R, int NI, MlaOut MODE, QIO X, bool PLANNED, bool GT>
__device__ __forceinline__ void finish_item(const MlaArgs& a, uint32_t t, uint32_t chunk,
                                            int lane, const Gamma8& gm, ItemLoads<NI>& L) {
  using HL = HeadLane<R>;
  constexpr int LP = HL::LP, HPI = kWave / LP;
  const HL hl(lane);
  const uint32_t h0 = chunk * (HPI * NI);
  const uint32_t h_lane = h0 + (uint32_t)(lane / LP);
  const bool all_heads = h0 + HPI * NI <= a.num_heads;  // wave-uniform
  constexpr bool INPLACE = MODE == MlaOut::Bf16InPlace;
  const bool latent_wave = chunk == 0;
  const int freq_type = GT ? a.freq_type : (int)kF32;
  const int gamma_type = GT ? a.gamma_type : (int)kBf16;

  // ---- address chain -----------------------------------------------------------
  // step 1: request and slot (= position); step 2: the freqs row and the
  // page-table entry, both needing only the slot, issued together.
  // Planned: one 16-byte plan entry (page, offset, position, placed) replaces
  // both steps; the entry is checked against the pool and the freqs table
  // before anything derived from it is dereferenced.
  const CacheView& cv = a.cache;
  TokenSlot ts{};
  if constexpr (PLANNED) {
    ts.slot = uniform(L.pe.z);
    ts.ok = L.pe.w != 0;
  } else {
    if constexpr (chain_first<NI, PLANNED>())
      ts = slot_resolve(L.sl, a.offsets, a.batch, cv.cache_lengths, t, lane);
    else
      ts = find_slot(a.offsets, a.batch, cv.cache_lengths, t, lane);
  }
  const bool pos_ok = ts.ok && ts.slot < a.max_seq_len;
  // The freqs row is loaded without a branch (a skipped token reads row 0,
  // which always exists, and returns before using it), so that nothing
  // issued after the latent row has to complete before the statistic below.
  const TailLane<R> tl(lane);
  float cs[16];
  float2 tcs;
  {
    const int64_t first = (int64_t)(pos_ok ? ts.slot : 0u) * R;  // row's first element
    if constexpr (!GT) {
      const float* frow = static_cast<const float*>(a.freqs) + first;
      const float4* fr = reinterpret_cast<const float4*>(frow + 16 * hl.pair_block);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = fr[i];
        cs[4 * i] = v.x; cs[4 * i + 1] = v.y; cs[4 * i + 2] = v.z; cs[4 * i + 3] = v.w;
      }
      tcs = *reinterpret_cast<const float2*>(frow + 2 * tl.pair);
    } else {
      // Any type, with the same loads for each (a load under a branch would
      // put a wait for it in front of the latent statistic): the lane's 16
      // values are four 16-byte chunks of fp32, or two of a 16-bit type,
      // loaded twice; the tail's (cos, sin) two 4-byte words, or one.
      const bool f32 = freq_type == kF32, f16 = freq_type == kF16;
      const char* row = static_cast<const char*>(a.freqs) + (f32 ? 4 : 2) * first;
      const uint4* p = reinterpret_cast<const uint4*>(row + (f32 ? 64 : 32) * hl.pair_block);
      const uint4 r0 = p[0], r1 = p[1], r2 = p[f32 ? 2 : 0], r3 = p[f32 ? 3 : 1];
      const uint32_t* tp = reinterpret_cast<const uint32_t*>(row + (f32 ? 8 : 4) * tl.pair);
      const uint32_t t0 = tp[0], t1 = tp[f32 ? 1 : 0];
      if (f32) {
        const uint4 r[4] = {r0, r1, r2, r3};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cs[4 * i] = __uint_as_float(r[i].x); cs[4 * i + 1] = __uint_as_float(r[i].y);
          cs[4 * i + 2] = __uint_as_float(r[i].z); cs[4 * i + 3] = __uint_as_float(r[i].w);
        }
        tcs = make_float2(__uint_as_float(t0), __uint_as_float(t1));
      } else {
        float lo[8], hi[8];
        unpack8_16(r0, f16, lo);
        unpack8_16(r1, f16, hi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          cs[k] = lo[k];
          cs[8 + k] = hi[k];
        }
        tcs = make_float2(half_of(t0, 0, f16), half_of(t0, 1, f16));
      }
    }
  }
  uint32_t col = 0, page = 0;
  bool col_ok = pos_ok;
  if constexpr (!PLANNED) {
    col = pos_ok ? page_column(ts.slot, cv.page_size) : 0u;
    col_ok = pos_ok && col < cv.pt_stride;
    if (col_ok) page = cv.page_table[(uint64_t)ts.request * cv.pt_stride + col];
  }
  // Buffer form: the latent row arrived with the bulk loads, so its
  // statistic is reduced while the freqs row and the page-table entry are
  // still in flight.
  float xg[8];
  float r = 0.0f;
  if constexpr (!INPLACE) {
    if (latent_wave) r = latent_rms(L.xn, gm, gamma_type, xg, a.inv_dn, a.epsilon);
  }
  PageSlot ps{};
  bool placed;
  if constexpr (PLANNED) {
    ps.page = uniform(L.pe.x);
    ps.offset = uniform(L.pe.y);
    placed = pos_ok && ps.page < cv.num_pages && ps.offset < cv.page_size;
  } else {
    ps.page = uniform(page);
    ps.offset = ts.slot - col * cv.page_size;
    placed = col_ok && ps.page < cv.num_pages;
  }
  if (!placed) {
    if (latent_wave) count_skip(cv.error_count, lane);
    return;
  }
  const int64_t row_elems = (int64_t)ps.page * cv.page_stride + (int64_t)ps.offset * cv.slot_stride;
  if constexpr (INPLACE) {
    if (latent_wave) {
      const uint16_t* row = static_cast<const uint16_t*>(cv.layer_base) + row_elems;
      if ((uint32_t)lane < a.nope_chunks) L.xn = load16_stream(row + 8 * lane);
      load_tail<R>(row + 8 * a.nope_chunks, lane, L.tail, L.tail_hi);
    }
  }
  if (hl.first) {
#pragma unroll
    for (int j = 0; j < 8; ++j) cs[2 * j + 1] = -cs[2 * j + 1];
  }

  // ---- q: exchange with the mirrored lane, rotate, store --------------------
  constexpr int64_t QB = QTypes<X>::kOutBytes;  // bytes per q output element
  char* qdst = static_cast<char*>(a.q_out) + QB * ((int64_t)t * a.qo_tok + (int64_t)h0 * a.qo_head);
  const uint32_t qo_lane =
      (uint32_t)QB * ((uint32_t)(lane / LP) * (uint32_t)a.qo_head + 8 * hl.chunk);
  if (all_heads)
    rotate_store_q<NI, HPI, LP, false, X>(L.q, cs, qdst, HPI * QB * a.qo_head, qo_lane, h_lane,
                                             a.num_heads);
  else
    rotate_store_q<NI, HPI, LP, true, X>(L.q, cs, qdst, HPI * QB * a.qo_head, qo_lane, h_lane,
                                            a.num_heads);
  if (!latent_wave) return;

  // ---- latent row: RMSNorm (non-rope part), RoPE (tail) ---------------------
  if constexpr (INPLACE) r = latent_rms(L.xn, gm, gamma_type, xg, a.inv_dn, a.epsilon);
  float tv[2];
  // The tail words came with the bulk loads.  Left free, the compiler moves
  // their widening next to the 2-byte loads, and the wait for them then holds
  // the chunk-0 wave's address chain back until all of its q and latent loads
  // are in.  With 32 heads per wave (NI 4: a 128-head token spans 4 waves,
  // and its chunk-0 wave is the slowest), and with a plan entry (a scalar
  // load, which then arrives without waiting for the vector loads), an empty
  // asm pins the widening here, which measured faster: 128-head decode batch
  // 4.10 -> 3.80 us, 17108-token prefill 95.5 -> 94.4 us, planned 16-head
  // mixed batch 10.64 -> 10.23 us.  With at most 16 heads and the address
  // chain in the kernel (every wave owns a latent row) the compiler's early
  // wait measured faster (mixed batch 10.96 us against 11.3 us pinned), so it
  // is kept there.
  constexpr bool kPinTail = NI == 4 || PLANNED;
  uint32_t tail_word = L.tail;
  if constexpr (R == 128) {
    if constexpr (kPinTail) asm volatile("" : "+v"(tail_word), "+v"(L.tail_hi));
    tail_word |= L.tail_hi << 16;
  } else if constexpr (kPinTail) {
    asm volatile("" : "+v"(tail_word));
  }
  rotate_tail<R>(tail_word, tcs, tl, tv);  // meaningful on active tail lanes only
  const bool nope_lane = (uint32_t)lane < a.nope_chunks;
  const uint32_t tail0 = 8 * a.nope_chunks + lane;  // element of the lane's (first) tail value

  if constexpr (MODE == MlaOut::Bf16 || INPLACE) {
    uint16_t* row = static_cast<uint16_t*>(cv.layer_base) + row_elems;
#pragma unroll
    for (int k = 0; k < 8; ++k) xg[k] *= r;
    if (nope_lane) store16_stream(row + 8 * lane, pack8_bf16(xg));
    const uint32_t w = pack_bf16x2(tv[0], tv[1]);
    if (tl.active) __builtin_nontemporal_store((uint16_t)w, row + tail0);
    if (R == 128) __builtin_nontemporal_store((uint16_t)(w >> 16), row + tail0 + 64);
    return;
  } else {
    float inv;
    if constexpr (MODE == MlaOut::Fp8PerTensor) {
      inv = rcp_hw(*a.tensor_scale);
    } else {
      // max |y| over the row: the non-rope part scales monotonically by r
      // (lanes past the non-rope chunks hold zeros), so the lane's largest
      // |x * gamma| times r is its largest normalised value
      float am = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(xg[k]));
      am *= r;
      if (tl.active) am = fmaxf(am, fmaxf(fabsf(tv[0]), fabsf(tv[1])));
      am = wave_max_abs(am);
      const float st = am / 448.0f;
      inv = st > 0.0f ? rcp_hw(st) : 0.0f;
      if (lane == 0)
        a.token_scales[((int64_t)ps.page * cv.page_size + ps.offset) * cv.num_heads] = st;
    }
    const float rs = r * inv;
#pragma unroll
    for (int k = 0; k < 8; ++k) xg[k] *= rs;
    uint8_t* row = static_cast<uint8_t*>(cv.layer_base) + row_elems;
    if (nope_lane) store8_stream(row + 8 * lane, pack8_fp8(xg));
    const uint32_t codes = pack4_fp8(tv[0] * inv, tv[1] * inv, 0.0f, 0.0f);
    if (tl.active) __builtin_nontemporal_store((uint8_t)codes, row + tail0);
    if (R == 128) __builtin_nontemporal_store((uint8_t)(codes >> 8), row + tail0 + 64);
  }
}

// One work item per wave (item = token * chunks + chunk).  (A persistent
// grid -- fewer waves, each looping over items with the next item's loads
// issued before the current one is finished -- measured slower: each wave
// then resolves its items' address chains one after another.)
template <int R, int NI, MlaOut MODE, QIO X, bool PLANNED, bool GT>
__global__ __launch_bounds__(256) void mla_kernel(const MlaArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform item index: the division by the head chunks runs on the
  // scalar unit (a shift for 1, 2 or 4 chunks) instead of on every lane
  const uint32_t wave = uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
  const uint32_t t = uniform(udiv_uniform(wave, a.chunks));
  const uint32_t chunk = wave - t * a.chunks;
  if (t >= a.total_tokens) return;
  ItemLoads<NI> L;
  Gamma8 gm{make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  const auto issue_gamma = [&] {
    if (chunk == 0 && (uint32_t)lane < a.nope_chunks)
      gm = load_gamma8(a.gamma, GT ? a.gamma_type : (int)kBf16, lane);
  };
  if constexpr (chain_first<NI, PLANNED>()) {
    issue_gamma();
    issue_item<R, NI, MODE, PLANNED>(a, t, chunk, lane, L);
  } else {
    issue_item<R, NI, MODE, PLANNED>(a, t, chunk, lane, L);
    issue_gamma();
  }
  finish_item<R, NI, MODE, X, PLANNED, GT>(a, t, chunk, lane, gm, L);
}

template <int R, int NI, MlaOut MODE, QIO X, bool PLANNED, bool GT>
hipError_t launch_one(const MlaArgs& a, hipStream_t stream) {
  const uint64_t items = (uint64_t)a.total_tokens * a.chunks;
  const uint64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((mla_kernel<R, NI, MODE, X, PLANNED, GT>), dim3((uint32_t)blocks),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int R, int NI, QIO X, bool PLANNED, bool GT>
hipError_t launch_mode(const MlaArgs& a, MlaOut mode, hipStream_t stream) {
  switch (mode) {
    case MlaOut::Fp8PerTensor:
      return launch_one<R, NI, MlaOut::Fp8PerTensor, X, PLANNED, GT>(a, stream);
    case MlaOut::Fp8PerToken:
      return launch_one<R, NI, MlaOut::Fp8PerToken, X, PLANNED, GT>(a, stream);
    case MlaOut::Bf16:
      return launch_one<R, NI, MlaOut::Bf16, X, PLANNED, GT>(a, stream);
    case MlaOut::Bf16InPlace:
      return launch_one<R, NI, MlaOut::Bf16InPlace, X, PLANNED, GT>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int R, QIO X, bool PLANNED, bool GT>
hipError_t launch_ni(const MlaArgs& a, MlaOut mode, int ni, hipStream_t stream) {
  switch (ni) {
    case 2: return launch_mode<R, 2, X, PLANNED, GT>(a, mode, stream);
    case 4: return launch_mode<R, 4, X, PLANNED, GT>(a, mode, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int R, bool PLANNED, bool GT>
hipError_t launch_x(const MlaArgs& a, MlaOut mode, int ni, hipStream_t stream) {
  switch (a.qio) {
    case QIO::B_B: return launch_ni<R, QIO::B_B, PLANNED, GT>(a, mode, ni, stream);
    case QIO::B_H: return launch_ni<R, QIO::B_H, PLANNED, GT>(a, mode, ni, stream);
    case QIO::B_F: return launch_ni<R, QIO::B_F, PLANNED, GT>(a, mode, ni, stream);
    case QIO::H_H: return launch_ni<R, QIO::H_H, PLANNED, GT>(a, mode, ni, stream);
    case QIO::H_B: return launch_ni<R, QIO::H_B, PLANNED, GT>(a, mode, ni, stream);
    case QIO::H_F: return launch_ni<R, QIO::H_F, PLANNED, GT>(a, mode, ni, stream);
  }
  return hipErrorInvalidValue;
}

// Freqs and gamma of the default types (fp32, bf16) take kernels without the
// type branches: a uniform branch still costs issue slots in the latency-bound
// decode waves (measured 3.90 against 4.07 us on the 128-request decode batch).
template <int R, bool PLANNED>
hipError_t launch_gt(const MlaArgs& a, MlaOut mode, int ni, hipStream_t stream) {
  if (a.freq_type == kF32 && a.gamma_type == kBf16)
    return launch_x<R, PLANNED, false>(a, mode, ni, stream);
  return launch_x<R, PLANNED, true>(a, mode, ni, stream);
}

template <int R>
hipError_t launch_r(const MlaArgs& a, MlaOut mode, int ni, hipStream_t stream) {
  return a.plan != nullptr ? launch_gt<R, true>(a, mode, ni, stream)
                           : launch_gt<R, false>(a, mode, ni, stream);
}

}  // namespace

// Heads per wave: four 1 KiB instructions of 64 / (rope_dim / 8) heads each,
// two for head counts that fit in two (rope_dim 64: 32 heads, or 16 for at
// most 16 heads).  32 heads per wave measured best on 128-head prefill and
// decode batches: small enough to keep 8 waves per SIMD resident and to
// spread a token over 4 waves, large enough to amortise each wave's address
// chain (rotating outputs, 17108-token prefill: 16 heads per wave 104 us,
// 32 heads 97 us, 64 heads 98 us).
uint32_t mla_heads_per_wave(uint32_t heads, uint32_t rope_dim) {
  const uint32_t per_instr = kWave / (rope_dim / 8);
  return heads > 2 * per_instr ? 4 * per_instr : 2 * per_instr;
}

bool mla_rope_dim_supported(uint32_t rope_dim) {
  return rope_dim == 32 || rope_dim == 64 || rope_dim == 128;
}

bool mla_nope_dim_supported(uint32_t kv_norm_dim) {
  return kv_norm_dim > 0 && kv_norm_dim % 8 == 0 && kv_norm_dim <= kMaxNope;
}

hipError_t launch_mla(const MlaArgs& a, MlaOut mode, int heads_per_wave, hipStream_t stream) {
  const uint64_t items = (uint64_t)a.total_tokens * a.chunks;
  if (items == 0) return hipSuccess;
  // the kernel numbers waves (block * waves per block + wave) in 32 bits
  if (items + kWavesPerBlock > 0xffffffffull) return hipErrorInvalidValue;
  const int R = (int)a.rope_dim;
  const int ni = heads_per_wave / (kWave / (R / 8));
  switch (R) {
    case 32: return launch_r<32>(a, mode, ni, stream);
    case 64: return launch_r<64>(a, mode, ni, stream);
    case 128: return launch_r<128>(a, mode, ni, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
