// pkv_device.h -- device-side building blocks shared by the gfx950 kernels:
// bf16 / fp8 packing, wave64 cross-lane reductions, streaming loads and
// stores, and the ragged / paged address chain.
//
// Launch order: every kernel numbers its waves in hardware block order, so
// consecutive tokens are spread over the 8 XCDs and the whole chip streams
// through one window of addresses at a time; giving each XCD its own
// contiguous token range measured slower (more DRAM streams open at once).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// Smallest power of two >= n (n >= 1): lanes per head group for a head of n
// 16-byte chunks.
__host__ __device__ constexpr int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p *= 2;
  return p;
}

// ---- bf16 <-> fp32 ---------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack 8 bf16 (one 16-byte chunk) into fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one dword, round-to-nearest-even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// ---- fp16 (IEEE binary16) <-> fp32 -------------------------------------------
// Widening is exact; narrowing rounds to nearest even (the default mode),
// overflowing to infinity, subnormals kept.

__device__ __forceinline__ f32x2_t f16x2_to_f32(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

__device__ __forceinline__ void unpack8_f16(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t p = f16x2_to_f32(w[i]);
    f[2 * i] = p[0];
    f[2 * i + 1] = p[1];
  }
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

__device__ __forceinline__ uint4 pack8_f16(const float (&f)[8]) {
  return make_uint4(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]),
                    pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7]));
}

// Element types of q, freqs and gamma arrays (the values of pkv_dtype).
enum ElemType : int { kBf16 = 0, kF32 = 2, kF16 = 3 };

// 8 values of a 16-bit type (bf16 or fp16) from one 16-byte chunk.
__device__ __forceinline__ void unpack8_16(const uint4& v, bool f16, float (&f)[8]) {
  if (f16) unpack8_f16(v, f);
  else unpack8(v, f);
}

// Value k (0 or 1) of a dword holding two 16-bit values of either type.
__device__ __forceinline__ float half_of(uint32_t w, int k, bool f16) {
  if (f16) return f16x2_to_f32(w)[k];
  return k ? bf16_hi(w) : bf16_lo(w);
}

// Element i of an fp32 / bf16 / fp16 array, widened to fp32 (exact).
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int type) {
  if (type == kF32) return static_cast<const float*>(p)[i];
  const uint16_t b = static_cast<const uint16_t*>(p)[i];
  if (type == kF16) return (float)__builtin_bit_cast(_Float16, b);
  return __uint_as_float((uint32_t)b << 16);
}

// n consecutive values of an fp32 / bf16 / fp16 array, widened to fp32
// (n a multiple of 8; p 16-byte aligned for 16-bit types, 32-byte for fp32).
template <int N>
__device__ __forceinline__ void load_typed(const void* p, int type, float (&f)[N]) {
  static_assert(N % 8 == 0, "whole 16-byte chunks");
  if (type == kF32) {
    const float4* q = static_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 v = q[i];
      f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
    }
  } else {
    const uint4* q = static_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      float t[8];
      unpack8_16(q[i], type == kF16, t);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[8 * i + j] = t[j];
    }
  }
}

// ---- fp32 -> FP8 E4M3FN (OCP), saturating, round-to-nearest-even -----------
// Values are clamped to +-448 (the largest finite E4M3FN value; infinities
// saturate too) and then converted by v_cvt_pk_fp8_f32, which rounds to
// nearest even in the OCP format on gfx950; -0 keeps its sign.  The clamp is
// IEEE 754-2019 maximum / minimum (v_maximum3_f32, v_minimum3_f32 on gfx950),
// which pass a NaN through where fmaxf / fminf would replace it by a bound,
// so a NaN converts to the NaN code and stays visible in the cache: two
// instructions per value.

__device__ __forceinline__ float sat448(float v) {
  return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, -448.0f), 448.0f);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

// 8 fp8 codes (two dwords) -> 8 fp32 values (exact; v_cvt_pk_f32_fp8).
__device__ __forceinline__ void unpack8_fp8(uint32_t w0, uint32_t w1, float (&f)[8]) {
  const uint32_t w[2] = {w0, w1};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
    f[4 * q] = lo[0];
    f[4 * q + 1] = lo[1];
    f[4 * q + 2] = hi[0];
    f[4 * q + 3] = hi[1];
  }
}

__device__ __forceinline__ uint2 pack8_fp8(const float (&f)[8]) {
  return make_uint2(pack4_fp8(f[0], f[1], f[2], f[3]), pack4_fp8(f[4], f[5], f[6], f[7]));
}

// ---- norm factors and scale reciprocals ------------------------------------------
// 1/sqrt(x) and 1/x by the hardware approximations (v_rsq_f32, v_rcp_f32,
// within about 1 ulp).  They give the RMSNorm factor r and the reciprocal of
// an fp8 scale, which only scale values that are rounded to bf16 or fp8
// afterwards: an fp32 ulp moves such a result only at a near-tie, inside the
// rounding the results already carry.  The IEEE square root and division cost
// about ten VALU instructions each, which latency-bound launches pay per wave
// (K-cache norm on the Llama-shaped batch 17.85 -> 16.66 us, 16-head mixed
// MLA batch 11.94 -> 11.62 us, alternating in one process).  Zero, infinite and NaN inputs give the IEEE
// results (1/sqrt(0) = inf, 1/inf = 0, NaN stays NaN).
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- rotation arithmetic --------------------------------------------------------
// A rotated value is x c - y s or y c + x s: a sum of two products.  It is
// evaluated with Kahan's FMA algorithm -- the rounding error of one product is
// recovered exactly and added back -- so the fp32 result is within 2 ulps of
// the exact value even when the two products nearly cancel (a plain fma would
// lose all relative accuracy there).
// a*b + c*d with the rounding error of c*d recovered exactly.  An infinite
// c*d has no rounding error to recover: the error term is then inf - inf =
// NaN, which fminf replaces by the largest finite float, so the sum stays
// +-inf (or NaN when a*b is the opposite infinity), like the exact value;
// a finite error term passes fminf unchanged (one instruction per value).
__device__ __forceinline__ float sum_of_products(float a, float b, float c, float d) {
  const float cd = c * d;
  const float cd_err = fminf(fmaf(c, d, -cd), 3.402823466e38f);  // c*d - cd, exact
  return fmaf(a, b, cd) + cd_err;
}

// ---- memory access helpers ---------------------------------------------------

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte load marked non-temporal (streamed once; keeps it from displacing
// reusable lines in the caches).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// An empty asm that takes a loaded value in place (one 16-byte register
// tuple, so the value stays in the registers the load wrote): code that uses
// the value cannot be moved above it, and the wait for the load lands here.
__device__ __forceinline__ void pin_vgprs(uint4& v) {
  u32x4_t t = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(t));
  v = make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 8-byte non-temporal load.
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// 16-byte non-temporal store.  Every output of the path is written with these:
// a store that allocates in the Infinity Cache leaves dirty lines there whose
// write-back the next kernel pays for.
__device__ __forceinline__ void store16_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// 8-byte non-temporal store (cache rows: written once, never re-read here).
__device__ __forceinline__ void store8_stream(void* p, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}

// ---- wave64 reductions (DPP inside 16-lane rows, readlane across rows) ------

// Lane permutation within 16-lane rows (every lane reads a valid source for
// the patterns used here, so no "old" value is needed).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadMirror = 0x1B;   // quad_perm [3,2,1,0]
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside each 16 lanes

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// Lane exchanges across 16-lane rows, inside 32-lane halves: ds_swizzle in
// bitmask mode (source lane = (lane & 0x1F) ^ xor_mask within each half).
constexpr int kSwizzleXor16 = 0x1F | (0x10 << 10);  // lane i <-> i ^ 16
constexpr int kSwizzleMirror32 = 0x1F | (0x1F << 10);  // lane i <-> 31 - i

template <int PATTERN>
__device__ __forceinline__ uint32_t swizzle_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, PATTERN);
}

template <int PATTERN>
__device__ __forceinline__ float swizzle(float v) {
  return __uint_as_float(swizzle_u32<PATTERN>(__float_as_uint(v)));
}

// Lane l receives lane (l ^ 32)'s value; low_half = (l < 32).
// v_permlane32_swap exchanges the upper 32 lanes of one register with the
// lower 32 of another; given the value twice, one result holds the lower
// half in both halves and the other the upper half, and each lane takes the
// one that is not its own: two VALU instructions, no LDS round trip.
__device__ __forceinline__ uint32_t swap_halves_u32(uint32_t x, bool low_half) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return low_half ? r[1] : r[0];
}

// Lane k of an aligned group of N lanes (N = 4, 8, 16 or 32) receives lane
// (N-1-k)'s 32-bit value.
template <int N>
__device__ __forceinline__ uint32_t mirror_u32(uint32_t x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "mirror over 4, 8, 16 or 32 lanes");
  if constexpr (N == 4) return dpp_u32<kDppQuadMirror>(x);
  else if constexpr (N == 8) return dpp_u32<kDppHalfMirror>(x);
  else if constexpr (N == 16) return dpp_u32<kDppMirror>(x);
  else return swizzle_u32<kSwizzleMirror32>(x);
}

// Exchange a 16-byte chunk with the mirrored lane of its group of N lanes.
template <int N>
__device__ __forceinline__ uint4 mirror16(const uint4& v) {
  return make_uint4(mirror_u32<N>(v.x), mirror_u32<N>(v.y), mirror_u32<N>(v.z),
                    mirror_u32<N>(v.w));
}

// Sum over aligned groups of N lanes (N in 1, 2, 4, 8, 16, 32); every lane of
// a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += swizzle<kSwizzleXor16>(v);
  return v;
}

// Max of |v| over aligned groups of N lanes, a NaN counting as 0 (as fmaxf
// drops it).  Non-negative floats order like their bit patterns, so each
// step is one integer max with the DPP operand folded in; a float max would
// first canonicalise the DPP result (three instructions per step).
template <int N>
__device__ __forceinline__ float group_max_abs(float v) {
  uint32_t u = __float_as_uint(fmaxf(fabsf(v), 0.0f));
  if constexpr (N >= 2) u = max(u, dpp_u32<kDppXor1>(u));
  if constexpr (N >= 4) u = max(u, dpp_u32<kDppXor2>(u));
  if constexpr (N >= 8) u = max(u, dpp_u32<kDppHalfMirror>(u));
  if constexpr (N >= 16) u = max(u, dpp_u32<kDppMirror>(u));
  if constexpr (N >= 32) u = max(u, swizzle_u32<kSwizzleXor16>(u));
  return __uint_as_float(u);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-uniform sum / max of one value per lane (all 64 lanes active).
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Wave-uniform max of |v| (a NaN counting as 0), the last step on the
// scalar unit.
__device__ __forceinline__ float wave_max_abs(float v) {
  const uint32_t u = __float_as_uint(group_max_abs<16>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)u, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)u, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)u, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)u, 48);
  return __uint_as_float(max(max(a, b), max(c, d)));
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// n / d for wave-uniform n and d: a shift when d is a power of two (scalar
// instructions only: the usual case for page sizes and head-chunk counts),
// else the general division, whose reciprocal estimate runs on the vector
// unit.
__device__ __forceinline__ uint32_t udiv_uniform(uint32_t n, uint32_t d) {
  if ((d & (d - 1)) == 0) return n >> __builtin_ctz(d);
  return n / d;
}

// ---- ragged batch and page table -------------------------------------------

// Request owning token t: the number of offsets[1..B] that are <= t (offsets
// non-decreasing).  All 64 lanes load in parallel; the result is wave-uniform.
// Returns B when t lies past offsets[B].
__device__ __forceinline__ uint32_t find_request(const uint32_t* __restrict__ offsets,
                                                 uint32_t B, uint32_t t, int lane) {
  uint32_t count = 0;
  for (uint32_t base = 0; base < B; base += kWave) {
    const uint32_t i = base + (uint32_t)lane + 1;
    const uint32_t v = (i <= B) ? offsets[i] : 0xffffffffu;
    count += (uint32_t)__popcll(__ballot(v <= t));
  }
  return uniform(count);
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, uint32_t lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)lane);
}

// First step of the address chain: the request owning token t and the
// token's cache slot (prior length + index within the request).  For batches
// of up to 256 requests every lane loads entries i, i+64, ... of the offsets
// and the prior lengths in one step; the request is the number of offsets
// <= t (ballot), and its start and prior length are read from the owning lane.
struct TokenSlot {
  uint32_t request;
  uint32_t slot;
  bool ok;           // request < B
};

// The loads of the first step, for batches of up to kSlotChunks * 64
// requests (each lane: entries lane, lane + 64, ... of the offsets and the
// prior lengths).  Issued on their own (slot_issue) they can be put in front
// of other loads, and then waited for alone: the load counter is in order.
constexpr int kSlotChunks = 4;
struct SlotLoads {
  uint32_t nxt[kSlotChunks], beg[kSlotChunks], len[kSlotChunks];
};

__device__ __forceinline__ void slot_issue(const uint32_t* __restrict__ offsets, uint32_t B,
                                           const uint32_t* __restrict__ cache_lengths, int lane,
                                           SlotLoads& s) {
  if (B <= kSlotChunks * kWave) {
    // offsets + 1 through an opaque copy of its address (kept a global
    // pointer): the compiler would otherwise join each lane's two offsets into
    // one 8-byte load, which measured slower on a 68-request batch (16-head
    // MLA 10.9 -> 11.4 us)
    uint64_t next_addr = reinterpret_cast<uint64_t>(offsets + 1);
    asm("" : "+s"(next_addr));
    const __attribute__((address_space(1))) uint32_t* next =
        reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(next_addr);
#pragma unroll
    for (int k = 0; k < kSlotChunks; ++k) {
      const uint32_t i = k * kWave + (uint32_t)lane;
      const bool in = i < B;
      s.nxt[k] = in ? next[i] : 0xffffffffu;
      s.beg[k] = in ? offsets[i] : 0u;
      s.len[k] = in ? cache_lengths[i] : 0u;
    }
  }
}

__device__ __forceinline__ TokenSlot slot_resolve(const SlotLoads& s,
                                                  const uint32_t* __restrict__ offsets, uint32_t B,
                                                  const uint32_t* __restrict__ cache_lengths,
                                                  uint32_t t, int lane) {
  TokenSlot r{};
  if (B <= kSlotChunks * kWave) {
    uint32_t count = 0;
#pragma unroll
    for (int k = 0; k < kSlotChunks; ++k) count += (uint32_t)__popcll(__ballot(s.nxt[k] <= t));
    r.request = uniform(count);
    r.ok = r.request < B;
    if (!r.ok) return r;
    const uint32_t kb = r.request / kWave, lb = r.request % kWave;
    uint32_t start = 0, prior = 0;
#pragma unroll
    for (int k = 0; k < kSlotChunks; ++k) {
      if (kb == (uint32_t)k) {
        start = lane_u32(s.beg[k], lb);
        prior = lane_u32(s.len[k], lb);
      }
    }
    r.slot = prior + (t - start);
  } else {
    r.request = find_request(offsets, B, t, lane);
    r.ok = r.request < B;
    if (!r.ok) return r;
    r.slot = uniform(cache_lengths[r.request] + (t - offsets[r.request]));
  }
  return r;
}

__device__ __forceinline__ TokenSlot find_slot(const uint32_t* __restrict__ offsets, uint32_t B,
                                               const uint32_t* __restrict__ cache_lengths,
                                               uint32_t t, int lane) {
  SlotLoads s;
  slot_issue(offsets, B, cache_lengths, lane, s);
  return slot_resolve(s, offsets, B, cache_lengths, t, lane);
}

// Second step: physical page and offset of a slot.  Returns false when the
// slot lies past the request's page-table row or the page id past the pool.
struct PageSlot {
  uint32_t page;
  uint32_t offset;
};

__device__ __forceinline__ uint32_t page_column(uint32_t slot, uint32_t page_size) {
  return udiv_uniform(slot, page_size);
}

__device__ __forceinline__ bool page_of(const uint32_t* __restrict__ page_table,
                                        uint32_t pt_stride, uint32_t num_pages,
                                        uint32_t page_size, const TokenSlot& ts, PageSlot* ps) {
  const uint32_t col = page_column(ts.slot, page_size);
  if (col >= pt_stride) return false;
  ps->page = uniform(page_table[(uint64_t)ts.request * pt_stride + col]);
  ps->offset = ts.slot - col * page_size;
  return ps->page < num_pages;
}

__device__ __forceinline__ void count_skip(uint32_t* error_count, int lane) {
  if (error_count != nullptr && lane == 0) atomicAdd(error_count, 1u);
}

}  // namespace pkv
