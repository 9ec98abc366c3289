// mla_gather_latent_paged.hip -- paged latent cache -> dense buffer, gfx950.
//
// What it computes ("mla_graph" module page, mla_prefill_branch_fp8: the
// latent values are copied from the paged cache into a contiguous buffer and
// quantised to fp8): row kv_row_offsets[b] + j of the output is cache slot j
// of request b, copied, dequantised (fp8 code x scale -> bf16) or quantised
// (bf16 / scale -> fp8, saturating round-to-nearest-even).
//
// One wave per group of rows: 6 rows (3 for bf16 -> bf16).  Lanes
// 0..rows-1 each resolve one row (request by ballot over the offsets -- once
// for the whole group when it lies in one request --, slot, page-table entry,
// per-token scale); a piece lane fetches its row's source address from the
// row lane with ds_bpermute.  Loads are non-temporal (each cache byte is read
// once) and so are the stores (the dense output is written once); every wave
// instruction reads and writes contiguous runs (fp8 -> bf16 reads 8-byte
// pieces so that each lane writes 16 contiguous bytes; writing 32 bytes per
// lane as two 16-byte stores at a 32-byte lane stride measured 1.8x slower).
//
// Rows per wave, measured on MI355X with rotating outputs over 1 022 807
// rows of 576 elements (microseconds, 16 / 8 / 6 / 4 / 3 rows per wave):
// fp8 -> bf16 326 / 320 / 316 / 317 / 327, fp8 -> fp8 217 / - / 202 / 206 /
// 217; bf16 -> bf16 (8 / 6 / 4 / 3 / 2 rows) 435 / 430 / 414 / 400 / 411,
// bf16 -> fp8 292 / 288 / 291 / 311 / 352.  Two rows or one per wave leave
// lanes idle and cost far more (fp8 -> bf16 383 and 548).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr uint32_t kMaxElems = 1024;  // widest row supported
constexpr uint32_t kMlaElems = 576;   // the MLA latent row

// Launch geometry of one conversion: rows per wave, input bytes per piece
// (one lane's share of one wave instruction) and the wave instructions that
// cover the rows of a given width.
template <bool IN_FP8, bool OUT_FP8>
struct Shape {
  static constexpr uint32_t kRows = (!IN_FP8 && !OUT_FP8) ? 3 : 6;
  static constexpr uint32_t kPiece = (IN_FP8 && !OUT_FP8) ? 8 : 16;
  static constexpr uint32_t kInBytes = IN_FP8 ? 1 : 2;
  static constexpr int instr(uint32_t elems) {
    return (int)((kRows * (elems * kInBytes / kPiece) + kWave - 1) / kWave);
  }
};

__device__ __forceinline__ uint32_t shfl_u32(uint32_t v, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

template <bool IN_FP8, bool OUT_FP8, bool PER_TOKEN, int NI>
__global__ __launch_bounds__(256) void gather_kernel(const GatherArgs a) {
  using G = Shape<IN_FP8, OUT_FP8>;
  constexpr uint32_t RPW = G::kRows;
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t wave =
      blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave);
  const uint32_t r0 = uniform(wave * RPW);
  if (r0 >= a.total_rows) return;
  const uint32_t nrows = min(RPW, a.total_rows - r0);
  const CacheView& cv = a.cache;
  const uint32_t B = a.batch;

  // ---- stage 1: request and slot of each row (lane j <- row r0 + j) ----------
  uint32_t my_req = 0xffffffffu, my_slot = 0;
  if (B <= 4 * kWave) {
    uint32_t nxt[4], beg[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = k * kWave + (uint32_t)lane;
      nxt[k] = i < B ? a.kv_row_offsets[i + 1] : 0xffffffffu;
      beg[k] = i < B ? a.kv_row_offsets[i] : 0u;
    }
    auto request_of = [&](uint32_t r) {
      uint32_t b = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) b += (uint32_t)__popcll(__ballot(nxt[k] <= r));
      return uniform(b);
    };
    auto start_of = [&](uint32_t b) {
      uint32_t start = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (b / kWave == (uint32_t)k) start = lane_u32(beg[k], b % kWave);
      return start;
    };
    const uint32_t b_first = request_of(r0), b_last = request_of(r0 + nrows - 1);
    if (b_first == b_last) {
      // the usual case: every row of the group belongs to one request
      if (b_first < B) {
        my_req = b_first;
        my_slot = r0 + (uint32_t)lane - start_of(b_first);
      }
    } else {
      for (uint32_t j = 0; j < nrows; ++j) {
        const uint32_t b = request_of(r0 + j);
        const uint32_t start = b < B ? start_of(b) : 0;
        if ((uint32_t)lane == j) {
          my_req = b < B ? b : 0xffffffffu;
          my_slot = r0 + j - start;
        }
      }
    }
  } else {
    for (uint32_t j = 0; j < nrows; ++j) {
      const uint32_t r = r0 + j;
      const uint32_t b = find_request(a.kv_row_offsets, B, r, lane);
      uint32_t start = 0;
      if (b < B) start = uniform(a.kv_row_offsets[b]);
      if ((uint32_t)lane == j) {
        my_req = b < B ? b : 0xffffffffu;
        my_slot = r - start;
      }
    }
  }

  // ---- stage 2: page of each row, its source offset and scale ----------------
  bool row_ok = false;
  uint64_t row_src = 0;  // byte offset of the row inside this layer's pool
  float row_scale = 1.0f;
  if ((uint32_t)lane < nrows && my_req != 0xffffffffu) {
    const uint32_t col = my_slot / cv.page_size;
    if (col < cv.pt_stride) {
      const uint32_t page = cv.page_table[(uint64_t)my_req * cv.pt_stride + col];
      if (page < cv.num_pages) {
        const uint32_t off = my_slot - col * cv.page_size;
        const int64_t elem = IN_FP8 ? 1 : 2;
        row_ok = true;
        row_src = (uint64_t)((int64_t)page * cv.page_stride + (int64_t)off * cv.slot_stride) * elem;
        if constexpr (IN_FP8 && PER_TOKEN)
          row_scale = a.cache_scale[((int64_t)page * cv.page_size + off) * cv.num_heads];
      }
    }
  }
  if constexpr (IN_FP8 && !PER_TOKEN) row_scale = *a.cache_scale;
  {
    const uint64_t bad = __ballot((uint32_t)lane < nrows && !row_ok);
    if (bad && cv.error_count != nullptr && lane == 0)
      atomicAdd(cv.error_count, (uint32_t)__popcll(bad));
  }
  float inv_out = 1.0f;
  if constexpr (!IN_FP8 && OUT_FP8) inv_out = 1.0f / *a.out_scale;
  if constexpr (IN_FP8 && OUT_FP8 && PER_TOKEN) {
    if (row_ok && a.out_scales != nullptr) a.out_scales[r0 + lane] = row_scale;
  }

  // ---- stage 3: copies -------------------------------------------------------------
  // piece g = i * 64 + lane of the wave's rows: row g / ppr, piece g % ppr.  A
  // piece is 16 input bytes, except for fp8 -> bf16 where it is 8 input bytes
  // so that every lane stores 16 contiguous output bytes.
  constexpr uint32_t PIECE = G::kPiece;
  constexpr uint32_t OUT_PIECE = IN_FP8 == OUT_FP8 ? PIECE : (IN_FP8 ? 2 * PIECE : PIECE / 2);
  const uint32_t ppr = a.row_bytes / PIECE;  // pieces per row
  const uint32_t pieces = nrows * ppr;
  const char* src_base = static_cast<const char*>(cv.layer_base);
  char* out_base = static_cast<char*>(a.out) + (int64_t)r0 * a.out_row_bytes;
  const uint64_t ok_rows = __ballot(row_ok);  // bit j: row j has a page
  uint4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t g = (uint32_t)i * kWave + (uint32_t)lane;
    const uint32_t j = g < pieces ? g / ppr : 0;
    const uint32_t lo = shfl_u32((uint32_t)row_src, (int)j);
    const uint32_t hi = shfl_u32((uint32_t)(row_src >> 32), (int)j);
    v[i] = make_uint4(0, 0, 0, 0);
    if (g < pieces && ((ok_rows >> j) & 1u)) {
      const char* p = src_base + ((uint64_t)hi << 32 | lo) + PIECE * (g - j * ppr);
      if constexpr (PIECE == 16) {
        v[i] = load16_stream(p);
      } else {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        v[i].x = w.x;
        v[i].y = w.y;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t g = (uint32_t)i * kWave + (uint32_t)lane;
    const uint32_t j = g < pieces ? g / ppr : 0;
    const uint32_t c = g - j * ppr;
    float scl = 1.0f;
    if constexpr (IN_FP8 && !OUT_FP8) scl = __uint_as_float(shfl_u32(__float_as_uint(row_scale), (int)j));
    if (!(g < pieces && ((ok_rows >> j) & 1u))) continue;
    char* dst = out_base + (int64_t)j * a.out_row_bytes + OUT_PIECE * c;
    if constexpr (IN_FP8 == OUT_FP8) {
      store16_stream(dst, v[i]);
    } else if constexpr (IN_FP8) {
      // 8 fp8 codes -> 8 bf16 (one 16-byte store)
      float f[8];
      const uint32_t w[2] = {v[i].x, v[i].y};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x2_t lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
        const f32x2_t hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
        f[4 * q] = lo2[0] * scl;
        f[4 * q + 1] = lo2[1] * scl;
        f[4 * q + 2] = hi2[0] * scl;
        f[4 * q + 3] = hi2[1] * scl;
      }
      store16_stream(dst, pack8_bf16(f));
    } else {
      // 8 bf16 -> 8 fp8 codes (one 8-byte store)
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] *= inv_out;
      store8_stream(dst, pack8_fp8(f));
    }
  }
}

template <bool IN_FP8, bool OUT_FP8, int NI>
hipError_t launch_ni(const GatherArgs& a, bool per_token, uint32_t blocks, hipStream_t stream) {
  if (per_token)
    hipLaunchKernelGGL((gather_kernel<IN_FP8, OUT_FP8, true, NI>), dim3(blocks), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((gather_kernel<IN_FP8, OUT_FP8, false, NI>), dim3(blocks), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

// Wave instructions per row group: enough for rows of the MLA latent width,
// or for the widest rows supported.
template <bool IN_FP8, bool OUT_FP8>
hipError_t launch_kind(const GatherArgs& a, bool per_token, uint32_t blocks, hipStream_t stream) {
  using G = Shape<IN_FP8, OUT_FP8>;
  const uint32_t elems = a.row_bytes / G::kInBytes;
  if (elems <= kMlaElems)
    return launch_ni<IN_FP8, OUT_FP8, G::instr(kMlaElems)>(a, per_token, blocks, stream);
  return launch_ni<IN_FP8, OUT_FP8, G::instr(kMaxElems)>(a, per_token, blocks, stream);
}

template <bool IN_FP8, bool OUT_FP8>
hipError_t launch_checked(const GatherArgs& a, bool per_token, hipStream_t stream) {
  using G = Shape<IN_FP8, OUT_FP8>;
  if (a.row_bytes % G::kPiece != 0 || a.row_bytes / G::kInBytes > kMaxElems)
    return hipErrorInvalidValue;
  const uint64_t waves = ((uint64_t)a.total_rows + G::kRows - 1) / G::kRows;
  const uint64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  return launch_kind<IN_FP8, OUT_FP8>(a, per_token, (uint32_t)blocks, stream);
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, GatherKind kind, bool per_token, hipStream_t stream) {
  switch (kind) {
    case GatherKind::Fp8ToFp8: return launch_checked<true, true>(a, per_token, stream);
    case GatherKind::Fp8ToBf16: return launch_checked<true, false>(a, per_token, stream);
    case GatherKind::Bf16ToBf16: return launch_checked<false, false>(a, false, stream);
    case GatherKind::Bf16ToFp8: return launch_checked<false, true>(a, false, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
