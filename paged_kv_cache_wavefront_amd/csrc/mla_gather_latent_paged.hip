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
// row lane with ds_bpermute.  Every lane loads 16-byte pieces; loads are
// non-temporal (each cache byte is read once) and so are the stores (the
// dense output is written once).  Each wave store instruction must cover a
// contiguous run: fp8 -> bf16 turns a lane's 16 codes into 32 output bytes,
// so the converted rows are staged in LDS (a wave-private region, no block
// barrier) and read back as 16-byte chunks in output order.  (Writing the 32
// bytes as two 16-byte stores at a 32-byte lane stride measured 1.8x slower;
// 8-byte loads so that each lane stores 16 contiguous bytes, 3.5 % slower
// than the LDS staging.)
//
// Rows per wave, measured on MI355X with rotating outputs over 1 022 807
// rows of 576 elements (microseconds, 16 / 8 / 6 / 4 / 3 rows per wave):
// fp8 -> fp8 217 / - / 202 / 206 / 217; bf16 -> bf16 (8 / 6 / 4 / 3 / 2
// rows) 435 / 430 / 414 / 400 / 411, bf16 -> fp8 292 / 288 / 291 / 311 / 352;
// fp8 -> bf16 staged through LDS 310 (4 rows), 305 (6), 307 (8), 313 (10),
// against 316 for 6 rows with 8-byte loads.  Two rows or one per wave leave
// lanes idle and cost far more.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr uint32_t kMaxElems = 1024;  // widest row supported
constexpr uint32_t kMlaElems = 576;   // the MLA latent row

// Launch geometry of one conversion: rows per wave, input bytes per piece
// (one lane's share of one load instruction), the load instructions that
// cover the rows of a given width, and the LDS staging area of a block.
template <bool IN_FP8, bool OUT_FP8>
struct Shape {
  static constexpr uint32_t kRows = (!IN_FP8 && !OUT_FP8) ? 3 : 6;
  static constexpr uint32_t kPiece = 16;
  static constexpr uint32_t kInBytes = IN_FP8 ? 1 : 2;
  static constexpr bool kStaged = IN_FP8 && !OUT_FP8;  // output twice the input
  static constexpr int instr(uint32_t elems) {
    return (int)((kRows * (elems * kInBytes / kPiece) + kWave - 1) / kWave);
  }
  static uint32_t stage_bytes(uint32_t row_bytes) {
    return kStaged ? (uint32_t)kWavesPerBlock * kRows * 2 * row_bytes : 0u;
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
  // piece g = i * 64 + lane of the wave's rows: row g / ppr, piece g % ppr
  // (16 input bytes).
  constexpr uint32_t PIECE = G::kPiece;
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
    if (g < pieces && ((ok_rows >> j) & 1u))
      v[i] = load16_stream(src_base + ((uint64_t)hi << 32 | lo) + PIECE * (g - j * ppr));
  }
  if constexpr (G::kStaged) {
    // 16 codes -> 32 bytes of bf16 per piece, staged densely (row j at
    // j * 2 * row_bytes) in this wave's LDS region, then read back and
    // stored as 16-byte chunks in output order.
    extern __shared__ uint4 stage[];
    const uint32_t opr = 2 * ppr;  // 16-byte output chunks per row
    uint4* st = stage + (threadIdx.x / kWave) * (RPW * opr);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t g = (uint32_t)i * kWave + (uint32_t)lane;
      const uint32_t j = g < pieces ? g / ppr : 0;
      const uint32_t c = g - j * ppr;
      const float scl = __uint_as_float(shfl_u32(__float_as_uint(row_scale), (int)j));
      if (!(g < pieces && ((ok_rows >> j) & 1u))) continue;
      float f[2][8];
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x2_t lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
        const f32x2_t hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
        f[q / 2][4 * (q & 1)] = lo2[0] * scl;
        f[q / 2][4 * (q & 1) + 1] = lo2[1] * scl;
        f[q / 2][4 * (q & 1) + 2] = hi2[0] * scl;
        f[q / 2][4 * (q & 1) + 3] = hi2[1] * scl;
      }
      st[j * opr + 2 * c] = pack8_bf16(f[0]);
      st[j * opr + 2 * c + 1] = pack8_bf16(f[1]);
    }
    // a wave's LDS accesses complete in issue order: only the compiler must
    // not move the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t chunks = nrows * opr;
#pragma unroll
    for (int i = 0; i < 2 * NI; ++i) {
      const uint32_t q = (uint32_t)i * kWave + (uint32_t)lane;
      if (q >= chunks) continue;
      const uint32_t j = q / opr;
      if (!((ok_rows >> j) & 1u)) continue;
      store16_stream(out_base + (int64_t)j * a.out_row_bytes + 16 * (q - j * opr), st[q]);
    }
    return;
  }
  constexpr uint32_t OUT_PIECE = IN_FP8 == OUT_FP8 ? PIECE : PIECE / 2;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t g = (uint32_t)i * kWave + (uint32_t)lane;
    const uint32_t j = g < pieces ? g / ppr : 0;
    const uint32_t c = g - j * ppr;
    if (!(g < pieces && ((ok_rows >> j) & 1u))) continue;
    char* dst = out_base + (int64_t)j * a.out_row_bytes + OUT_PIECE * c;
    if constexpr (IN_FP8 == OUT_FP8) {
      store16_stream(dst, v[i]);
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
  const uint32_t lds = Shape<IN_FP8, OUT_FP8>::stage_bytes(a.row_bytes);
  if (per_token)
    hipLaunchKernelGGL((gather_kernel<IN_FP8, OUT_FP8, true, NI>), dim3(blocks), dim3(256), lds,
                       stream, a);
  else
    hipLaunchKernelGGL((gather_kernel<IN_FP8, OUT_FP8, false, NI>), dim3(blocks), dim3(256), lds,
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
