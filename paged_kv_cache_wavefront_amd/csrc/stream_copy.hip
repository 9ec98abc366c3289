// stream_copy.hip -- the plain streaming kernels behind pkv_stream_copy and
// pkv_stream_mix (include/pkv_bench.h): measurement references, not part of
// the method.  Each thread moves 16-byte pieces with non-temporal loads and
// stores, grid-stride, so every wave instruction reads and writes 1 KiB
// contiguous.
#include <hip/hip_runtime.h>

#include "../../include/pkv.h"
#include "../../include/pkv_bench.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst,
                                                          uint64_t pieces) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// R pieces read and W pieces written, interleaved evenly over the launch.
// The longer stream sets the N = max(R, W) iterations; iteration i moves
// piece i of the longer stream and, when the shorter stream's index
// m(i) = (i * ratio) >> 32 moves on (ratio = ceil(shorter * 2^32 / longer),
// set by the host: no division in the loop), piece m(i) of the shorter one --
// a write after the reads that led to it, a read at the first iteration of
// its group.  A written piece is the XOR of the pieces its thread read since
// its previous write, XOR `key` (0 at run time, unknown to the compiler: no
// load or store can be dropped), so at 1:1 the kernel copies, and in place
// (src == dst) it rewrites every piece with its own value.  Work is dealt
// out in chunks of 256 pieces per wave: lane l takes pieces 64k + l of the
// chunk (k = 0..3), so each wave instruction covers 1 KiB contiguous and a
// lane has its four loads in flight before its stores.  With W = 0 the loads
// feed a store that only a value no thread can produce would trigger.
constexpr int kMixUnroll = 4;

__global__ __launch_bounds__(256) void stream_mix_kernel(const u32x4* src, u32x4* dst,
                                                         uint64_t R, uint64_t W, uint64_t ratio,
                                                         uint32_t key) {
  const int lane = threadIdx.x & 63;
  const uint64_t waves = (uint64_t)gridDim.x * (blockDim.x / 64);
  const uint64_t N = R > W ? R : W;
  const uint64_t chunks = (N + 64 * kMixUnroll - 1) / (64 * kMixUnroll);
  const u32x4 zero = {key, key, key, key};
  u32x4 acc = zero;
  for (uint64_t c = (uint64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; c < chunks;
       c += waves) {
    u32x4 v[kMixUnroll];
#pragma unroll
    for (int k = 0; k < kMixUnroll; ++k) {
      const uint64_t i = c * 64 * kMixUnroll + 64 * k + lane;
      v[k] = zero ^ zero;
      if (R >= W) {
        if (i < R) v[k] = __builtin_nontemporal_load(src + i);
      } else if (i < W && R != 0) {
        const uint64_t m = (i * ratio) >> 32;
        if ((i == 0 || ((i - 1) * ratio) >> 32 != m) && m < R)
          v[k] = __builtin_nontemporal_load(src + m);
      }
    }
#pragma unroll
    for (int k = 0; k < kMixUnroll; ++k) {
      const uint64_t i = c * 64 * kMixUnroll + 64 * k + lane;
      acc ^= v[k];
      if (R >= W) {
        const uint64_t m = (i * ratio) >> 32;
        if (i < R && ((i + 1) * ratio) >> 32 != m && m < W) {
          __builtin_nontemporal_store(acc, dst + m);
          acc = zero;
        }
      } else if (i < W) {
        __builtin_nontemporal_store(acc, dst + i);
        acc = zero;
      }
    }
  }
  if (W == 0 && acc.x == 0x9e3779b9u && acc.y == ~key && acc.z == 0x7f4a7c15u && acc.w == key + 1)
    dst[0] = acc;
}

}  // namespace

extern "C" int pkv_stream_copy(const void* src, void* dst, uint64_t bytes, uint32_t blocks,
                               void* stream) {
  if (src == nullptr || dst == nullptr) return PKV_ERR_NULL;
  if (blocks == 0) return PKV_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | bytes) & 15u)
    return PKV_ERR_ALIGN;
  if (bytes == 0) return PKV_OK;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

extern "C" int pkv_stream_mix(const void* src, uint64_t read_bytes, void* dst,
                              uint64_t write_bytes, uint32_t blocks, void* stream) {
  if (src == nullptr || dst == nullptr) return PKV_ERR_NULL;
  if (blocks == 0) return PKV_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | read_bytes |
       write_bytes) & 15u)
    return PKV_ERR_ALIGN;
  // piece indices are multiplied together: keep each count below 2^31
  if (read_bytes >= (16ull << 31) || write_bytes >= (16ull << 31)) return PKV_ERR_RANGE;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s == d) {
    if (read_bytes != write_bytes) return PKV_ERR_SHAPE;  // in place: every piece both ways
  } else if (s < d + write_bytes && d < s + read_bytes) {
    return PKV_ERR_RANGE;                                   // partial overlap
  }
  if (read_bytes == 0 && write_bytes == 0) return PKV_OK;
  const uint64_t R = read_bytes / 16, W = write_bytes / 16;
  const uint64_t lo = R < W ? R : W, hi = R < W ? W : R;
  const uint64_t ratio = ((lo << 32) + hi - 1) / hi;  // ceil(lo * 2^32 / hi) <= 2^32
  hipLaunchKernelGGL(stream_mix_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), R, W, ratio, 0u);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
