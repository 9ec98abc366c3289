// stream_copy.hip -- the plain streaming copy behind pkv_stream_copy
// (include/pkv_bench.h): a measurement reference, not part of the method.
// Each thread moves 16-byte pieces with non-temporal loads and stores,
// grid-stride, so every wave instruction reads and writes 1 KiB contiguous.
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
