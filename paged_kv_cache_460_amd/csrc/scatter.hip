// Cache write ("reshape_and_cache") as its own launch: one workgroup of 256 threads per
// (group of 16 consecutive tokens, kv head), with the slots read from the slot mapping.
// The layout and the store rules are stated in cache_write.h.
#include "cache_write.h"

namespace pa {

template <int kElemBytes>
__global__ __launch_bounds__(256) void scatter_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int64_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim) {
  const int h = (int)(blockIdx.x % num_kv_heads);
  const int64_t t0 = (int64_t)(blockIdx.x / num_kv_heads) * kWriteGroup;
  write_unit<kElemBytes>(k, v, k_cache, v_cache, t0, h, num_tokens, num_kv_heads, head_dim, threadIdx.x,
                         blockDim.x, [&](int j) { return slots[t0 + j]; });
}

hipError_t launch_scatter(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slots, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t grid = (num_tokens + kWriteGroup - 1) / kWriteGroup * num_kv_heads;
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(scatter_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  } else {
    hipLaunchKernelGGL(scatter_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  }
  return hipGetLastError();
}

}  // namespace pa
