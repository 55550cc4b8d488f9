// Cache write ("reshape_and_cache"): each new token's K/V rows go to the slot the slot
// mapping names (restatement section 一: the KV tensors are bound at init and the
// slot mapping is built each step).
//
// One thread moves 16 bytes of one (token, kv head) row. Keys keep their row layout in
// the block ([block][head][offset][d]), so a key row is one contiguous run and the
// 16-byte pieces of one row are written by neighbouring lanes. Values are stored
// dim-major inside a block ([block][head][d][offset]) so that the attention kernels can
// feed 8 consecutive tokens of one dimension straight into an MFMA operand; a value row
// therefore lands as D scattered elements, 32 (bf16) or 64 (fp32) bytes apart.
// A pure bit copy: nothing is converted or rounded.
#include "pa_internal.h"

namespace pa {

template <int kElemBytes>
__global__ __launch_bounds__(256) void scatter_kernel(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slots, int64_t num_tokens,
    int32_t num_kv_heads, int32_t head_dim) {
  const int vec_per_row = head_dim * kElemBytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = num_tokens * num_kv_heads * vec_per_row;
  if (idx >= total) return;
  const int vec = (int)(idx % vec_per_row);
  const int64_t rest = idx / vec_per_row;
  const int h = (int)(rest % num_kv_heads);
  const int64_t t = rest / num_kv_heads;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t block = slot / kBlock;
  const int off = (int)(slot % kBlock);
  const int64_t row_bytes = (int64_t)head_dim * kElemBytes;
  const int64_t src = (t * num_kv_heads + h) * row_bytes + vec * 16;

  const u32x4 kv = *reinterpret_cast<const u32x4*>(k + src);
  *reinterpret_cast<u32x4*>(k_cache + ((block * num_kv_heads + h) * kBlock + off) * row_bytes + vec * 16) = kv;

  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
  constexpr int kPerVec = 16 / kElemBytes;
  const int d0 = vec * kPerVec;
  // element (block, h, d, off) of the dim-major value block
  const int64_t base = ((block * num_kv_heads + h) * head_dim + d0) * kBlock + off;
  if constexpr (kElemBytes == 2) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(v_cache) + base;
#pragma unroll
    for (int e = 0; e < kPerVec; ++e) {
      const uint32_t w = vv[e >> 1];
      dst[(int64_t)e * kBlock] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(v_cache) + base;
#pragma unroll
    for (int e = 0; e < kPerVec; ++e) dst[(int64_t)e * kBlock] = vv[e];
  }
}

hipError_t launch_scatter(const void* k, const void* v, void* k_cache, void* v_cache,
                          const int64_t* slots, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t elem_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int64_t total = num_tokens * num_kv_heads * (int64_t)(head_dim * elem_bytes / 16);
  const int64_t blocks = (total + threads - 1) / threads;
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(scatter_kernel<2>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  } else {
    hipLaunchKernelGGL(scatter_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)k_cache, (uint8_t*)v_cache,
                       slots, num_tokens, num_kv_heads, head_dim);
  }
  return hipGetLastError();
}

}  // namespace pa
